// kda_sched.hip -- varlen work scheduler of the chunked KDA forward (gfx950).
//
// From the packed cu_seqlens (int64 [N+1], B = 1, T = total length; "Kernel
// API" table of the FlashKDA README digest) build, on the device and without
// a host round trip:
//   seq_tab[n]   = {first chunk index, number of 64-token chunks} of sequence n
//   seq_span[n]  = {first token, length} of sequence n (after clamping)
//   chunk_tab[i] = {first token, length <= 64} of chunk i (length 0: unused)
//   seq_order[k] = the sequence with the k-th most chunks (ties: lower index
//                  first), so the sequential state chains start longest first;
//                  input order when N > SORT_MAX
// and, for a call run in windows of win_chunks chunk slots (win_chunks > 0):
//   nz_seq[k]    = the k-th sequence with at least one chunk, in index (and so in
//                  chunk) order
//   win_first[w] = the first k whose sequence ends after chunk slot w * win_chunks,
//                  for w = 0 .. n_win (win_first[n_win] = the number of such sequences):
//                  window w's sequences are nz_seq[win_first[w]] onwards, up to the
//                  first that starts at or after its end
// Chunks never straddle sequences; a sequence's last chunk may be partial.
// Every sequence is clamped into [0, T] and the chunk count into the slot
// budget floor(T/64) + N, so malformed contents cannot drive the other kernels
// out of bounds (results are then unspecified, never a fault).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int SCHED_THREADS = 1024;
constexpr int SORT_MAX = 4096;   // sequences sorted in LDS (bitonic); beyond: input order

__global__ __launch_bounds__(SCHED_THREADS) void kda_sched_kernel(const int64_t* cu, int32_t N, int32_t T,
                                                                  int32_t max_chunks, int2* seq_tab,
                                                                  int2* chunk_tab, int2* seq_span,
                                                                  int32_t* seq_order, int32_t win_chunks,
                                                                  int32_t n_win, int32_t* nz_seq,
                                                                  int32_t* win_first) {
  __shared__ int32_t warp_sums[SCHED_THREADS / 64];
  __shared__ uint64_t keys[SORT_MAX];
  __shared__ int2 s_tab[SORT_MAX], s_span[SORT_MAX];   // LDS copies of the tables (N <= SORT_MAX)
  __shared__ int32_t carry_s;
  const bool in_lds = N <= SORT_MAX;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();

  // pass 1: clamped lengths, chunk counts, exclusive scan of the counts
  for (int base = 0; base < N; base += SCHED_THREADS) {
    const int n = base + tid;
    int32_t s = 0, len = 0, nc = 0;
    if (n < N) {
      int64_t a = cu[n], b = cu[n + 1];
      a = a < 0 ? 0 : (a > T ? T : a);
      b = b < a ? a : (b > T ? T : b);
      s = (int32_t)a;
      len = (int32_t)(b - a);
      nc = (len + CH - 1) / CH;
    }
    // inclusive scan of nc within the wave, then across waves
    int32_t x = nc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) warp_sums[wid] = x;
    __syncthreads();
    int32_t woff = 0;
    for (int k = 0; k < wid; ++k) woff += warp_sums[k];
    const int32_t carry = carry_s;
    const int32_t first = carry + woff + x - nc;
    if (n < N) {
      const int32_t f = first < max_chunks ? first : max_chunks;
      const int32_t cnt = nc < max_chunks - f ? nc : max_chunks - f;
      seq_tab[n] = make_int2(f, cnt);
      seq_span[n] = make_int2(s, len);
      if (in_lds) {
        s_tab[n] = make_int2(f, cnt);
        s_span[n] = make_int2(s, len);
      }
    }
    __syncthreads();
    if (tid == SCHED_THREADS - 1) carry_s = carry + woff + x;
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();

  // pass 2: every chunk slot finds its sequence by binary search over the table
  // (in LDS up to SORT_MAX sequences, else the global copy written above)
  auto tab = [&](int n) { return in_lds ? s_tab[n] : seq_tab[n]; };
  auto span = [&](int n) { return in_lds ? s_span[n] : seq_span[n]; };
  for (int i = tid; i < max_chunks; i += SCHED_THREADS) {
    int lo = 0, hi = N - 1, found = -1;
    while (lo <= hi) {   // last n with tab(n).x <= i
      const int mid = (lo + hi) >> 1;
      if (tab(mid).x <= i) {
        found = mid;
        lo = mid + 1;
      } else {
        hi = mid - 1;
      }
    }
    int2 e = make_int2(0, 0);
    if (found >= 0) {
      const int2 st = tab(found);
      const int jj = i - st.x;
      if (jj < st.y) {
        const int2 sp = span(found);
        const int32_t rem = sp.y - jj * CH;
        e = make_int2(sp.x + jj * CH, rem < CH ? rem : CH);
      }
    }
    chunk_tab[i] = e;
  }

  // windowed calls: the sequences with chunks, compacted in order, and each window's first
  if (win_chunks > 0) {
    if (tid == 0) carry_s = 0;
    __syncthreads();
    for (int base = 0; base < N; base += SCHED_THREADS) {
      const int n = base + tid;
      const int32_t nzf = (n < N && tab(n).y > 0) ? 1 : 0;
      int32_t x = nzf;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) warp_sums[wid] = x;
      __syncthreads();
      int32_t woff = 0;
      for (int k = 0; k < wid; ++k) woff += warp_sums[k];
      const int32_t carry = carry_s;
      if (nzf) nz_seq[carry + woff + x - 1] = n;
      __syncthreads();
      if (tid == SCHED_THREADS - 1) carry_s = carry + woff + x;
      __syncthreads();
    }
    __threadfence_block();
    __syncthreads();
    const int32_t nzc = carry_s;
    for (int w = tid; w <= n_win; w += SCHED_THREADS) {
      const int64_t cb = (int64_t)w * win_chunks;
      int lo = 0, hi = nzc;   // first k with end(k) > cb (ends increase with k)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int2 e = tab(nz_seq[mid]);
        if ((int64_t)e.x + e.y > cb) hi = mid; else lo = mid + 1;
      }
      win_first[w] = w == n_win ? nzc : lo;
    }
  }

  // pass 3: longest-first order of the sequences. Key = (INT32_MAX - chunks) << 32 | n,
  // sorted ascending by a bitonic network over the next power of two >= N.
  if (N > SORT_MAX) {
    for (int n = tid; n < N; n += SCHED_THREADS) seq_order[n] = n;
    return;
  }
  int np = 1;
  while (np < N) np <<= 1;
  for (int i = tid; i < np; i += SCHED_THREADS)
    keys[i] = i < N ? ((uint64_t)(uint32_t)(0x7fffffff - s_tab[i].y) << 32) | (uint32_t)i : ~0ull;
  __syncthreads();
  for (int k = 2; k <= np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np; i += SCHED_THREADS) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = keys[i], b = keys[ixj];
          if ((a > b) == ((i & k) == 0)) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int n = tid; n < N; n += SCHED_THREADS) seq_order[n] = (int32_t)(uint32_t)keys[n];
}

}  // namespace

hipError_t launch_sched(const int64_t* cu_seqlens, int32_t N, int32_t T, int32_t max_chunks, int2* seq_tab,
                        int2* chunk_tab, int2* seq_span, int32_t* seq_order, hipStream_t stream,
                        int32_t win_chunks, int32_t n_win, int32_t* nz_seq, int32_t* win_first) {
  hipLaunchKernelGGL(kda_sched_kernel, dim3(1), dim3(SCHED_THREADS), 0, stream, cu_seqlens, N, T, max_chunks,
                     seq_tab, chunk_tab, seq_span, seq_order, win_chunks, n_win, nz_seq, win_first);
  return hipGetLastError();
}

}  // namespace kda
