// kda_api.cpp -- C ABI of libkda.so: argument validation, workspace layout and
// the launch sequence of the chunked KDA forward on the caller's HIP stream.
//
// Argument list and rules follow flash_kda.fwd and its parameter table
// ("Kernel API" of the FlashKDA README digest, aiwatch.icu page) and the
// caller-owned in-place `out` of the 2kiu.com guide (sections 一 and 三):
// K = V = 128; bf16 q/k/v/g/beta/out; fp32 A_log/dt_bias; lower_bound in
// [-5, 0]; optional bf16/fp32 states of equal dtype; cu_seqlens requires B = 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/kda.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace {

static_assert(kda::FUSE_GATE == KDA_FUSE_GATE && kda::FUSE_QK_L2NORM == KDA_FUSE_QK_L2NORM &&
                  kda::FUSE_BETA_SIGMOID == KDA_FUSE_BETA_SIGMOID && kda::GATE_UNBOUNDED == KDA_GATE_UNBOUNDED,
              "switch values");

constexpr size_t ALIGN = 256;

inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  int64_t max_chunks = 0;
  int64_t nseg = 1;   // segments per row of the segment-parallel state chain (1: plain chain)
  size_t rec = 0, seq_tab = 0, chunk_tab = 0, seq_span = 0, seq_order = 0, maps = 0, seg_init = 0, total = 0;
};

// Segments per row (fixed length) or sequence (varlen, with nc the average chunk
// count, as the lengths stay on the device) for the state chain. The plain chain runs
// one workgroup per (row, head, pair of 16-wide value tiles) through all nc chunks of
// a row, one workgroup per compute unit, so with few (row, head) chains most of the
// GPU idles. Cutting each row into s segments costs a maps pass over twice the value
// rows, a scan of s steps and an outputs pass, each pass over nc / s chunks. Cost in
// chunk steps, for 256 compute units:
//   plain      nc * ceil(BH * 4 / 256)
//   segmented  (nc / s) * (ceil(BH * s * 8 / 256) + ceil(BH * s * 4 / 256)) + 2 s
// The smallest-cost power of two s with segments of at least 8 chunks is taken when it
// saves at least 15%.
int64_t chain_segments(int64_t B, int64_t nc, int64_t H) {
  constexpr int64_t CUS = 256;
  auto waves = [](int64_t wgs) { return (wgs + CUS - 1) / CUS; };
  const int64_t BH = B * H;
  const double plain = (double)nc * (double)waves(BH * 4);
  int64_t best = 1;
  double best_cost = plain;
  for (int64_t s = 2; nc >= 8 * s && s <= 64; s *= 2) {
    const int64_t sc = (nc + s - 1) / s;
    const double cost = (double)sc * (double)(waves(BH * s * 8) + waves(BH * s * 4)) + 2.0 * (double)s;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best_cost <= 0.85 * plain ? best : 1;
}

// Workspace regions: chunk records | seq_tab | chunk_tab | seq_span | seq_order |
// segment maps | segment initial states (the last two only with a segmented chain).
bool make_layout(int64_t B, int64_t T, int64_t H, int64_t N, bool varlen, Layout& L) {
  if (B < 1 || T < 0 || H < 1 || N < 0) return false;
  if (varlen) {
    L.max_chunks = T / kda::CH + N;
  } else {
    L.max_chunks = B * ((T + kda::CH - 1) / kda::CH);
  }
  if (L.max_chunks > INT32_MAX / 2) return false;
  const size_t rec = (size_t)L.max_chunks * (size_t)H * (size_t)kda::REC_BYTES;
  size_t off = 0;
  L.rec = off;
  off = align_up(off + rec);
  L.seq_tab = off;
  off = align_up(off + (varlen ? (size_t)N * sizeof(int2) : 0));
  L.chunk_tab = off;
  off = align_up(off + (varlen ? (size_t)L.max_chunks * sizeof(int2) : 0));
  L.seq_span = off;
  off = align_up(off + (varlen ? (size_t)N * sizeof(int2) : 0));
  L.seq_order = off;
  off = align_up(off + (varlen ? (size_t)N * sizeof(int32_t) : 0));
  const int64_t seqs = varlen ? N : B;
  L.nseg = seqs > 0 ? chain_segments(seqs, varlen ? T / (kda::CH * N) : (T + kda::CH - 1) / kda::CH, H) : 1;
  const size_t segs = L.nseg > 1 ? (size_t)(seqs * L.nseg * H) : 0;
  L.maps = off;
  off = align_up(off + segs * 2 * kda::VD * kda::KD * sizeof(float));
  L.seg_init = off;
  off = align_up(off + segs * kda::VD * kda::KD * sizeof(float));
  L.total = off;
  return true;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Fixed-length calls given less workspace than the full layout run in windows of chunk
// columns: launch pair w covers chunks jb = w * nc_win .. jb + nc_win - 1 of every row
// (the intra-chunk kernel, then the plain state chain), so the records of nc_win chunks
// per row are held at a time. A row's state crosses from one window to the next in fp32:
// in final_state itself when that is fp32 (each workgroup reads its slice of it when it
// starts and writes the slice when it ends), otherwise in a carry region of the
// workspace. Every window runs the same per-chunk arithmetic as one full launch and the
// carried state is exact, so the results are bit-identical to an unwindowed call; the
// chain takes the same number of steps per row, split over the windows.
constexpr size_t WORKSPACE_TARGET = (size_t)4 << 30;   // kda_fwd_workspace_size's bound where windows apply
struct Windows {
  int64_t count = 0, nc_win = 0;
  size_t rec = 0, carry = 0, total = 0;
  bool own_carry = false;
};
size_t carry_bytes(int64_t B, int64_t H) { return align_up((size_t)B * H * kda::VD * kda::KD * sizeof(float)); }
size_t column_bytes(int64_t B, int64_t H) { return (size_t)B * H * kda::REC_BYTES; }   // a multiple of 256
static_assert(kda::REC_BYTES % ALIGN == 0, "records keep the workspace alignment");
bool plan_windows(int64_t B, int64_t T, int64_t H, bool final_fp32, size_t bytes, Windows& W) {
  const int64_t nc_row = (T + kda::CH - 1) / kda::CH;
  if (nc_row < 1) return false;
  W.own_carry = !final_fp32;
  W.carry = W.own_carry ? carry_bytes(B, H) : 0;
  const size_t col = column_bytes(B, H);
  if (bytes < W.carry + col) return false;
  const int64_t fit = (int64_t)((bytes - W.carry) / col);
  W.count = (nc_row + fit - 1) / fit;                 // fewest windows, then balanced widths
  W.nc_win = (nc_row + W.count - 1) / W.count;
  W.rec = (size_t)W.nc_win * col;
  W.total = W.rec + W.carry;
  return true;
}

// Varlen calls given less workspace than the full layout run in windows of chunk slots:
// launch pair w is the intra kernel over slots w * nc_win .. (w + 1) * nc_win - 1 and the
// chain over the parts of the sequences inside them (the scheduler lists, per window, the
// sequences with chunks that reach into it). A sequence that crosses a window boundary
// passes its state to the next window in fp32 through one of two carry slots (at most one
// sequence crosses each boundary); sequences without chunks take their initial state (or
// zeros) in a kernel of their own, since no window visits them. Results are bit-identical
// to one launch pair. Layout: records | seq_tab | chunk_tab | seq_span | seq_order | nz_seq
// | win_first | carry.
struct VWindows {
  int64_t count = 0, nc_win = 0;
  size_t rec = 0, seq_tab = 0, chunk_tab = 0, seq_span = 0, seq_order = 0, nz_seq = 0, win_first = 0, carry = 0,
         total = 0;
};
size_t vwindow_fixed_bytes(int64_t N, int64_t max_chunks, int64_t H) {
  return align_up((size_t)N * sizeof(int2)) * 2 + align_up((size_t)max_chunks * sizeof(int2)) +
         align_up((size_t)N * sizeof(int32_t)) * 2 + align_up((size_t)(max_chunks + 1) * sizeof(int32_t)) +
         align_up((size_t)2 * H * kda::VD * kda::KD * sizeof(float));
}
bool plan_vwindows(int64_t T, int64_t H, int64_t N, size_t bytes, VWindows& W) {
  const int64_t max_chunks = T / kda::CH + N;
  if (max_chunks < 1) return false;
  const size_t fixed = vwindow_fixed_bytes(N, max_chunks, H);
  const size_t slot = (size_t)H * kda::REC_BYTES;   // a multiple of 256
  if (bytes < fixed + slot) return false;
  const int64_t fit = (int64_t)((bytes - fixed) / slot);
  W.count = (max_chunks + fit - 1) / fit;
  W.nc_win = (max_chunks + W.count - 1) / W.count;
  size_t off = 0;
  W.rec = off;
  off += (size_t)W.nc_win * slot;
  W.seq_tab = off;
  off += align_up((size_t)N * sizeof(int2));
  W.chunk_tab = off;
  off += align_up((size_t)max_chunks * sizeof(int2));
  W.seq_span = off;
  off += align_up((size_t)N * sizeof(int2));
  W.seq_order = off;
  off += align_up((size_t)N * sizeof(int32_t));
  W.nz_seq = off;
  off += align_up((size_t)N * sizeof(int32_t));
  W.win_first = off;
  off += align_up((size_t)(max_chunks + 1) * sizeof(int32_t));
  W.carry = off;
  off += align_up((size_t)2 * H * kda::VD * kda::KD * sizeof(float));
  W.total = off;
  return W.total <= bytes;
}

// Calls that kda_fwd / kda_fwd_ex hand to the token-recurrent kernel: fixed-length rows of
// at most REC_MAX_T tokens, or varlen batches of at most REC_MAX_AVG tokens per sequence on
// average (the lengths themselves stay on the device). The chunked path costs a full
// 64-token chunk of intra-chunk work and one chain step per (sequence, head) whatever the
// length, while the recurrent kernel's cost grows with each sequence's length. Measured at
// H = 64: fixed length, the recurrent kernel is faster up to T = 8 for B = 1, 4 and 16
// (the two cross between T = 12 and 16); varlen, it is 2.5x faster at up to 4 tokens per
// sequence, and with T <= 2 N even one sequence holding every token (up to 2 N tokens
// serially) costs no more than the chunked path does for the same call.
constexpr int64_t REC_MAX_T = 8, REC_MAX_AVG = 2;
inline bool short_call(int64_t T, int64_t N, bool varlen) {
  return varlen ? T <= REC_MAX_AVG * N : T <= REC_MAX_T;
}

bool env_flag(const char* name) {
  const char* s = std::getenv(name);
  return s && s[0] == '1';
}

// Shared argument checks of both entry points.
int check_common(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                 const void* out, const float* A_log, const float* dt_bias, float lower_bound,
                 const void* initial_state, int initial_dtype, const void* final_state, int final_dtype,
                 const int64_t* cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                 uint32_t flags) {
  if (flags & ~(uint32_t)(KDA_FUSE_ALL | KDA_GATE_UNBOUNDED | KDA_PATH_CHUNKED)) return KDA_ERR_VALUE;
  const bool gate_fused = (flags & KDA_FUSE_GATE) != 0;
  // with no tokens the token-indexed buffers hold no element (an empty tensor's data
  // pointer may be NULL); no kernel reads or writes them then
  if (T != 0 && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_NULL;
  if (gate_fused && (!A_log || !dt_bias)) return KDA_ERR_NULL;
  if (K != kda::KD || V != kda::VD) return KDA_ERR_SHAPE;
  if (B < 1 || T < 0 || H < 1 || H > (1 << 20)) return KDA_ERR_SHAPE;
  if (cu_seqlens && (B != 1 || N < 1)) return KDA_ERR_SHAPE;
  if (B * T >= (int64_t)INT32_MAX / 2) return KDA_ERR_SHAPE;
  const int64_t nseq = cu_seqlens ? N : B;
  if (nseq * H >= (int64_t)INT32_MAX / 256) return KDA_ERR_SHAPE;
  auto bad_code = [](int c) { return c != KDA_STATE_NONE && c != KDA_STATE_BF16 && c != KDA_STATE_FP32; };
  if (bad_code(initial_dtype) || bad_code(final_dtype)) return KDA_ERR_DTYPE;
  if ((initial_dtype == KDA_STATE_NONE) != (initial_state == nullptr))
    return initial_state ? KDA_ERR_DTYPE : KDA_ERR_NULL;
  if ((final_dtype == KDA_STATE_NONE) != (final_state == nullptr)) return final_state ? KDA_ERR_DTYPE : KDA_ERR_NULL;
  if (initial_state && final_state && initial_dtype != final_dtype) return KDA_ERR_DTYPE;
  if (!(flags & KDA_GATE_UNBOUNDED) && (!std::isfinite(lower_bound) || lower_bound < -5.0f || lower_bound > 0.0f))
    return KDA_ERR_VALUE;
  if (!std::isfinite(scale)) return KDA_ERR_VALUE;
  const void* a16[] = {q, k, v, g, out, A_log, dt_bias};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return KDA_ERR_ALIGN;
  if (!aligned(beta, 2)) return KDA_ERR_ALIGN;
  if (initial_state && !aligned(initial_state, 16)) return KDA_ERR_ALIGN;
  if (final_state && !aligned(final_state, 16)) return KDA_ERR_ALIGN;
  if (cu_seqlens && !aligned(cu_seqlens, 8)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

// Copies the boundaries to the host in pieces through a stack buffer (no allocation).
int validate_cu_on_host(const int64_t* cu, int64_t N, int64_t T, hipStream_t stream) {
  if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
  constexpr int64_t PIECE = 512;
  int64_t h[PIECE];
  int64_t prev = 0;
  for (int64_t i0 = 0; i0 <= N; i0 += PIECE) {
    const int64_t n = (N + 1 - i0) < PIECE ? (N + 1 - i0) : PIECE;
    if (hipMemcpy(h, cu + i0, sizeof(int64_t) * (size_t)n, hipMemcpyDeviceToHost) != hipSuccess) return KDA_ERR_HIP;
    for (int64_t i = 0; i < n; ++i) {
      if (i0 + i == 0 ? h[i] != 0 : h[i] < prev) return KDA_ERR_VALUE;
      prev = h[i];
    }
  }
  return prev == T ? KDA_OK : KDA_ERR_VALUE;
}

kda::FwdParams make_params(const void* q, const void* k, const void* v, const void* g, const void* beta,
                           float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
                           const void* initial_state, int initial_dtype, void* final_state, int final_dtype,
                           int64_t H, uint32_t flags) {
  kda::FwdParams p{};
  p.flags = flags;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = static_cast<const uint16_t*>(g);
  p.beta = static_cast<const uint16_t*>(beta);
  p.out = static_cast<uint16_t*>(out);
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.init_state = initial_state;
  p.final_state = final_state;
  p.init_dtype = initial_dtype;
  p.final_dtype = final_dtype;
  p.scale = scale;
  p.lower_bound = lower_bound;
  p.H = (int32_t)H;
  return p;
}


// ---- optional per-kernel timing of kda_fwd ---------------------------------
// While enabled, each kda_fwd call takes the next slot of NK + 1 HIP events and
// records one on the call's stream before its first kernel and one after each
// kernel, so consecutive events bracket one kernel each (the event before the
// scheduler only when the scheduler runs).
constexpr int NK = 3;   // 0 varlen scheduler, 1 intra-chunk, 2 state chain + output
const char* const kKernelNames[NK] = {"kda_sched_kernel", "kda_intra_kernel", "kda_chain_kernel"};

struct Profiler {
  std::mutex mu;
  bool on = false;
  int cap = 0, used = 0;
  std::vector<hipEvent_t> ev;   // cap x (NK + 1)
  std::vector<uint8_t> ran;     // cap x NK: kernel i launched in that call
};
Profiler& profiler() {
  static Profiler P;
  return P;
}
void profiler_release(Profiler& P) {
  for (hipEvent_t e : P.ev) (void)hipEventDestroy(e);
  P.ev.clear();
  P.ran.clear();
  P.on = false;
  P.cap = P.used = 0;
}

// Takes a slot for one call (or none when timing is off or the slots are used up).
struct CallTimer {
  hipEvent_t* ev = nullptr;
  uint8_t* ran = nullptr;
  hipStream_t st;
  explicit CallTimer(hipStream_t s) : st(s) {
    Profiler& P = profiler();
    std::lock_guard<std::mutex> lk(P.mu);
    if (!P.on || P.used >= P.cap) return;
    ev = &P.ev[(size_t)P.used * (NK + 1)];
    ran = &P.ran[(size_t)P.used * NK];
    ++P.used;
  }
  hipError_t mark(int i) {   // i = 0: before the first kernel; i > 0: after kernel i - 1
    return ev ? hipEventRecord(ev[i], st) : hipSuccess;
  }
  void launched(int k) {
    if (ran) ran[k] = 1;
  }
};
}  // namespace

extern "C" {

size_t kda_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t N) {
  Layout L;
  if (!make_layout(B, T, H, N, N > 0, L)) return 0;
  // calls on the plain chain: windows within WORKSPACE_TARGET (at T = 32768, B = 4, H = 64
  // the full 9.5 GiB, 4 GiB in three windows and 1 GiB in ten take the same time; fewer,
  // wider windows cost less where they do not: a ragged batch of 32 sequences, 2.2 GB in
  // one launch pair, took 3% longer in three windows)
  if (L.nseg == 1 && L.total > WORKSPACE_TARGET) {
    if (N == 0) {
      Windows W;
      if (plan_windows(B, T, H, false, WORKSPACE_TARGET, W) && W.total < L.total) return W.total;
    } else {
      VWindows V;
      if (plan_vwindows(T, H, N, WORKSPACE_TARGET, V) && V.total < L.total) return V.total;
    }
  }
  return L.total;
}

size_t kda_fwd_workspace_min(int64_t B, int64_t T, int64_t H, int64_t N) {
  Layout L;
  if (!make_layout(B, T, H, N, N > 0, L)) return 0;
  if (L.total == 0) return 0;
  const size_t one = N > 0 ? vwindow_fixed_bytes(N, L.max_chunks, H) + (size_t)H * kda::REC_BYTES   // one slot
                           : carry_bytes(B, H) + column_bytes(B, H);   // one chunk column and a carry
  return one < L.total ? one : L.total;
}

int kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale, void* out,
            const float* A_log, const float* dt_bias, float lower_bound, const void* initial_state,
            int initial_dtype, void* final_state, int final_dtype, const int64_t* cu_seqlens, int64_t N, int64_t B,
            int64_t T, int64_t H, int64_t K, int64_t V, void* workspace, size_t workspace_bytes, void* stream) {
  return kda_fwd_ex(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, initial_dtype,
                    final_state, final_dtype, cu_seqlens, N, B, T, H, K, V, KDA_FUSE_ALL, workspace,
                    workspace_bytes, stream);
}

int kda_fwd_ex(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale, void* out,
               const float* A_log, const float* dt_bias, float lower_bound, const void* initial_state,
               int initial_dtype, void* final_state, int final_dtype, const int64_t* cu_seqlens, int64_t N,
               int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, uint32_t flags, void* workspace,
               size_t workspace_bytes, void* stream) {
  int rc = check_common(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, initial_dtype,
                        final_state, final_dtype, cu_seqlens, N, B, T, H, K, V, flags);
  if (rc != KDA_OK) return rc;
  const bool varlen = cu_seqlens != nullptr;
  Layout L;
  if (!make_layout(B, T, H, varlen ? N : 0, varlen, L)) return KDA_ERR_SHAPE;
  Windows W;    // W.count > 0: the call runs in windows of chunk columns (fixed length)
  VWindows VW;   // VW.count > 0: in windows of chunk slots (varlen)
  if (L.total > 0) {
    if (!workspace) return KDA_ERR_WORKSPACE;
    if (workspace_bytes < L.total &&
        !(varlen ? plan_vwindows(T, H, N, workspace_bytes, VW)
                 : plan_windows(B, T, H, final_dtype == KDA_STATE_FP32, workspace_bytes, W)))
      return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, ALIGN)) return KDA_ERR_ALIGN;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (varlen && env_flag("KDA_VALIDATE")) {
    rc = validate_cu_on_host(cu_seqlens, N, T, st);
    if (rc != KDA_OK) return rc;
  }
  const bool force_chunked = (flags & KDA_PATH_CHUNKED) != 0;
  flags &= ~(uint32_t)KDA_PATH_CHUNKED;

  kda::FwdParams p = make_params(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                                 initial_dtype, final_state, final_dtype, H, flags);
  if (!force_chunked && short_call(T, N, varlen)) {   // decode-sized: token by token
    p.map.T = (int32_t)T;
    p.map.nseq = (int32_t)(varlen ? N : B);
    if (env_flag("KDA_LOG"))
      std::fprintf(stderr, "[kda] fwd B=%lld T=%lld H=%lld N=%lld path=recurrent\n", (long long)B, (long long)T,
                   (long long)H, (long long)N);
    const hipError_t e = kda::launch_recurrent(p, cu_seqlens, st);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.rec = ws + L.rec;
  p.map.T = (int32_t)T;
  p.map.max_chunks = (int32_t)L.max_chunks;
  p.map.nseq = (int32_t)(varlen ? N : B);
  p.map.nc_row = (int32_t)((T + kda::CH - 1) / kda::CH);
  p.map.jb = 0;
  p.map.nc_win = p.map.nc_row;
  if (W.count > 0) {   // windows of chunk columns (no per-kernel timing for these calls)
    if (env_flag("KDA_LOG"))
      std::fprintf(stderr, "[kda] fwd B=%lld T=%lld H=%lld windows=%lld x %lld chunks workspace=%zu of %zu\n",
                   (long long)B, (long long)T, (long long)H, (long long)W.count, (long long)W.nc_win, W.total,
                   L.total);
    p.rec = ws;
    void* carry = W.own_carry ? static_cast<void*>(ws + W.rec) : final_state;
    hipError_t e = hipSuccess;
    for (int64_t w = 0; w < W.count && e == hipSuccess; ++w) {
      const int64_t jb = w * W.nc_win;
      const int64_t width = std::min<int64_t>(W.nc_win, p.map.nc_row - jb);
      p.map.jb = (int32_t)jb;
      p.map.nc_win = (int32_t)width;
      p.map.max_chunks = (int32_t)(B * width);
      p.init_state = w == 0 ? initial_state : carry;
      p.init_dtype = w == 0 ? initial_dtype : KDA_STATE_FP32;
      const bool last = w + 1 == W.count;
      p.final_state = last ? final_state : carry;
      p.final_dtype = last ? final_dtype : KDA_STATE_FP32;
      e = kda::launch_intra(p, st);
      if (e == hipSuccess) e = kda::launch_chain(p, st);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  if (VW.count > 0) {   // varlen windows of chunk slots (no per-kernel timing for these calls)
    if (env_flag("KDA_LOG"))
      std::fprintf(stderr, "[kda] fwd T=%lld H=%lld N=%lld windows=%lld x %lld slots workspace=%zu of %zu\n",
                   (long long)T, (long long)H, (long long)N, (long long)VW.count, (long long)VW.nc_win, VW.total,
                   L.total);
    p.rec = ws + VW.rec;
    p.map.seq_tab = reinterpret_cast<const int2*>(ws + VW.seq_tab);
    p.map.chunk_tab = reinterpret_cast<const int2*>(ws + VW.chunk_tab);
    p.map.seq_span = reinterpret_cast<const int2*>(ws + VW.seq_span);
    p.map.seq_order = nullptr;
    p.map.nz_seq = reinterpret_cast<const int32_t*>(ws + VW.nz_seq);
    p.map.win_first = reinterpret_cast<const int32_t*>(ws + VW.win_first);
    p.map.carry = reinterpret_cast<float*>(ws + VW.carry);
    p.map.n_win = (int32_t)VW.count;
    hipError_t e = kda::launch_sched(cu_seqlens, (int32_t)N, (int32_t)T, (int32_t)L.max_chunks,
                                     reinterpret_cast<int2*>(ws + VW.seq_tab), reinterpret_cast<int2*>(ws + VW.chunk_tab),
                                     reinterpret_cast<int2*>(ws + VW.seq_span), reinterpret_cast<int32_t*>(ws + VW.seq_order),
                                     st, (int32_t)VW.nc_win, (int32_t)VW.count, reinterpret_cast<int32_t*>(ws + VW.nz_seq),
                                     reinterpret_cast<int32_t*>(ws + VW.win_first));
    if (e == hipSuccess) e = kda::launch_empty_states(p, (int32_t)N, st);
    for (int64_t w = 0; w < VW.count && e == hipSuccess; ++w) {
      const int64_t jb = w * VW.nc_win;
      p.map.jb = (int32_t)jb;
      p.map.nc_win = (int32_t)VW.nc_win;
      p.map.max_chunks = (int32_t)std::min<int64_t>(VW.nc_win, L.max_chunks - jb);
      p.map.win = (int32_t)w;
      // the chain's sequence capacity per window: a window meets at most nc_win + 1
      // sequences with chunks, and there are N in all
      p.map.nseq = (int32_t)std::min<int64_t>(VW.nc_win + 1, N);
      e = kda::launch_intra(p, st);
      if (e == hipSuccess) e = kda::launch_chain(p, st);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  // segment-parallel chain: the layout's segment count, or fewer with KDA_CHAIN_SEGMENTS
  int64_t nseg = L.nseg;
  if (const char* e = std::getenv("KDA_CHAIN_SEGMENTS")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v < nseg) nseg = v;
  }
  if (nseg > 1) {
    p.seg.nseg = (int32_t)nseg;
    p.seg.maps = reinterpret_cast<float*>(ws + L.maps);
    p.seg.seg_init = reinterpret_cast<float*>(ws + L.seg_init);
  }
  if (varlen) {
    p.map.seq_tab = reinterpret_cast<const int2*>(ws + L.seq_tab);
    p.map.chunk_tab = reinterpret_cast<const int2*>(ws + L.chunk_tab);
    p.map.seq_span = reinterpret_cast<const int2*>(ws + L.seq_span);
    p.map.seq_order = reinterpret_cast<const int32_t*>(ws + L.seq_order);
  }
  if (env_flag("KDA_LOG"))
    std::fprintf(stderr, "[kda] fwd B=%lld T=%lld H=%lld N=%lld chunks=%lld workspace=%zu varlen=%d segments=%lld\n",
                 (long long)B, (long long)T, (long long)H, (long long)N, (long long)L.max_chunks, L.total,
                 (int)varlen, (long long)nseg);

  CallTimer tm(st);
  hipError_t e = hipSuccess;
  if (varlen && L.max_chunks > 0) {   // (without the scheduler its interval is unused: no event)
    e = tm.mark(0);
    if (e == hipSuccess)
      e = kda::launch_sched(cu_seqlens, (int32_t)N, (int32_t)T, (int32_t)L.max_chunks,
                            reinterpret_cast<int2*>(ws + L.seq_tab), reinterpret_cast<int2*>(ws + L.chunk_tab),
                            reinterpret_cast<int2*>(ws + L.seq_span), reinterpret_cast<int32_t*>(ws + L.seq_order),
                            st);
    tm.launched(0);
  }
  if (e == hipSuccess) e = tm.mark(1);
  if (e == hipSuccess) {
    e = kda::launch_intra(p, st);
    tm.launched(1);
  }
  if (e == hipSuccess) e = tm.mark(2);
  if (e == hipSuccess && nseg > 1) {   // segment maps, their composition, then the outputs
    p.seg.mode = kda::CHAIN_MAPS;
    e = kda::launch_chain(p, st);
    if (e == hipSuccess) e = kda::launch_scan(p, p.map.nseq, st);
    p.seg.mode = kda::CHAIN_OUTPUTS;
    if (e == hipSuccess) e = kda::launch_chain(p, st);
    tm.launched(2);
  } else if (e == hipSuccess) {
    e = kda::launch_chain(p, st);
    tm.launched(2);
  }
  if (e == hipSuccess) e = tm.mark(3);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_fwd_recurrent(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                      void* out, const float* A_log, const float* dt_bias, float lower_bound,
                      const void* initial_state, int initial_dtype, void* final_state, int final_dtype,
                      const int64_t* cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                      void* stream) {
  return kda_fwd_recurrent_ex(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                              initial_dtype, final_state, final_dtype, cu_seqlens, N, B, T, H, K, V, KDA_FUSE_ALL,
                              stream);
}

int kda_fwd_recurrent_ex(const void* q, const void* k, const void* v, const void* g, const void* beta, float scale,
                         void* out, const float* A_log, const float* dt_bias, float lower_bound,
                         const void* initial_state, int initial_dtype, void* final_state, int final_dtype,
                         const int64_t* cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K,
                         int64_t V, uint32_t flags, void* stream) {
  if (flags & KDA_PATH_CHUNKED) return KDA_ERR_VALUE;
  int rc = check_common(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state, initial_dtype,
                        final_state, final_dtype, cu_seqlens, N, B, T, H, K, V, flags);
  if (rc != KDA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool varlen = cu_seqlens != nullptr;
  if (varlen && env_flag("KDA_VALIDATE")) {
    rc = validate_cu_on_host(cu_seqlens, N, T, st);
    if (rc != KDA_OK) return rc;
  }
  kda::FwdParams p = make_params(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                                 initial_dtype, final_state, final_dtype, H, flags);
  p.map.T = (int32_t)T;
  p.map.nseq = (int32_t)(varlen ? N : B);
  hipError_t e = kda::launch_recurrent(p, cu_seqlens, st);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: unsupported or inconsistent sizes (K = V = 128, B = 1 with cu_seqlens)";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown state dtype or initial/final state dtypes differ";
    case KDA_ERR_VALUE: return "KDA_ERR_VALUE: lower_bound outside [-5, 0], non-finite scale, or bad cu_seqlens";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: pointer not aligned (16 bytes; workspace 256 bytes)";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or smaller than kda_fwd_workspace_size";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime or kernel launch error";
    case KDA_ERR_CAPACITY:
      return "KDA_ERR_CAPACITY: the call needs more workspace than kda_fwd_noalloc's fixed array (256 MiB) holds";
    default: return "KDA: unknown status";
  }
}

const char* kda_version(void) { return "0.1.0 gfx950"; }

int kda_profile_start(int max_calls) {
  if (max_calls < 1 || max_calls > 65536) return KDA_ERR_VALUE;
  Profiler& P = profiler();
  std::lock_guard<std::mutex> lk(P.mu);
  profiler_release(P);
  P.ev.reserve((size_t)max_calls * (NK + 1));
  for (size_t i = 0; i < (size_t)max_calls * (NK + 1); ++i) {
    hipEvent_t e;
    // timing only: no system-scope fence (cache write-back) at each record, which would
    // otherwise add several microseconds to every timed call
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      profiler_release(P);
      return KDA_ERR_HIP;
    }
    P.ev.push_back(e);
  }
  P.ran.assign((size_t)max_calls * NK, 0);
  P.cap = max_calls;
  P.used = 0;
  P.on = true;
  return KDA_OK;
}

int kda_profile_stop(double* total_ms, int* launches, int n_kernels) {
  if (!total_ms || !launches) return KDA_ERR_NULL;
  if (n_kernels < NK) return KDA_ERR_SHAPE;
  Profiler& P = profiler();
  std::lock_guard<std::mutex> lk(P.mu);
  if (!P.on) return KDA_ERR_VALUE;
  for (int i = 0; i < n_kernels; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  int rc = KDA_OK;
  for (int c = 0; c < P.used && rc == KDA_OK; ++c) {
    hipEvent_t* ev = &P.ev[(size_t)c * (NK + 1)];
    if (hipEventSynchronize(ev[NK]) != hipSuccess) {
      rc = KDA_ERR_HIP;
      break;
    }
    for (int k = 0; k < NK; ++k) {
      if (!P.ran[(size_t)c * NK + k]) continue;
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, ev[k], ev[k + 1]) != hipSuccess) {
        rc = KDA_ERR_HIP;
        break;
      }
      total_ms[k] += ms;
      launches[k] += 1;
    }
  }
  profiler_release(P);
  return rc;
}

int kda_profile_kernel_count(void) { return NK; }

const char* kda_profile_kernel_name(int i) { return (i >= 0 && i < NK) ? kKernelNames[i] : ""; }

}  // extern "C"
