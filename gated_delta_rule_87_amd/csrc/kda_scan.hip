// kda_scan.hip -- composes the segment maps of the segment-parallel state chain
// (gfx950).
//
// A segment of chunks acts on the state S (V x K) as the affine map S -> S P + R:
// R is the segment's final state from a zero start, P (K x K) the final state of the
// identity run through the recurrence without U~ (both written by the chain kernel's
// maps pass). Per fixed-length row and head the segments are composed in order,
//     S_0 = initial state (or 0),   S_{s+1} = S_s P_s + R_s,
// writing every S_s as that segment's initial state and the last one as final_state.
// This is the exchange step of the context-parallel form of the recurrence (page
// "FlashKDA：面向SM90+的高性能KDA CUDA内核库", Q2 on long contexts and state
// passing), done here between the segments of one GPU.
//
// Value rows are independent, so one workgroup handles one 16-row value tile of one
// (row, head): wave w computes output channel tiles 2w and 2w+1 of
//     S^T_new = P^T S^T + R^T
// on fp32 MFMA 16x16x4, with the slice of P it needs (128 x 32) loaded straight into
// registers as A fragments. The 16 x 128 state tile is the B operand: with the
// contraction index of k-step (mt, j) held by lane group gq as channel 16 mt + 4 gq + j,
// the D layout of the result (lane (gq, lt) -> S[16 vt + lt][16 ct + 4 gq + j]) is the
// operand layout itself; the waves exchange their tiles through 8 KiB of LDS per step.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

__global__ __launch_bounds__(256) void kda_scan_kernel(FwdParams p, int32_t rows) {
  __shared__ f32x4 sx[8][64];   // the state tile, [channel tile][lane] in D layout
  const int H = p.H;
  const int vt = blockIdx.x & 7, bh = blockIdx.x >> 3;
  const int b = bh / H, h = bh - (bh / H) * H;
  if (b >= rows) return;   // uniform over the block
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lt = l & 15, gq = l >> 4;
  const int nseg = p.seg.nseg;

  // this wave's two output channel tiles ct = 2w + c
  f32x4 S[2];
  const size_t st_off = ((size_t)(b * H + h) * VD + 16 * vt + lt) * KD;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ct = 2 * w + c;
    if (p.init_dtype == 2) {
      S[c] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.init_state) + st_off + 16 * ct + 4 * gq);
    } else if (p.init_dtype == 1) {
      const u32x2 r = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.init_state) + st_off + 16 * ct + 4 * gq);
      S[c] = f32x4{bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y)};
    } else {
      S[c] = f32x4{0, 0, 0, 0};
    }
    sx[ct][l] = S[c];
  }

  for (int sg = 0; sg < nseg; ++sg) {
    const size_t seg = (size_t)(b * nseg + sg) * H + h;
    float* init = p.seg.seg_init + (seg * VD + 16 * vt + lt) * KD;
#pragma unroll
    for (int c = 0; c < 2; ++c) *reinterpret_cast<f32x4*>(init + 16 * (2 * w + c) + 4 * gq) = S[c];

    const float* map = p.seg.maps + seg * (2 * VD) * KD;   // rows 0-127 R, 128-255 P
    // A fragments: a[c][mt][j] = P[16 mt + 4 gq + j][16 (2w + c) + lt]
    float a[2][8][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          a[c][mt][jj] = map[(size_t)(VD + 16 * mt + 4 * gq + jj) * KD + 16 * (2 * w + c) + lt];
    f32x4 acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
      acc[c] = *reinterpret_cast<const f32x4*>(map + (size_t)(16 * vt + lt) * KD + 16 * (2 * w + c) + 4 * gq);
    __syncthreads();   // sx holds this step's state tile
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const f32x4 sb = sx[mt][l];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c][mt][jj], sb[jj], acc[c], 0, 0, 0);
    }
    __syncthreads();   // every wave has read sx
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      S[c] = acc[c];
      sx[2 * w + c][l] = acc[c];
    }
  }

#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ct = 2 * w + c;
    if (p.final_dtype == 2) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.final_state) + st_off + 16 * ct + 4 * gq) = S[c];
    } else if (p.final_dtype == 1) {
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.final_state) + st_off + 16 * ct + 4 * gq) =
          u32x2{pack_bf16x2(S[c].x, S[c].y), pack_bf16x2(S[c].z, S[c].w)};
    }
  }
}

}  // namespace

hipError_t launch_scan(const FwdParams& p, int32_t rows, hipStream_t stream) {
  const int64_t blocks = (int64_t)rows * p.H * (VD / 16);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, rows);
  return hipGetLastError();
}

}  // namespace kda
