// kda_recurrent.hip -- token-by-token KDA forward (gfx950).
//
// One workgroup of 128 threads per (sequence, head). Thread v keeps state row
// S[v][0..127] in fp32 registers; every token it
//     decays the row (S[v][c] *= exp(g~[c])),
//     applies the delta update (S[v] -= beta (S[v].k^ - v_t[v]) k^),
//     and reads out o[v] = scale S[v].q^,
// with the per-token prologue (gate activation, beta sigmoid, q/k L2 norms)
// computed once per wave into LDS. Used for online generation with state
// passing (page "FlashKDA：面向SM90+的高性能KDA CUDA内核库", Q2 on
// stateful/streaming use), where T per call is small, and as an independent
// long-input reference for the chunked path.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

__device__ __forceinline__ float decay(float g, float dt, float rate, float lb, bool fuse_gate, bool unbounded) {
  if (fuse_gate)
    return unbounded ? fast_exp2(-rate * softplus_log2((g + dt) * LOG2E)) : expf(lb / (1.0f + expf(-rate * (g + dt))));
  return expf(unbounded ? fminf(g, 0.0f) : fminf(fmaxf(g, lb), 0.0f));
}

__global__ __launch_bounds__(128) void kda_recurrent_kernel(FwdParams p, const int64_t* cu) {
  __shared__ f32x4 sk[2][2][KD / 4], sq[2][2][KD / 4], sa[2][2][KD / 4];   // [buffer][wave][channel/4]
  const int H = p.H;
  const int n = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int T = p.map.T;

  int64_t tb, te;
  if (cu) {
    int64_t a = cu[n], b = cu[n + 1];
    a = a < 0 ? 0 : (a > T ? T : a);
    b = b < a ? a : (b > T ? T : b);
    tb = a;
    te = b;
  } else {
    tb = (int64_t)n * T;
    te = tb + T;
  }

  float S[KD];
  const size_t st_off = ((size_t)(n * H + h) * VD + tid) * KD;
  if (p.init_dtype == 2) {
    const float* src = static_cast<const float*>(p.init_state) + st_off;
#pragma unroll
    for (int c = 0; c < KD; c += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + c);
      S[c] = x.x; S[c + 1] = x.y; S[c + 2] = x.z; S[c + 3] = x.w;
    }
  } else if (p.init_dtype == 1) {
    const uint16_t* src = static_cast<const uint16_t*>(p.init_state) + st_off;
#pragma unroll
    for (int c = 0; c < KD; c += 2) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(src + c);
      S[c] = bf16_lo(x); S[c + 1] = bf16_hi(x);
    }
  } else {
#pragma unroll
    for (int c = 0; c < KD; ++c) S[c] = 0.0f;
  }

  const bool fuse_gate = (p.flags & FUSE_GATE) != 0, fuse_norm = (p.flags & FUSE_QK_L2NORM) != 0;
  const bool fuse_beta = (p.flags & FUSE_BETA_SIGMOID) != 0, unbounded = (p.flags & GATE_UNBOUNDED) != 0;
  const float rate = fuse_gate ? expf(p.A_log[h]) : 0.0f;
  const float lb = p.lower_bound, scale = p.scale;
  const float2 dt = fuse_gate ? *reinterpret_cast<const float2*>(p.dt_bias + (size_t)h * KD + 2 * lane)
                              : make_float2(0.0f, 0.0f);
  int buf = 0;
  for (int64_t t = tb; t < te; ++t, buf ^= 1) {
    const size_t row = ((size_t)t * H + h) * KD;
    // prologue, computed by each wave for all 128 channels (lane: channels 2*lane, 2*lane+1)
    const uint32_t qw = *reinterpret_cast<const uint32_t*>(p.q + row + 2 * lane);
    const uint32_t kw = *reinterpret_cast<const uint32_t*>(p.k + row + 2 * lane);
    const uint32_t gw = *reinterpret_cast<const uint32_t*>(p.g + row + 2 * lane);
    const float q0 = bf16_lo(qw), q1 = bf16_hi(qw), k0 = bf16_lo(kw), k1 = bf16_hi(kw);
    float ssq = q0 * q0 + q1 * q1, ssk = k0 * k0 + k1 * k1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      ssq += __shfl_xor(ssq, o, 64);
      ssk += __shfl_xor(ssk, o, 64);
    }
    const float rq = fuse_norm ? rsqrtf(ssq + 1e-6f) : 1.0f, rk = fuse_norm ? rsqrtf(ssk + 1e-6f) : 1.0f;
    // decay factors exp(g~): fused gate activation (safe: lb sigmoid(rate x); unbounded:
    // -rate softplus(x), as 2^(-rate log2(1 + 2^(x log2 e)))), or the given log-decay
    // clamped into [lb, 0] (unbounded: min(g, 0))
    const float a0 = decay(bf16_lo(gw), dt.x, rate, lb, fuse_gate, unbounded);
    const float a1 = decay(bf16_hi(gw), dt.y, rate, lb, fuse_gate, unbounded);
    float* skf = reinterpret_cast<float*>(&sk[buf][w][0]);
    float* sqf = reinterpret_cast<float*>(&sq[buf][w][0]);
    float* saf = reinterpret_cast<float*>(&sa[buf][w][0]);
    skf[2 * lane] = k0 * rk; skf[2 * lane + 1] = k1 * rk;
    sqf[2 * lane] = q0 * rq; sqf[2 * lane + 1] = q1 * rq;
    saf[2 * lane] = a0; saf[2 * lane + 1] = a1;
    const float braw = bf16_to_f32(p.beta[(size_t)t * H + h]);
    const float beta = fuse_beta ? 1.0f / (1.0f + expf(-braw)) : braw;
    const float vv = bf16_to_f32(p.v[row + tid]);
    __syncthreads();

    float dot = 0.0f;
#pragma unroll
    for (int c4 = 0; c4 < KD / 4; ++c4) {
      const f32x4 a = sa[buf][w][c4], kk = sk[buf][w][c4];
      S[4 * c4] *= a.x; S[4 * c4 + 1] *= a.y; S[4 * c4 + 2] *= a.z; S[4 * c4 + 3] *= a.w;
      dot += S[4 * c4] * kk.x + S[4 * c4 + 1] * kk.y + S[4 * c4 + 2] * kk.z + S[4 * c4 + 3] * kk.w;
    }
    const float u = beta * (dot - vv);
    float o = 0.0f;
#pragma unroll
    for (int c4 = 0; c4 < KD / 4; ++c4) {
      const f32x4 kk = sk[buf][w][c4], qq = sq[buf][w][c4];
      S[4 * c4] -= u * kk.x; S[4 * c4 + 1] -= u * kk.y; S[4 * c4 + 2] -= u * kk.z; S[4 * c4 + 3] -= u * kk.w;
      o += S[4 * c4] * qq.x + S[4 * c4 + 1] * qq.y + S[4 * c4 + 2] * qq.z + S[4 * c4 + 3] * qq.w;
    }
    p.out[row + tid] = to_bf16(scale * o);
  }

  if (p.final_dtype == 2) {
    float* dst = static_cast<float*>(p.final_state) + st_off;
#pragma unroll
    for (int c = 0; c < KD; c += 4) *reinterpret_cast<f32x4*>(dst + c) = f32x4{S[c], S[c + 1], S[c + 2], S[c + 3]};
  } else if (p.final_dtype == 1) {
    uint16_t* dst = static_cast<uint16_t*>(p.final_state) + st_off;
#pragma unroll
    for (int c = 0; c < KD; c += 2) *reinterpret_cast<uint32_t*>(dst + c) = pack_bf16x2(S[c], S[c + 1]);
  }
}

}  // namespace

hipError_t launch_recurrent(const FwdParams& p, const int64_t* cu_seqlens, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.map.nseq * p.H;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_recurrent_kernel, dim3((unsigned)blocks), dim3(128), 0, stream, p, cu_seqlens);
  return hipGetLastError();
}

}  // namespace kda
