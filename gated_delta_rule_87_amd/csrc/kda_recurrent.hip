// kda_recurrent.hip -- token-by-token KDA forward (gfx950).
//
// One workgroup of 4 waves per (sequence, head); wave w owns state rows (value
// index) 32w..32w+31 and keeps them in fp32 registers for the whole sequence.
// The state is laid out so that every load and store instruction of a wave moves
// 1 KiB of contiguous memory: in instruction i, lanes 0-31 hold row 32w + 2i and
// lanes 32-63 row 32w + 2i + 1, each lane four channels 4p..4p+3 (p = lane & 31).
// Every token, for each row v with decays alpha = exp(g~):
//     s      = S[v] . Diag(alpha)
//     u[v]   = beta (s . k^ - v_t[v])
//     o[v]   = scale (s . q^ - u[v] (k^ . q^))         (= scale S'[v] . q^)
//     S'[v]  = s - u[v] k^
// The two row dot products are partial sums over each lane's channels, reduced with
// a reduce-scatter over the 32 lanes of a row pair (cross-row lane swap, then DPP
// mirrors and quad permutations): afterwards lanes 2m and 2m+1 of each half hold the
// totals of one row. u is passed back to the row's lanes through 128 bytes of LDS
// per wave. Waves never wait for each other.
//
// Used for online generation with state passing (page "FlashKDA：面向SM90+的高性能
// KDA CUDA内核库", Q2 on stateful/streaming use), where T per call is small, and as an
// independent long-input reference for the chunked path.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

__device__ __forceinline__ float decay(float g, float dt, float rate, float lb, bool fuse_gate, bool unbounded) {
  if (fuse_gate)
    return unbounded ? fast_exp2(-rate * softplus_log2((g + dt) * LOG2E)) : expf(lb / (1.0f + expf(-rate * (g + dt))));
  return expf(unbounded ? fminf(g, 0.0f) : fminf(fmaxf(g, lb), 0.0f));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_REV = 0x1B;    // quad_perm [3,2,1,0]: lane ^ 3
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1

// sum over the 32 lanes of each half-wave
__device__ __forceinline__ float half_sum(float x) {
  x += dpp<DPP_QUAD_XOR1>(x);
  x += dpp<DPP_QUAD_REV>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  x += dpp<DPP_ROW_MIRROR>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Reduce-scatter over the 32 lanes of each half-wave: v[i] are partial sums of 16
// quantities; lane p ends with the total of quantity p >> 1 (lanes p and p ^ 1 agree).
// Each step pairs lanes that differ in one more bit of p, keeps the half of the values
// selected by that bit and adds the partner's copy of it.
__device__ __forceinline__ float reduce_scatter32(const float* v, int p) {
  float t[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {   // lane ^ 16 (row swap): even rows keep 0..7, odd rows 8..15
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[m]), __float_as_uint(v[8 + m]), false, false);
    t[m] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  const bool b3 = (p & 8) != 0, b2 = (p & 4) != 0, b1 = (p & 2) != 0;
  float r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // lane ^ 15 (mirror): keep by bit 3
    const float keep = b3 ? t[4 + j] : t[j], send = b3 ? t[j] : t[4 + j];
    r[j] = keep + dpp<DPP_ROW_MIRROR>(send);
  }
  float s[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {   // lane ^ 7 (half mirror): keep by bit 2
    const float keep = b2 ? r[2 + j] : r[j], send = b2 ? r[j] : r[2 + j];
    s[j] = keep + dpp<DPP_ROW_HALF_MIRROR>(send);
  }
  const float keep = b1 ? s[1] : s[0], send = b1 ? s[0] : s[1];
  const float x = keep + dpp<DPP_QUAD_REV>(send);   // lane ^ 3: keep by bit 1
  return x + dpp<DPP_QUAD_XOR1>(x);                 // lane ^ 1: same quantity
}

__device__ __forceinline__ f32x4 unpack4_bf16(u32x2 w) {
  return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
}

__global__ __launch_bounds__(256) void kda_recurrent_kernel(FwdParams p, const int64_t* cu) {
  __shared__ f32x4 su[4][2][4];   // [wave][half][i/4]: u of row 32w + 2i + half
  const int H = p.H;
  const int n = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, half = lane >> 5, pl = lane & 31;
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

  // S[i]: row 32w + 2i + half, channels 4pl..4pl+3
  f32x4 S[16];
  const size_t st_off = ((size_t)(n * H + h) * VD + 32 * w + half) * KD + 4 * pl;   // + 2i rows
  if (p.init_dtype == 2) {
    const float* src = static_cast<const float*>(p.init_state) + st_off;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = *reinterpret_cast<const f32x4*>(src + (size_t)2 * i * KD);
  } else if (p.init_dtype == 1) {
    const uint16_t* src = static_cast<const uint16_t*>(p.init_state) + st_off;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = unpack4_bf16(*reinterpret_cast<const u32x2*>(src + (size_t)2 * i * KD));
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const bool fuse_gate = (p.flags & FUSE_GATE) != 0, fuse_norm = (p.flags & FUSE_QK_L2NORM) != 0;
  const bool fuse_beta = (p.flags & FUSE_BETA_SIGMOID) != 0, unbounded = (p.flags & GATE_UNBOUNDED) != 0;
  const float rate = fuse_gate ? expf(p.A_log[h]) : 0.0f;
  const float lb = p.lower_bound, scale = p.scale;
  const f32x4 dt = fuse_gate ? *reinterpret_cast<const f32x4*>(p.dt_bias + (size_t)h * KD + 4 * pl)
                             : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int vrow = 32 * w + 2 * (pl >> 1) + half;   // the row whose totals this lane ends with

  // inputs of token t, loaded one token ahead
  u32x2 qn, kn, gn;
  float bn = 0.0f, vn = 0.0f;
  auto load_token = [&](int64_t t) {
    const size_t row = ((size_t)t * H + h) * KD + 4 * pl;
    qn = *reinterpret_cast<const u32x2*>(p.q + row);
    kn = *reinterpret_cast<const u32x2*>(p.k + row);
    gn = *reinterpret_cast<const u32x2*>(p.g + row);
    bn = bf16_to_f32(p.beta[(size_t)t * H + h]);
    vn = bf16_to_f32(p.v[((size_t)t * H + h) * VD + vrow]);
  };
  if (tb < te) load_token(tb);
  for (int64_t t = tb; t < te; ++t) {
    const f32x4 qf = unpack4_bf16(qn), kf = unpack4_bf16(kn), gf = unpack4_bf16(gn);
    const float braw = bn, vv = vn;
    if (t + 1 < te) load_token(t + 1);

    const float ssq = half_sum(qf.x * qf.x + qf.y * qf.y + qf.z * qf.z + qf.w * qf.w);
    const float ssk = half_sum(kf.x * kf.x + kf.y * kf.y + kf.z * kf.z + kf.w * kf.w);
    const float rq = fuse_norm ? rsqrtf(ssq + 1e-6f) : 1.0f, rk = fuse_norm ? rsqrtf(ssk + 1e-6f) : 1.0f;
    const f32x4 qh = qf * rq, kh = kf * rk;
    const f32x4 al = {decay(gf.x, dt.x, rate, lb, fuse_gate, unbounded), decay(gf.y, dt.y, rate, lb, fuse_gate, unbounded),
                      decay(gf.z, dt.z, rate, lb, fuse_gate, unbounded), decay(gf.w, dt.w, rate, lb, fuse_gate, unbounded)};
    const float beta = fuse_beta ? 1.0f / (1.0f + expf(-braw)) : braw;
    const float kq = half_sum(kh.x * qh.x + kh.y * qh.y + kh.z * qh.z + kh.w * qh.w);

    float dk[16], dq[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] *= al;
      dk[i] = S[i].x * kh.x + S[i].y * kh.y + S[i].z * kh.z + S[i].w * kh.w;
      dq[i] = S[i].x * qh.x + S[i].y * qh.y + S[i].z * qh.z + S[i].w * qh.w;
    }
    const float sk = reduce_scatter32(dk, pl), sq = reduce_scatter32(dq, pl);
    const float u = beta * (sk - vv);
    if ((pl & 1) == 0) {
      p.out[((size_t)t * H + h) * VD + vrow] = to_bf16(scale * (sq - u * kq));
      reinterpret_cast<float*>(&su[w][half][0])[pl >> 1] = u;
    }
    // LDS accesses of one wave complete in order: the reads below see this wave's writes
    f32x4 uu[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) uu[j] = su[w][half][j];
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] -= uu[i >> 2][i & 3] * kh;
  }

  if (p.final_dtype == 2) {
    float* dst = static_cast<float*>(p.final_state) + st_off;
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<f32x4*>(dst + (size_t)2 * i * KD) = S[i];
  } else if (p.final_dtype == 1) {
    uint16_t* dst = static_cast<uint16_t*>(p.final_state) + st_off;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<u32x2*>(dst + (size_t)2 * i * KD) = u32x2{pack_bf16x2(S[i].x, S[i].y), pack_bf16x2(S[i].z, S[i].w)};
  }
}

}  // namespace

hipError_t launch_recurrent(const FwdParams& p, const int64_t* cu_seqlens, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.map.nseq * p.H;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_recurrent_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, cu_seqlens);
  return hipGetLastError();
}

}  // namespace kda
