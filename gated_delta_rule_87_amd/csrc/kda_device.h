// kda_device.h -- device-side building blocks shared by the gfx950 KDA kernels:
// vector types, MFMA wrappers, bf16/fp16 packing, DPP scans, wave reductions,
// and the workspace layout of the per-chunk intermediates.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_{bf16,f16}, wave64):
//   A operand: lane l holds row (l & 15) and 8 contraction indices chosen by
//              the lane group (l >> 4);
//   B operand: lane l holds column (l & 15) and the same 8 contraction indices
//              for lane group (l >> 4);
//   D (4 fp32): lane l holds D[4*(l >> 4) + j][l & 15], j = 0..3.
// Because A and B use the same lane-group -> contraction-index assignment, any
// fixed permutation of the contraction index is allowed. The kernels use the
// "D-compatible" order: within a 32-wide contraction step s, lane group gq
// holds indices 32s + {4gq..4gq+3} (e = 0..3) and 32s + 16 + {4gq..4gq+3}
// (e = 4..7). With that order the D registers of two vertically adjacent 16x16
// tiles are exactly an operand fragment of a following product, so chains of
// products need no transposes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int KD = 128;      // key dim K (fixed)
constexpr int VD = 128;      // value dim V (fixed)
constexpr int CH = 64;       // chunk length
constexpr int SUB = 16;      // sub-chunk length (one wave's rows in the intra kernel)

// ---- per-chunk-head intermediate record written by the intra kernel -------
// All fragments are 64 lanes x 16 bytes = 1 KiB, stored in lane order.
constexpr int FRAG = 1024;
constexpr int OFF_WNEG = 0;                       // f16  [4 tok-tile][4 k-step]  : -W
constexpr int OFF_QG = OFF_WNEG + 16 * FRAG;      // f16  [4 tok-tile][4 k-step]  : Q^.Gamma
constexpr int OFF_KP = OFF_QG + 16 * FRAG;        // f16  [8 chan-tile][2 k-step] : K'^T
constexpr int OFF_AQK = OFF_KP + 16 * FRAG;       // f16  [4 tok-tile][2 k-step]  : Aqk
constexpr int OFF_UT = OFF_AQK + 8 * FRAG;        // f16  [8 v-tile][4 tok-tile][64][4] : U~ * scale
constexpr int OFF_USC = OFF_UT + 16 * FRAG;       // f32  [8 v-tile][4 tok-tile][16]    : 1 / scale
constexpr int OFF_GAML = OFF_USC + 2048;          // f32  [128] : exp(G_L)
constexpr int REC_BYTES = OFF_GAML + 512;         // 76288 bytes per chunk and head

// ---- small helpers ---------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round-to-nearest-even fp32 pair -> packed bf16 (one v_cvt_pk_bf16_f32 on gfx950;
// converting the two scalars separately costs two conversions, a shift and an or)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint16_t to_bf16(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }
// round-to-nearest-even fp32 pair -> packed fp16 (one v_cvt_pk_f16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ uint16_t to_f16(float a) { return __builtin_bit_cast(uint16_t, (_Float16)a); }
// packed fp16 pair -> two fp32. The argument is a plain scalar on purpose: clang
// bit-casts an ext-vector element (v.y) from the vector's base address, so
// callers must never pass such an element straight to __builtin_bit_cast.
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t u) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations are
// complete, then s_barrier. Unlike __syncthreads() it does not wait for global
// loads or stores in flight (a release fence would add s_waitcnt vmcnt(0)). The
// asm is also a compiler memory barrier, so no memory access moves across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 u) { return __builtin_bit_cast(f16x8, u); }

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf_fast(float x) { return fast_rcp(1.0f + fast_exp(-x)); }
// 2^x in one v_exp_f32 (callers keep their exponents in log2 units)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;
// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Inclusive prefix sum across the 16 lanes of each DPP row (lane & 15 is the
// position in the row). Row-shift DPP with bound_ctrl yields 0 past the row
// start, so lanes with fewer predecessors add zeros.
__device__ __forceinline__ float row16_inclusive_scan(float v) {
  float s = v;
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x111, 0xf, 0xf, true));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x112, 0xf, 0xf, true));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x114, 0xf, 0xf, true));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x118, 0xf, 0xf, true));
  return s;
}

// max over the four lanes {l, l^16, l^32, l^48} (the lane groups sharing l & 15),
// with the gfx950 cross-half lane swaps (no LDS round trip)
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// log2(1 + 2^y): softplus(y ln 2) in log2 units, without overflow for large y
__device__ __forceinline__ float softplus_log2(float y) {
  return fmaxf(y, 0.0f) + __builtin_amdgcn_logf(1.0f + fast_exp2(-fabsf(y)));
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Power-of-two scale s and its inverse such that max|x| * s lies in [1, 2).
// The exponent is clamped so that both stay normal fp32 numbers; max|x| = 0
// gives an arbitrary (harmless) scale because every scaled value is then 0.
__device__ __forceinline__ void pow2_scale(float m, float& s, float& inv) {
  int e = (int)((__float_as_uint(m) >> 23) & 0xff);   // biased exponent
  e = e < 27 ? 27 : (e > 227 ? 227 : e);
  s = __uint_as_float((uint32_t)(254 - e) << 23);
  inv = __uint_as_float((uint32_t)e << 23);
}

}  // namespace kda
