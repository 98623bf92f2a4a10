// kda_chain.hip -- inter-chunk state chain + output of the chunked KDA forward
// (gfx950).
//
// One wave per (sequence, head, 16-wide value slice); a workgroup holds NW such
// waves. Rows v of the state only ever meet column v of V and U, so value
// slices are independent chains. Each wave keeps its 16 x 128 slice of the
// fp32 state in registers for the whole sequence and walks the chunks in
// order; per chunk (records written by the intra kernel):
//     U      = U~ - W S0^T                            (16x128 . 128x16 per tile)
//     O^T    = scale (S0 (Q^.Gamma)^T + U^T Aqk^T)     -> out (bf16), every row t < L
//     S1^T   = Diag(Gamma_L) S0^T + K'^T U
// with the state written to final_state after the last chunk. This is the
// recurrent "state passing" half of the forward; initial_state/final_state
// follow the "Kernel API" table of the FlashKDA README digest ([B|N,H,V,K],
// bf16 or fp32, dtypes equal when both are given) and out is written once in
// place (2kiu.com guide, section 二).
//
// Precision: MFMA operands are fp16. The state and U are scaled per 16-wide
// slice by a power of two (max |x| * s in [1, 2)) before rounding, so fp16's
// range is never exceeded and the scale is exact; accumulation is fp32.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int NW>
__global__ __launch_bounds__(NW * 64) void kda_chain_kernel(FwdParams p, int nvg) {
  const int H = p.H;
  const int NH = p.map.nseq * H;
  // blocks of the same (sequence, head) share blockIdx % 8, i.e. one XCD and its L2
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vg = rest % nvg, grp = rest / nvg;
  const int nh = grp * 8 + xcd;
  if (nh >= NH) return;
  const int n = nh / H, h = nh - n * H;

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lt = l & 15, gq = l >> 4;
  const int vt = vg * NW + w;          // 16-wide value tile
  const int v = 16 * vt + lt;          // this lane's state row

  int c0, nc;
  if (p.map.seq_tab) {
    const int2 e = p.map.seq_tab[n];
    c0 = e.x;
    nc = e.y;
  } else {
    c0 = n * p.map.nc_row;
    nc = p.map.nc_row;
  }

  // state slice, D layout of S^T: S[mt][j] = S[v][16mt + 4gq + j]
  f32x4 S[8];
  const size_t st_off = ((size_t)(n * H + h) * VD + v) * KD;
  if (p.init_dtype == 2) {
    const float* src = static_cast<const float*>(p.init_state) + st_off;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = *reinterpret_cast<const f32x4*>(src + 16 * mt + 4 * gq);
  } else if (p.init_dtype == 1) {
    const uint16_t* src = static_cast<const uint16_t*>(p.init_state) + st_off;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const u32x2 r = *reinterpret_cast<const u32x2*>(src + 16 * mt + 4 * gq);
      S[mt] = f32x4{bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y)};
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = f32x4{0, 0, 0, 0};
  }

  const float scale = p.scale;
  for (int j = 0; j < nc; ++j) {
    const int ci = c0 + j;
    int t0, L;
    if (p.map.chunk_tab) {
      const int2 e = p.map.chunk_tab[ci];
      t0 = e.x;
      L = e.y;
    } else {
      t0 = n * p.map.T + j * CH;
      L = min(CH, p.map.T - j * CH);
    }
    const uint8_t* rec = p.rec + ((size_t)ci * H + h) * REC_BYTES;
    auto frag = [&](int off, int f) { return *reinterpret_cast<const u32x4*>(rec + off + (f * 64 + l) * 16); };

    // scale the state slice into fp16 operand fragments (k-step s: channel tiles 2s, 2s+1)
    float m = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(S[mt].x), fabsf(S[mt].y)), fmaxf(fabsf(S[mt].z), fabsf(S[mt].w))));
    m = wave_max(m);
    float sS, iS;
    pow2_scale(m, sS, iS);
    u32x4 sf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 a = S[2 * s] * sS, b = S[2 * s + 1] * sS;
      sf[s] = u32x4{pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y), pack_f16x2(b.z, b.w)};
    }

    // U = U~ + (-W) S0^T       D layout: lane <-> v, registers <-> tokens 16mt + 4gq + j
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma_f16(frag(OFF_WNEG, mt * 4 + s), sf[s], acc);
      const f32x4 ut = *reinterpret_cast<const f32x4*>(rec + OFF_UT + ((vt * 4 + mt) * 64 + l) * 16);
      U[mt] = ut + acc * iS;
    }
    float mu = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      mu = fmaxf(mu, fmaxf(fmaxf(fabsf(U[mt].x), fabsf(U[mt].y)), fmaxf(fabsf(U[mt].z), fabsf(U[mt].w))));
    mu = wave_max(mu);
    float sU, iU;
    pow2_scale(mu, sU, iU);
    u32x4 uf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 a = U[2 * s] * sU, b = U[2 * s + 1] * sU;
      uf[s] = u32x4{pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y), pack_f16x2(b.z, b.w)};
    }

    // O^T = scale (S0 Qg^T + U^T Aqk^T)   D layout: lane <-> token 16nt + lt, registers <-> v
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 aq = {0, 0, 0, 0}, aa = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) aq = mfma_f16(sf[s], frag(OFF_QG, nt * 4 + s), aq);
      aa = mfma_f16(uf[0], frag(OFF_AQK, nt * 2), aa);
      if (nt >= 2) aa = mfma_f16(uf[1], frag(OFF_AQK, nt * 2 + 1), aa);
      const f32x4 o = (aq * iS + aa * iU) * scale;
      const int t = 16 * nt + lt;
      if (t < L) {
        uint16_t* dst = p.out + ((size_t)(t0 + t) * H + h) * VD + 16 * vt + 4 * gq;
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
      }
    }

    // S1^T = Diag(Gamma_L) S0^T + K'^T U
    const float* gam = reinterpret_cast<const float*>(rec + OFF_GAML);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 acc = {0, 0, 0, 0};
      acc = mfma_f16(frag(OFF_KP, mt * 2), uf[0], acc);
      acc = mfma_f16(frag(OFF_KP, mt * 2 + 1), uf[1], acc);
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(gam + 16 * mt + 4 * gq);
      S[mt] = S[mt] * g4 + acc * iU;
    }
  }

  if (p.final_dtype == 2) {
    float* dst = static_cast<float*>(p.final_state) + st_off;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt + 4 * gq) = S[mt];
  } else if (p.final_dtype == 1) {
    uint16_t* dst = static_cast<uint16_t*>(p.final_state) + st_off;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      *reinterpret_cast<u32x2*>(dst + 16 * mt + 4 * gq) =
          u32x2{pack_bf16x2(S[mt].x, S[mt].y), pack_bf16x2(S[mt].z, S[mt].w)};
  }
}

constexpr int CHAIN_NW = 4;   // waves per workgroup (64 value columns)

}  // namespace

hipError_t launch_chain(const FwdParams& p, hipStream_t stream) {
  const int NH = p.map.nseq * p.H;
  if (NH <= 0) return hipSuccess;
  const int nvg = VD / (16 * CHAIN_NW);
  const int64_t blocks = (int64_t)((NH + 7) / 8) * 8 * nvg;
  hipLaunchKernelGGL(kda_chain_kernel<CHAIN_NW>, dim3((unsigned)blocks), dim3(CHAIN_NW * 64), 0, stream, p, nvg);
  return hipGetLastError();
}

}  // namespace kda
