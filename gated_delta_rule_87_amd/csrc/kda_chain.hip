// kda_chain.hip -- inter-chunk state chain + output of the chunked KDA forward
// (gfx950).
//
// One workgroup per (sequence, head, group of NW*VT*16 value columns); wave w
// owns VT 16-wide value tiles. Rows v of the state only ever meet column v of
// V and U, so value slices are independent chains. Each wave keeps its slice
// of the fp32 state in registers for the whole sequence and walks the chunks
// in order; per chunk (records written by the intra kernel):
//     U      = U~ - W S0^T
//     O^T    = scale (S0 (Q^.Gamma)^T + U^T Aqk^T)     -> out (bf16), every row t < L
//     S1^T   = Diag(Gamma_L) S0^T + K'^T U
// and the state goes to final_state after the last chunk. This is the
// recurrent "state passing" half of the forward; initial_state/final_state
// follow the "Kernel API" table of the FlashKDA README digest ([B|N,H,V,K],
// bf16 or fp32, dtypes equal when both are given) and out is written once in
// place (2kiu.com guide, section 二).
//
// Memory pipeline: everything a chunk step reads -- the 56 fragments shared by
// all value tiles (-W, Qg, K'^T, Aqk: 56 KiB, contiguous at the start of the
// record), each wave's U~ tiles and scales, and Gamma_L -- is copied one chunk ahead
// into a two-deep LDS ring with direct global->LDS loads (no VGPR staging).
// Waits are explicit vmcnt counts with bare s_barrier, so the prefetch of chunk
// j+1 stays in flight while chunk j computes.
//
// Precision: MFMA operands are fp16. Each state row and each column of U is
// scaled by its own power of two (max |x| * s in [1, 2)) before rounding, so
// fp16's range is never exceeded and the scaling is exact; accumulation is
// fp32.
#include "kda_device.h"
#include "kda_internal.h"

#ifndef KDA_CHAIN_NW
#define KDA_CHAIN_NW 2
#endif
#ifndef KDA_CHAIN_VT
#define KDA_CHAIN_VT 1
#endif

namespace kda {
namespace {

constexpr int NSHARED = 56;   // fragments per chunk shared by all value tiles

#define LDSPTR(p) ((__attribute__((address_space(3))) void*)(p))

// buffer resource word 3 for raw (stride 0) dword-granular loads on gfx9-family parts
constexpr int RSRC_WORD3 = 0x00020000;

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// max |x| over one state row / U column: this lane's registers, then the four
// lane groups that hold the other channels (tokens) of the same row (column)
__device__ __forceinline__ float row_absmax(const f32x4* x, int n) {
  float m = 0.0f;
  for (int i = 0; i < n; ++i) m = fmaxf(m, fmaxf(fmaxf(fabsf(x[i].x), fabsf(x[i].y)), fmaxf(fabsf(x[i].z), fabsf(x[i].w))));
  return max_over_groups(m);
}

// the same pointer in every lane, made explicit so it lives in SGPRs
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ u32x4 pack_pair_f16(f32x4 a, f32x4 b, float s) {
  a *= s;
  b *= s;
  return u32x4{pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y), pack_f16x2(b.z, b.w)};
}

template <int NW, int VT>
struct ChainSmem {
  u32x4 shared[NSHARED][64];     // -W, Qg, K'^T, Aqk fragments of the chunk (all value tiles)
  u32x2 ut[NW][VT][4][64];       // U~ (fp16, scaled) of each wave's value tiles [token tile][lane]
  float usc[NW][VT][4][16];      // 1 / scale per (token tile, value column)
  float gam[NW][KD];             // Gamma_L (one copy per wave: every wave loads its own)
};

template <int NW, int VT>
__global__ __launch_bounds__(NW * 64) void kda_chain_kernel(FwdParams p, int nvg) {
  __shared__ ChainSmem<NW, VT> ring[2];

  const int H = p.H;
  const int NH = p.map.nseq * H;
  // workgroups of one (sequence, head) share blockIdx % 8, i.e. one XCD and its L2
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vg = rest % nvg, grp = rest / nvg;
  const int nh = grp * 8 + xcd;
  if (nh >= NH) return;   // uniform over the block
  const int n = nh / H, h = nh - n * H;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  const int l = threadIdx.x & 63, lt = l & 15, gq = l >> 4;
  const int vt0 = (vg * NW + w) * VT;   // first 16-wide value tile of this wave

  int c0, nc, tok0, len;
  if (p.map.seq_tab) {
    const int2 e = p.map.seq_tab[n];
    const int2 sp = p.map.seq_span[n];
    c0 = __builtin_amdgcn_readfirstlane(e.x);
    nc = __builtin_amdgcn_readfirstlane(e.y);
    tok0 = __builtin_amdgcn_readfirstlane(sp.x);
    len = __builtin_amdgcn_readfirstlane(sp.y);
  } else {
    c0 = n * p.map.nc_row;
    nc = p.map.nc_row;
    tok0 = n * p.map.T;
    len = p.map.T;
  }

  // state slices, D layout of S^T: S[t][mt][j] = S[16(vt0+t) + lt][16mt + 4gq + j]
  f32x4 S[VT][8];
#pragma unroll
  for (int t = 0; t < VT; ++t) {
    const size_t st_off = ((size_t)(n * H + h) * VD + 16 * (vt0 + t) + lt) * KD;
    if (p.init_dtype == 2) {
      const float* src = static_cast<const float*>(p.init_state) + st_off;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[t][mt] = *reinterpret_cast<const f32x4*>(src + 16 * mt + 4 * gq);
    } else if (p.init_dtype == 1) {
      const uint16_t* src = static_cast<const uint16_t*>(p.init_state) + st_off;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const u32x2 r = *reinterpret_cast<const u32x2*>(src + 16 * mt + 4 * gq);
        S[t][mt] = f32x4{bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y)};
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[t][mt] = f32x4{0, 0, 0, 0};
    }
  }
  wait_vmcnt<0>();   // the loop below then carries no pending register loads

  const int lane16 = l * 16;   // this lane's 16 bytes of a 1 KiB fragment (VGPR offset of every load)
  // one prefetch = NSHARED/NW shared fragments + 2*VT U~ halves + VT scale rows + Gamma_L, all
  // straight into LDS with buffer loads: a scalar resource per record, the lane offset in one
  // VGPR and the in-record offset in an SGPR, so no per-load vector address arithmetic. The
  // resource spans exactly one record, which the hardware range-checks.
  auto prefetch = [&](int j, int buf) {
    const uint8_t* rec = uniform_ptr(p.rec + ((size_t)(c0 + j) * H + h) * REC_BYTES);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, REC_BYTES, RSRC_WORD3);
#pragma unroll
    for (int i = 0; i < NSHARED / NW; ++i) {
      const int f = i * NW + w;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&ring[buf].shared[f][0]), 16, lane16, f * FRAG, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&ring[buf].ut[w][t][2 * hh][0]), 16, lane16,
                                                 OFF_UT + (vt0 + t) * 2048 + hh * FRAG, 0, 0);
      if (l < 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&ring[buf].usc[w][t][0][0]), 16, lane16,
                                                 OFF_USC + (vt0 + t) * 256, 0, 0);
    }
    if (l < 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&ring[buf].gam[w][0]), 16, lane16, OFF_GAML, 0, 0);
  };
  constexpr int KPF = NSHARED / NW + 3 * VT + 1;   // vector-memory ops issued per prefetch

  if (nc > 0) prefetch(0, 0);
  const float scale = p.scale;
  for (int j = 0; j < nc; ++j) {
    const int b = j & 1;
    __builtin_amdgcn_s_barrier();            // everyone is done with the buffer we refill next
    if (j + 1 < nc) {
      prefetch(j + 1, b ^ 1);
      wait_vmcnt<KPF>();                       // chunk j's loads (issued earlier) have landed
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();            // ... for every wave of the block
    const ChainSmem<NW, VT>& R = ring[b];
    const int t0 = tok0 + j * CH;
    const int L = min(CH, len - j * CH);

    // state -> fp16 operand fragments (k-step s: channel tiles 2s, 2s+1), each state
    // row v scaled by its own power of two
    float sS[VT], iS[VT];
    u32x4 sf[VT][4];
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      pow2_scale(row_absmax(S[t], 8), sS[t], iS[t]);
#pragma unroll
      for (int s = 0; s < 4; ++s) sf[t][s] = pack_pair_f16(S[t][2 * s], S[t][2 * s + 1], sS[t]);
    }

    // U = U~ + (-W) S0^T     D layout: lane <-> v, registers <-> tokens 16mt + 4gq + j
    f32x4 U[VT][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc[VT];
#pragma unroll
      for (int t = 0; t < VT; ++t) acc[t] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = R.shared[mt * 4 + s][l];
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[t] = mfma_f16(a, sf[t][s], acc[t]);
      }
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const u32x2 uh = R.ut[w][t][mt][l];
        const f32x2 u01 = unpack_f16x2(uh.x), u23 = unpack_f16x2(uh.y);
        U[t][mt] = f32x4{u01.x, u01.y, u23.x, u23.y} * R.usc[w][t][mt][lt] + acc[t] * iS[t];
      }
    }
    float sU[VT], iU[VT];
    u32x4 uf[VT][2];
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      pow2_scale(row_absmax(U[t], 4), sU[t], iU[t]);
#pragma unroll
      for (int s = 0; s < 2; ++s) uf[t][s] = pack_pair_f16(U[t][2 * s], U[t][2 * s + 1], sU[t]);
    }

    // O^T = scale (S0 Qg^T + U^T Aqk^T)   D layout: lane <-> token 16nt + lt, registers <-> v.
    // Register j of lane group gq belongs to value row 4gq + j, whose scales live in lane 4gq + j.
    f32x4 oS[VT], oU[VT];
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        oS[t][jj] = __shfl(iS[t], 4 * gq + jj, 64) * scale;
        oU[t][jj] = __shfl(iU[t], 4 * gq + jj, 64) * scale;
      }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 aq[VT], aa[VT];
#pragma unroll
      for (int t = 0; t < VT; ++t) aq[t] = aa[t] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 qv = R.shared[16 + nt * 4 + s][l];
#pragma unroll
        for (int t = 0; t < VT; ++t) aq[t] = mfma_f16(sf[t][s], qv, aq[t]);
      }
      {
        const u32x4 a0 = R.shared[48 + nt * 2][l];
#pragma unroll
        for (int t = 0; t < VT; ++t) aa[t] = mfma_f16(uf[t][0], a0, aa[t]);
      }
      if (nt >= 2) {
        const u32x4 a1 = R.shared[48 + nt * 2 + 1][l];
#pragma unroll
        for (int t = 0; t < VT; ++t) aa[t] = mfma_f16(uf[t][1], a1, aa[t]);
      }
      const int tok = 16 * nt + lt;
      if (tok < L) {
        uint16_t* dst = p.out + ((size_t)(t0 + tok) * H + h) * VD + 4 * gq;
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const f32x4 o = aq[t] * oS[t] + aa[t] * oU[t];
          *reinterpret_cast<u32x2*>(dst + 16 * (vt0 + t)) = u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
        }
      }
    }

    // S1^T = Diag(Gamma_L) S0^T + K'^T U
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const u32x4 k0 = R.shared[32 + mt * 2][l], k1 = R.shared[32 + mt * 2 + 1][l];
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(&R.gam[w][16 * mt + 4 * gq]);
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        f32x4 acc = {0, 0, 0, 0};
        acc = mfma_f16(k0, uf[t][0], acc);
        acc = mfma_f16(k1, uf[t][1], acc);
        S[t][mt] = S[t][mt] * g4 + acc * iU[t];
      }
    }
  }

#pragma unroll
  for (int t = 0; t < VT; ++t) {
    const size_t st_off = ((size_t)(n * H + h) * VD + 16 * (vt0 + t) + lt) * KD;
    if (p.final_dtype == 2) {
      float* dst = static_cast<float*>(p.final_state) + st_off;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt + 4 * gq) = S[t][mt];
    } else if (p.final_dtype == 1) {
      uint16_t* dst = static_cast<uint16_t*>(p.final_state) + st_off;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        *reinterpret_cast<u32x2*>(dst + 16 * mt + 4 * gq) =
            u32x2{pack_bf16x2(S[t][mt].x, S[t][mt].y), pack_bf16x2(S[t][mt].z, S[t][mt].w)};
    }
  }
}

static_assert(NSHARED % KDA_CHAIN_NW == 0, "shared fragments must split evenly over the waves");
static_assert(VD % (16 * KDA_CHAIN_NW * KDA_CHAIN_VT) == 0, "value tiles must split evenly");
static_assert(OFF_QG == 16 * FRAG && OFF_KP == 32 * FRAG && OFF_AQK == 48 * FRAG,
              "shared fragments must be contiguous at the record start");

}  // namespace

hipError_t launch_chain(const FwdParams& p, hipStream_t stream) {
  const int NH = p.map.nseq * p.H;
  if (NH <= 0) return hipSuccess;
  constexpr int NW = KDA_CHAIN_NW, VT = KDA_CHAIN_VT;
  const int nvg = VD / (16 * NW * VT);
  const int64_t blocks = (int64_t)((NH + 7) / 8) * 8 * nvg;
  hipLaunchKernelGGL((kda_chain_kernel<NW, VT>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p, nvg);
  return hipGetLastError();
}

}  // namespace kda
