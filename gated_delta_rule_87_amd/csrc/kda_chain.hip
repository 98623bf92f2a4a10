// kda_chain.hip -- inter-chunk state chain + output of the chunked KDA forward
// (gfx950).
//
// One workgroup per (sequence, head, group of NW 16-wide value tiles). Rows v
// of the state only ever meet column v of V and U, so value slices are
// independent chains. Per chunk (records written by the intra kernel):
//     U      = U~ - W S0^T
//     O^T    = scale (S0 (Q^.Gamma)^T + U^T Aqk^T)     -> out (bf16), every row t < L
//     S1^T   = Diag(Gamma_L) S0^T + K'^T U
// and the state goes to final_state after the last chunk. This is the
// recurrent "state passing" half of the forward; initial_state/final_state
// follow the "Kernel API" table of the FlashKDA README digest ([B|N,H,V,K],
// bf16 or fp32, dtypes equal when both are given) and out is written once in
// place (2kiu.com guide, section 二).
//
// Wave roles (3 NW + 1 waves):
//   state waves 2s, 2s + 1  keep the two channel halves of value tile s's fp32
//                           state in registers; per chunk each forms half of U
//                           (one token half, over all channels) and updates its
//                           own channel half (from both token halves of U); each
//                           publishes its fp16 operands (its half of S0 and of
//                           U, scaled by powers of two) in LDS for the partner
//                           and the output wave
//   output wave 2 NW + s    computes O^T of value tile s from those operands and
//                           the chunk's Q^.Gamma and Aqk, stores out
//   DMA wave 3 NW           streams the records into LDS with buffer loads, 1.5
//                           chunk steps ahead of their use
// Two workgroup barriers per chunk: (A) the first part of chunk j's record and
// S0's operands are in LDS; (B) the second part and U's operands are in LDS.
// The state update runs while the output waves finish O, so neither the loads
// nor the output sit on the state recurrence's critical path; splitting each
// tile's state over two waves halves the MFMA chain and the rescaling on it.
//
// Precision: MFMA operands are fp16. Each state row and each column of U is
// scaled by its own power of two (max |x| * s in [1, 2)) before rounding, so
// fp16's range is never exceeded and the scaling is exact; accumulation is
// fp32.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

#define LDSPTR(p) ((__attribute__((address_space(3))) void*)(p))

// buffer resource word 3 for raw (stride 0) dword-granular loads on gfx9-family parts
constexpr int RSRC_WORD3 = 0x00020000;

// At most N of this wave's vector-memory operations (the LDS DMA included) are
// still outstanding; they complete in issue order. The counter holds at most 63.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8));
  asm volatile("" ::: "memory");
}

// the same pointer in every lane, made explicit so it lives in SGPRs
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// max |x| over one state row / U column: this lane's registers, then the four
// lane groups that hold the other channels (tokens) of the same row (column)
__device__ __forceinline__ float row_absmax(const f32x4* x, int n) {
  float m = 0.0f;
  for (int i = 0; i < n; ++i) m = fmaxf(m, fmaxf(fmaxf(fabsf(x[i].x), fabsf(x[i].y)), fmaxf(fabsf(x[i].z), fabsf(x[i].w))));
  return max_over_groups(m);
}

__device__ __forceinline__ u32x4 pack_pair_f16(f32x4 a, f32x4 b, float s) {
  a *= s;
  b *= s;
  return u32x4{pack_f16x2(a.x, a.y), pack_f16x2(a.z, a.w), pack_f16x2(b.x, b.y), pack_f16x2(b.z, b.w)};
}

// Every LDS DMA load is issued by all 64 lanes (1 KiB): a lane-dependent branch
// around one would let the optimiser merge call sites and derive M0 (the LDS
// destination, one per wave) from a per-lane value. So the scale rows and
// Gamma_L come in 1 KiB windows of the record that end inside it:
//   usc window  OFF_USC + NW*256*vg   -> the first NW*256 bytes are this group's scales
//   gam window  OFF_GAML - 512        -> Gamma_L is its second half
constexpr int USC_WIN = 1024;
constexpr int GAM_WIN_OFF = OFF_GAML - 512;
static_assert(OFF_USC + 2048 == OFF_GAML && OFF_GAML + 512 == REC_BYTES, "record tail layout");

// A chunk's record is staged in two parts, each in its own two-slot ring: the
// part read between barriers (A) and (B) of a chunk step, and the part read
// between (B) and the next (A). A slot is refilled as soon as its part of the
// step is over, so every load is issued 1.5 chunk steps before it is needed.
template <int NW>
struct ChainPart1 {              // read in [A, B): U and the S0 half of O
  u32x4 wneg[16][64];            // -W fragments [token tile * 4 + k-step][lane]
  u32x4 qg[16][64];              // Q^.Gamma fragments [token tile * 4 + k-step][lane]
  u32x2 ut[NW][4][64];           // U~ (fp16, scaled) of each value tile [token tile][lane]
  float usc[USC_WIN / 4];        // [s][token tile][value column]: 1 / scale (first NW*64 floats)
};
template <int NW>
struct ChainPart2 {              // read in [B, next A): the state update and the U half of O
  u32x4 kp[16][64];              // K'^T fragments [channel tile * 2 + k-step][lane]
  u32x4 aqk[6][64];              // the Aqk fragments that are not all zero (see AQK_FRAG)
  float gamw[256];               // Gamma_L in [128, 256)
};
// Aqk fragment (token tile nt, k-step q) with q <= nt / 2 -> slot in ChainPart2::aqk
__device__ __forceinline__ constexpr int aqk_slot(int nt, int q) { return nt < 2 ? nt : 2 * nt - 2 + q; }
constexpr int AQK_FRAG[6] = {0, 2, 4, 5, 6, 7};   // record fragment index (nt * 2 + q) of each slot

template <int NW>
struct ChainXchg {               // operands of one chunk, shared by a tile's three waves
  u32x4 sf[NW][4][64];           // S0 rows, fp16, scaled: MFMA fragments per k-step (channels 32q..)
  u32x4 uf[NW][2][64];           // U columns, fp16, scaled: MFMA fragments per k-step (tokens 32q..)
  float iS[NW][2][16];           // 1 / row scale of S0, per channel half
  float iU[NW][2][16];           // 1 / column scale of U, per token half
};

template <int NW, int MODE>
__global__ __launch_bounds__((3 * NW + 1) * 64) void kda_chain_kernel(FwdParams p, int nvg) {
  __shared__ ChainPart1<NW> r1[2];
  __shared__ ChainPart2<NW> r2[2];
  __shared__ ChainXchg<NW> xc;
  __shared__ uint32_t touch_lds[64];   // landing window of the L2 touches (never read)

  const int H = p.H;
  constexpr int mode = MODE;   // ChainMode, fixed per instantiation
  // segment modes: "sequence" n' = row * nseg + segment
  const int NH = (mode == CHAIN_FULL ? p.map.nseq : p.map.nseq * p.seg.nseg) * H;
  // workgroups of one (sequence, head) share blockIdx % 8, i.e. one XCD and its L2
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int vg = rest % nvg, grp = rest / nvg;
  const int nh = grp * 8 + xcd;
  if (nh >= NH) return;   // uniform over the block
  // varlen: walk the sequences longest first, so long chains do not start last
  const int rank = nh / H, h = nh - rank * H;
  // varlen window: the rank-th sequence with chunks from the window's first on, if it starts
  // inside the window (uniform over the block)
  const bool vwin = mode == CHAIN_FULL && p.map.win >= 0 && p.map.seq_tab;
  int n;
  if (vwin) {
    const int k = __builtin_amdgcn_readfirstlane(p.map.win_first[p.map.win]) + rank;
    if (k >= __builtin_amdgcn_readfirstlane(p.map.win_first[p.map.n_win])) return;
    n = __builtin_amdgcn_readfirstlane(p.map.nz_seq[k]);
    if (__builtin_amdgcn_readfirstlane(p.map.seq_tab[n].x) >= p.map.jb + p.map.nc_win) return;
  } else {
    n = (mode == CHAIN_FULL && p.map.seq_order) ? __builtin_amdgcn_readfirstlane(p.map.seq_order[rank]) : rank;
  }

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  const int l = threadIdx.x & 63, lt = l & 15, gq = l >> 4;

  int c0, nc, tok0, len;
  bool win_in = false, win_out = false;   // (varlen window) state from / to the carry slots
  if (mode != CHAIN_FULL) {   // one segment of a row (fixed length) or a sequence (varlen)
    const int row = n / p.seg.nseg, sg = n - row * p.seg.nseg;
    int first, count, t0, length;
    if (p.map.seq_tab) {
      const int2 e = p.map.seq_tab[row], sp = p.map.seq_span[row];
      first = __builtin_amdgcn_readfirstlane(e.x);
      count = __builtin_amdgcn_readfirstlane(e.y);
      t0 = __builtin_amdgcn_readfirstlane(sp.x);
      length = __builtin_amdgcn_readfirstlane(sp.y);
    } else {
      first = row * p.map.nc_win;
      count = p.map.nc_win;
      t0 = row * p.map.T + p.map.jb * CH;
      length = p.map.T - p.map.jb * CH;
    }
    const int sc = (count + p.seg.nseg - 1) / p.seg.nseg;   // chunks per segment of this row
    const int cs = sg * sc;
    c0 = first + cs;
    nc = max(0, min(sc, count - cs));
    tok0 = t0 + cs * CH;
    len = max(0, min(sc * CH, length - cs * CH));
  } else if (p.map.seq_tab) {
    const int2 e = p.map.seq_tab[n];
    const int2 sp = p.map.seq_span[n];
    c0 = __builtin_amdgcn_readfirstlane(e.x);
    nc = __builtin_amdgcn_readfirstlane(e.y);
    tok0 = __builtin_amdgcn_readfirstlane(sp.x);
    len = __builtin_amdgcn_readfirstlane(sp.y);
    if (vwin) {   // this window's chunks of the sequence, records indexed from the window's first slot
      const int a = max(c0, p.map.jb), b = min(c0 + nc, p.map.jb + p.map.nc_win);
      tok0 += (a - c0) * CH;
      len -= (a - c0) * CH;
      win_in = a > c0;        // the state comes from the previous window
      win_out = b < c0 + nc;  // and goes on to the next
      c0 = a - p.map.jb;
      nc = b - a;
    }
  } else {
    c0 = n * p.map.nc_win;   // this launch's chunks jb .. jb + nc_win - 1 of row n
    nc = p.map.nc_win;
    tok0 = n * p.map.T + p.map.jb * CH;
    len = p.map.T - p.map.jb * CH;
  }

  if (w == 3 * NW) {
    // ---------------- DMA wave ----------------
    // Straight into LDS with buffer loads: a scalar resource per record (which the
    // hardware range-checks), the lane offset in one VGPR, the in-record offset in an
    // SGPR. Issue order P1(0) P2(0) P1(1) | P2(1) P1(2) | P2(2) P1(3) | ..., and loads
    // complete in issue order, so each wait names how many later loads may still fly.
    const int lane16 = l * 16;
    auto rsrc = [&](int j) {
      const uint8_t* rec = uniform_ptr(p.rec + ((size_t)(c0 + j) * H + h) * REC_BYTES);
      return __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, REC_BYTES, RSRC_WORD3);
    };
    auto load_part1 = [&](int j) {
      const __amdgpu_buffer_rsrc_t rs = rsrc(j);
      ChainPart1<NW>& d = r1[j & 1];
#pragma unroll
      for (int f = 0; f < 16; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.wneg[f][0]), 16, lane16, OFF_WNEG + f * FRAG, 0, 0);
#pragma unroll
      for (int f = 0; f < 16; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.qg[f][0]), 16, lane16, OFF_QG + f * FRAG, 0, 0);
#pragma unroll
      for (int s = 0; s < NW; ++s) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.ut[s][2 * hh][0]), 16, lane16,
                                                   OFF_UT + ((vg * NW + s) & 7) * 2048 + hh * FRAG, 0, 0);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.usc[0]), 16, lane16,
                                               OFF_USC + NW * 256 * (vg % (VD / (16 * NW))), 0, 0);
    };
    auto load_part2 = [&](int j) {
      const __amdgpu_buffer_rsrc_t rs = rsrc(j);
      ChainPart2<NW>& d = r2[j & 1];
#pragma unroll
      for (int f = 0; f < 16; ++f)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.kp[f][0]), 16, lane16, OFF_KP + f * FRAG, 0, 0);
#pragma unroll
      for (int i = 0; i < 6; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.aqk[i][0]), 16, lane16, OFF_AQK + AQK_FRAG[i] * FRAG, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&d.gamw[0]), 16, lane16, GAM_WIN_OFF, 0, 0);
    };
    constexpr int N1 = 32 + 2 * NW + 1, N2 = 16 + 6 + 1;   // loads per part
    // L2 touch of the record TD steps ahead (two value tiles per workgroup, every mode):
    // one dword of every 128-byte line, the nvg workgroups of a head taking every nvg-th
    // line, so each line is requested once per head; lines past the record's end fall
    // outside the resource's range and are dropped. The touches go to a scratch LDS
    // window (no destination register), are issued after the wait that follows each
    // first-part refill and count in the waits after it, which keeps every wait within
    // the 63-load counter (N1 + N2 + TP = 63 for NW = 2).
    constexpr int TP = NW == 2 ? 3 : 0, TD = 3;
    static_assert(TP == 0 || N1 + N2 + TP <= 63, "touches must fit the load counter");
    // nvg is VD / 32 (plain chain, outputs pass) or 2 VD / 32 (maps pass) with NW = 2
    static_assert(TP == 0 || 64 * TP * (VD / 32) * 128 >= REC_BYTES, "touches cover the record");
    auto touch = [&](int j) {
      const __amdgpu_buffer_rsrc_t rs = rsrc(j);
#pragma unroll
      for (int i = 0; i < TP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDSPTR(&touch_lds[0]), 4, (vg + nvg * (64 * i + l)) * 128, 0, 0, 0);
    };
    if (nc > 0) {
      load_part1(0);
      load_part2(0);
      if (nc > 1) {
        load_part1(1);
        wait_vmcnt<N2 + N1>();                     // P1(0) landed
      } else {
        wait_vmcnt<N2>();
      }
    }
    for (int j = 0; j < nc; ++j) {
      lds_barrier();                               // (A): P1(j) landed; P2 slot (j+1)&1 is free
      const bool touched = TP > 0 && j >= 1 && j + TD - 1 < nc;   // T(j+TD-1) was issued in step j-1
      if (j + 1 < nc) {
        load_part2(j + 1);
        if (touched)                               // P2(j) landed (P1(j+1), T(j+TD-1), P2(j+1) may fly)
          wait_vmcnt<N1 + TP + N2>();
        else                                       // P2(j) landed (P1(j+1), P2(j+1) may fly)
          wait_vmcnt<N1 + N2>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();                               // (B): P2(j) landed; P1 slot j&1 is free
      if (j + 2 < nc) {
        load_part1(j + 2);
        if (touched)                               // P1(j+1) landed (T(j+TD-1), P2(j+1), P1(j+2) may fly)
          wait_vmcnt<TP + N2 + N1>();
        else                                       // P1(j+1) landed (P2(j+1), P1(j+2) may fly)
          wait_vmcnt<N2 + N1>();
        if (TP > 0 && j + TD < nc) touch(j + TD);
      } else if (j + 1 < nc) {
        wait_vmcnt<N2>();
      }
    }
    return;
  }

  // state waves 2s and 2s + 1 own the two channel halves of value tile s; output wave 2NW + s
  const int s = w < 2 * NW ? (w >> 1) : w - 2 * NW;   // value tile of this wave within the group
  const int vt = vg * NW + s;                         // 16-wide value tile

  if (w < 2 * NW) {
    // ---------------- state wave ----------------
    // Half hh of the tile's state: channels 64 hh .. 64 hh + 63, D layout of S^T:
    // S[i][j] = S[16 vt + lt][16 (4 hh + i) + 4 gq + j]. Per chunk the wave forms U for
    // token tiles 2hh, 2hh + 1 over all channels (its own half of S0 from registers, the
    // partner's from LDS), then updates its own channel half from both token halves of U
    // (its own from registers, the partner's from LDS). Every exchanged operand carries the
    // power-of-two scale of its own half.
    const int hh = w & 1;
    f32x4 S[4];
    const size_t st_off = ((size_t)(n * H + h) * VD + 16 * vt + lt) * KD + 64 * hh;
    // (varlen window) the carry slot of this window / the next, one sequence each
    const size_t carry_off = ((size_t)h * VD + 16 * vt + lt) * KD + 64 * hh;
    const size_t carry_slot = (size_t)H * VD * KD;
    // maps pass: tiles 0-7 are the value rows from a zero state (R), tiles 8-15 the rows
    // of the identity run without U~ (P); outputs pass: the scanned segment state
    const bool ptile = mode == CHAIN_MAPS && vt >= 8;
    if (mode == CHAIN_MAPS) {
      const int r = 16 * (vt - 8) + lt;   // identity row of a P tile
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) S[i][jj] = (ptile && 64 * hh + 16 * i + 4 * gq + jj == r) ? 1.0f : 0.0f;
    } else if (mode == CHAIN_OUTPUTS) {
      const float* src = p.seg.seg_init + st_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = *reinterpret_cast<const f32x4*>(src + 16 * i + 4 * gq);
    } else if (win_in) {
      const float* src = p.map.carry + (size_t)(p.map.win & 1) * carry_slot + carry_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = *reinterpret_cast<const f32x4*>(src + 16 * i + 4 * gq);
    } else if (p.init_dtype == 2) {
      const float* src = static_cast<const float*>(p.init_state) + st_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = *reinterpret_cast<const f32x4*>(src + 16 * i + 4 * gq);
    } else if (p.init_dtype == 1) {
      const uint16_t* src = static_cast<const uint16_t*>(p.init_state) + st_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 r = *reinterpret_cast<const u32x2*>(src + 16 * i + 4 * gq);
        S[i] = f32x4{bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y)};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = f32x4{0, 0, 0, 0};
    }

    // S0 half -> fp16 operand fragments (k-steps 2hh, 2hh + 1), each row v scaled by its own
    // power of two; published for the partner and the output wave as well
    float iS;
    u32x4 sf[2];
    auto publish_state = [&]() {
      float sS;
      pow2_scale(row_absmax(S, 4), sS, iS);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        sf[q] = pack_pair_f16(S[2 * q], S[2 * q + 1], sS);
        xc.sf[s][2 * hh + q][l] = sf[q];
      }
      if (gq == 0) xc.iS[s][hh][lt] = iS;
    };
    publish_state();

    for (int j = 0; j < nc; ++j) {
      const ChainPart1<NW>& P1 = r1[j & 1];
      const ChainPart2<NW>& P2 = r2[j & 1];
      lds_barrier();   // (A)

      // U = U~ + (-W) S0^T for token tiles 2hh + i.  D layout: lane <-> v, registers <-> tokens
      const u32x4 so0 = xc.sf[s][2 * (1 - hh)][l], so1 = xc.sf[s][2 * (1 - hh) + 1][l];
      const float iSo = xc.iS[s][1 - hh][lt];
      f32x4 U[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int mt = 2 * hh + i;
        f32x4 am = {0, 0, 0, 0}, ao = {0, 0, 0, 0};
        am = mfma_f16(P1.wneg[mt * 4 + 2 * hh][l], sf[0], am);
        ao = mfma_f16(P1.wneg[mt * 4 + 2 * (1 - hh)][l], so0, ao);
        am = mfma_f16(P1.wneg[mt * 4 + 2 * hh + 1][l], sf[1], am);
        ao = mfma_f16(P1.wneg[mt * 4 + 2 * (1 - hh) + 1][l], so1, ao);
        const u32x2 uh = P1.ut[s][mt][l];
        const f32x2 u01 = unpack_f16x2(uh.x), u23 = unpack_f16x2(uh.y);
        const f32x4 ut = ptile ? f32x4{0, 0, 0, 0} : f32x4{u01.x, u01.y, u23.x, u23.y} * P1.usc[s * 64 + mt * 16 + lt];
        U[i] = ut + am * iS + ao * iSo;
      }
      float sU, iU;
      pow2_scale(row_absmax(U, 2), sU, iU);
      const u32x4 uf = pack_pair_f16(U[0], U[1], sU);   // k-step hh of the state update
      xc.uf[s][hh][l] = uf;
      if (gq == 0) xc.iU[s][hh][lt] = iU;
      lds_barrier();   // (B)

      // S1^T = Diag(Gamma_L) S0^T + K'^T U   (this wave's channel tiles 4hh + i)
      const u32x4 ufo = xc.uf[s][1 - hh][l];
      const float iUo = xc.iU[s][1 - hh][lt];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mt = 4 * hh + i;
        const f32x4 g4 = *reinterpret_cast<const f32x4*>(&P2.gamw[128 + 16 * mt + 4 * gq]);
        const f32x4 am = mfma_f16(P2.kp[mt * 2 + hh][l], uf, f32x4{0, 0, 0, 0});
        const f32x4 ao = mfma_f16(P2.kp[mt * 2 + 1 - hh][l], ufo, f32x4{0, 0, 0, 0});
        S[i] = S[i] * g4 + am * iU + ao * iUo;
      }
      // the partner and the output wave have read S0's operands before (B); publish S1's
      publish_state();
    }

    if (mode == CHAIN_MAPS) {
      float* dst = p.seg.maps + ((size_t)(n * H + h) * (2 * VD) + 16 * vt + lt) * KD + 64 * hh;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(dst + 16 * i + 4 * gq) = S[i];
    } else if (mode == CHAIN_OUTPUTS) {
      // the scan writes final_state
    } else if (win_out) {
      float* dst = p.map.carry + (size_t)((p.map.win + 1) & 1) * carry_slot + carry_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(dst + 16 * i + 4 * gq) = S[i];
    } else if (p.final_dtype == 2) {
      float* dst = static_cast<float*>(p.final_state) + st_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(dst + 16 * i + 4 * gq) = S[i];
    } else if (p.final_dtype == 1) {
      uint16_t* dst = static_cast<uint16_t*>(p.final_state) + st_off;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x2*>(dst + 16 * i + 4 * gq) =
            u32x2{pack_bf16x2(S[i].x, S[i].y), pack_bf16x2(S[i].z, S[i].w)};
    }
    return;
  }

  // ---------------- output wave ----------------
  // O^T = scale (S0 Qg^T + U^T Aqk^T)   D layout: lane <-> token 16 nt + lt, registers <-> v.
  // Register jj of lane group gq belongs to value row 4 gq + jj of the tile. S0's channel
  // halves and U's token halves each come with their own scales.
  const float scale = p.scale;
  if (mode == CHAIN_MAPS) {   // no outputs: keep the two barriers of every chunk step
    for (int j = 0; j < nc; ++j) {
      lds_barrier();   // (A)
      lds_barrier();   // (B)
    }
    return;
  }
  for (int j = 0; j < nc; ++j) {
    const ChainPart1<NW>& P1 = r1[j & 1];
    const ChainPart2<NW>& P2 = r2[j & 1];
    lds_barrier();   // (A)
    u32x4 sf[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sf[q] = xc.sf[s][q][l];
    const f32x4 oS0 = *reinterpret_cast<const f32x4*>(&xc.iS[s][0][4 * gq]) * scale;
    const f32x4 oS1 = *reinterpret_cast<const f32x4*>(&xc.iS[s][1][4 * gq]) * scale;
    f32x4 aq[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
      a0 = mfma_f16(sf[0], P1.qg[nt * 4 + 0][l], a0);
      a1 = mfma_f16(sf[2], P1.qg[nt * 4 + 2][l], a1);
      a0 = mfma_f16(sf[1], P1.qg[nt * 4 + 1][l], a0);
      a1 = mfma_f16(sf[3], P1.qg[nt * 4 + 3][l], a1);
      aq[nt] = a0 * oS0 + a1 * oS1;
    }
    lds_barrier();   // (B)
    const u32x4 uf0 = xc.uf[s][0][l], uf1 = xc.uf[s][1][l];
    const f32x4 oU0 = *reinterpret_cast<const f32x4*>(&xc.iU[s][0][4 * gq]) * scale;
    const f32x4 oU1 = *reinterpret_cast<const f32x4*>(&xc.iU[s][1][4 * gq]) * scale;
    const int L = min(CH, len - j * CH);
    // every product first, then the stores: a store under a per-lane condition would
    // order each tile's LDS read, product and store one after another
    u32x4 af[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) af[i] = P2.aqk[i][l];
    u32x2 ob[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 o = aq[nt] + mfma_f16(uf0, af[aqk_slot(nt, 0)], f32x4{0, 0, 0, 0}) * oU0;
      if (nt >= 2) o += mfma_f16(uf1, af[aqk_slot(nt, 1)], f32x4{0, 0, 0, 0}) * oU1;
      ob[nt] = u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
    }
    // token 16 nt + lt of this chunk; consecutive tiles are 16 token rows apart
    uint16_t* dst = p.out + ((size_t)(tok0 + j * CH + lt) * H + h) * VD + 16 * vt + 4 * gq;
    const size_t tile_stride = (size_t)16 * H * VD;
    if (L == CH) {   // full chunk (uniform): no per-lane condition
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) *reinterpret_cast<u32x2*>(dst + nt * tile_stride) = ob[nt];
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (16 * nt + lt < L) *reinterpret_cast<u32x2*>(dst + nt * tile_stride) = ob[nt];
    }
  }
}

template <int NW>
constexpr bool chain_layout_ok() {
  return VD % (16 * NW) == 0 &&
         // the last group's scale window ends inside the record
         NW * 256 * (VD / (16 * NW) - 1) + USC_WIN <= OFF_GAML + 512 - OFF_USC;
}
static_assert(chain_layout_ok<2>() && chain_layout_ok<4>(), "value-tile grouping");
static_assert(OFF_QG == 16 * FRAG && OFF_KP == 32 * FRAG && OFF_AQK == 48 * FRAG,
              "shared fragments must be contiguous at the record start");

template <int NW>
hipError_t launch_chain_nw(const FwdParams& p, int NH, int rows, hipStream_t stream) {
  const int nvg = rows / (16 * NW);
  const int64_t blocks = (int64_t)((NH + 7) / 8) * 8 * nvg;
  const dim3 grid((unsigned)blocks), block((3 * NW + 1) * 64);
  if (p.seg.mode == CHAIN_MAPS)
    hipLaunchKernelGGL((kda_chain_kernel<NW, CHAIN_MAPS>), grid, block, 0, stream, p, nvg);
  else if (p.seg.mode == CHAIN_OUTPUTS)
    hipLaunchKernelGGL((kda_chain_kernel<NW, CHAIN_OUTPUTS>), grid, block, 0, stream, p, nvg);
  else
    hipLaunchKernelGGL((kda_chain_kernel<NW, CHAIN_FULL>), grid, block, 0, stream, p, nvg);
  return hipGetLastError();
}

}  // namespace

// Varlen calls in windows: final_state of the sequences without chunks, which no window's
// chain visits (in one launch the chain writes them itself, with no steps): their initial
// state, or zeros. One workgroup per sequence (most leave at once); 256 threads copy the
// 128 x 128 state of each head.
__global__ __launch_bounds__(256) void kda_empty_states_kernel(FwdParams p, int32_t N) {
  const int n = blockIdx.x;
  if (n >= N || p.final_dtype == 0) return;
  if (__builtin_amdgcn_readfirstlane(p.map.seq_tab[n].y) > 0) return;   // the windows carry it
  const int tid = threadIdx.x;
  for (int h = 0; h < p.H; ++h) {
    const size_t base = (size_t)(n * p.H + h) * VD * KD;
    for (int e = tid * 4; e < VD * KD; e += 256 * 4) {
      if (p.final_dtype == 2) {
        const f32x4 v = p.init_dtype == 2 ? *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.init_state) + base + e)
                                          : f32x4{0, 0, 0, 0};
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.final_state) + base + e) = v;
      } else {
        const u32x2 v = p.init_dtype == 1 ? *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.init_state) + base + e)
                                          : u32x2{0u, 0u};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.final_state) + base + e) = v;
      }
    }
  }
}

// Two value tiles per workgroup while the (sequence, head) chains alone leave
// compute units idle (more, shorter workgroups); four once there are enough
// chains, which halves how often each record's shared fragments are fetched.
hipError_t launch_chain(const FwdParams& p, hipStream_t stream) {
  const int NH = (p.seg.mode == CHAIN_FULL ? p.map.nseq : p.map.nseq * p.seg.nseg) * p.H;
  const int rows = p.seg.mode == CHAIN_MAPS ? 2 * VD : VD;   // value rows, plus the P rows of the maps pass
  if (NH <= 0) return hipSuccess;
  static const int cus = [] {   // compute units of the device (thread-safe one-time query)
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      return n;
    return 256;
  }();
  return (int64_t)NH * (rows / 32) <= cus ? launch_chain_nw<2>(p, NH, rows, stream)
                                          : launch_chain_nw<4>(p, NH, rows, stream);
}

hipError_t launch_empty_states(const FwdParams& p, int32_t N, hipStream_t stream) {
  if (N <= 0 || p.final_dtype == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_empty_states_kernel, dim3((unsigned)N), dim3(256), 0, stream, p, N);
  return hipGetLastError();
}

}  // namespace kda
