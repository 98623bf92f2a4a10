// kda_intra.hip -- intra-chunk kernel of the chunked KDA forward (gfx950).
//
// One workgroup (4 waves) per (64-token chunk, head); all chunks run in
// parallel. Wave w owns sub-chunk w (tokens 16w..16w+15); in the elementwise
// phase lane l holds token 16w + (l & 15) and 32 of its 128 channels (lane
// group l >> 4, "D-compatible" channel order, see kda_device.h).
//
// For the chunk (L <= 64 tokens; the start state S0 is the chain kernel's):
//   fused prologue : g~ = lb * sigmoid(exp(A_log) (g + dt_bias)),  beta = sigmoid(b),
//                    q^, k^ = L2-normalised q, k (eps 1e-6 under the root)
//   cumulative gate: G_t = sum_{s<=t} g~_s, kept as sub-chunk-local sums Gs plus
//                    per-sub-chunk reference points (so every exponential below
//                    stays within fp32 range when lb >= -5: |16 * lb| <= 80)
//   A   = StrictLower(diag(beta) (K^.Gamma)(K^/Gamma)^T)       (gram blocks on MFMA)
//   Aqk = Lower((Q^.Gamma)(K^/Gamma)^T)                        (gram blocks on MFMA)
//   Tm  = (I + A)^-1     diagonal 16x16 blocks by fp32 forward substitution, then
//                        each wave solves one column block with fp32 MFMA
//   W   = Tm diag(beta) (K^.Gamma),  U~ = Tm diag(beta) V       (MFMA)
//   K'  = K^ . Gamma_L / Gamma,  Qg = Q^ . Gamma,  Gamma_L = exp(G_L)
// and writes them in the fragment order the chain kernel loads. Channel-major
// copies (K'^T, (K^.Gamma)^T, V^T) are produced by an MFMA against a permutation
// operand, which is exact and needs no LDS scatter.
//
// Precision: diagonal gram blocks use bf16 operands (their column factor
// exp(-Gs) reaches e^80, beyond fp16 range); every other MFMA operand bounded by
// 1 in magnitude (normalised keys/queries times decays <= 1, W, Tm diag(beta))
// is fp16 for its 11-bit mantissa; U~ = Tm diag(beta) V uses a hi/lo bf16 split
// of Tm diag(beta) against the exact bf16 V, and is stored in fp16 with a
// power-of-two scale per (16-token tile, value column).
//
// The pages describe the method at the level of "gate activation, beta sigmoid
// and q/k L2 norm fused into the kernel, intermediates kept on chip" (page
// "FlashKDA：面向SM90+的高性能KDA CUDA内核库", Q1) and name the chunked form
// (2kiu.com guide, section 四, "分块、融合、精度"); the chunk algebra here is the
// standard WY/UT form of the gated delta rule.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int AROW = 68;   // floats per row of the padded 64x64 fp32 A matrix

// 52,480 bytes, so that three workgroups share a compute unit's 160 KiB. The region
// 'r' is reused three times: the gate constants and gram column fragments until the
// off-diagonal grams are formed (phases A-D), then A until Tm is solved (phases D-E),
// then V^T for phase F.
struct IntraSmem {
  float beta[CH];            // sigmoid(beta logits), 0 for padded tokens
  union {
    struct {
      float tot[4][KD];      // sub-chunk gate totals
      float eend[4][KD];     // exp(total of sub-chunk w)                     <= 1
      _Float16 exref_h[4][KD];   // exp(reference point of sub-chunk w)      <= 1, fp16
      _Float16 eend_h[4][KD];    // eend in fp16
      _Float16 c2_h[4][KD];      // exp(G_L - reference point of sub-chunk w+1) <= 1, fp16
      u32x4 tk[3][4][64];    // off-diagonal gram column fragments [sub-chunk][k-step][lane]
                             // (sub-chunk 3 is never the column block of a later one)
    } g;
    float A[CH][AROW];       // beta * gram, strictly lower (blocks on and below the diagonal)
    u32x4 vt[8][2][64];      // V^T bf16 fragments [value tile][token k-step][lane]
  } r;
  float tm[CH * CH];         // Tm, rows XOR-swizzled (see tmi)
  u32x4 kgt[8][2][64];       // (K^.Gamma)^T fp16 fragments [channel tile][token k-step][lane]
};
static_assert(sizeof(IntraSmem) <= 163840 / 3, "three workgroups per compute unit");

// swizzled index of Tm[r][c]: 16-byte column groups XORed with the row, so that
// 16 lanes reading 16 consecutive rows at one column hit 16 different banks
__device__ __forceinline__ int tmi(int r, int c) { return r * CH + (c ^ ((r & 15) << 2)); }

__device__ __forceinline__ void unpack8(u32x4 r, float* f) {
  f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
  f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
}
__device__ __forceinline__ u32x4 pk_f16(const float* f) {
  return u32x4{pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]), pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7])};
}
__device__ __forceinline__ u32x4 pk_bf16(const float* f) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}
__device__ __forceinline__ u32x4 mul_f16x8(u32x4 a, u32x4 b) {   // packed fp16 multiply (v_pk_mul_f16)
  return __builtin_bit_cast(u32x4, __builtin_bit_cast(f16x8, a) * __builtin_bit_cast(f16x8, b));
}
__device__ __forceinline__ u32x2 pk4_f16(f32x4 v) { return u32x2{pack_f16x2(v.x, v.y), pack_f16x2(v.z, v.w)}; }
__device__ __forceinline__ u32x2 pk4_bf16(f32x4 v) { return u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)}; }

// channels chan(s, 0..7, gq) = 32s + {4gq..4gq+3, 16+4gq..16+4gq+3} of one token row.
// One 16-byte load per lane: lane group gq reads the 8 channels 32s + 8c.. with
// c = (0, 2, 1, 3)[gq], so lane groups (0, 1) hold channels 0-7 and 16-23 and (2, 3)
// hold 8-15 and 24-31; one cross-row swap per register pair then gives even groups
// their partner's first four channels and odd groups their partner's last four.
__device__ __forceinline__ u32x4 load_row8(const uint16_t* row, int s, int gq, bool valid) {
  if (!valid) return u32x4{0u, 0u, 0u, 0u};
  const int c = ((gq & 1) << 1) | (gq >> 1);
  const u32x4 x = *reinterpret_cast<const u32x4*>(row + 32 * s + 8 * c);
  const auto a = __builtin_amdgcn_permlane16_swap(x.x, x.z, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(x.y, x.w, false, false);
  return u32x4{a[0], b[0], a[1], b[1]};
}
// p -> fp16 channels +0..3 and +16..19, packed in the order pk_f16 gives
__device__ __forceinline__ u32x4 ld8h(const _Float16* p) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(p);
  const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
  return u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void ld8f(const float* p, float* f) {   // p -> channels +0..3 and +16..19
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Permutation operand P (B side of a 16x16x32 MFMA over k-step s) with
// P[k][n] = 1 iff channel(k) == 16*(2s + par) + n, so that X_frag * P gives the
// 16x16 tile of channels 16*(2s+par).. in D layout: lane <-> channel, registers
// <-> tokens. 'one' is the bit pattern of 1.0 in the operand type.
__device__ __forceinline__ u32x4 perm_operand(int lt, int gq, int par, uint32_t one) {
  const int pos = lt - 4 * gq + 4 * par;   // register e holding channel 16*ct + lt, if 0 <= pos - 4 par < 4
  uint32_t r[4] = {0u, 0u, 0u, 0u};
  const bool hit = (lt - 4 * gq) >= 0 && (lt - 4 * gq) < 4;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (hit && e == pos) r[e >> 1] |= one << (16 * (e & 1));
  return u32x4{r[0], r[1], r[2], r[3]};
}

// Column block W of Tm = (I + A)^-1, given the diagonal blocks: for a = W+1..3,
//   Tm_aW = -Tm_aa * sum_{m=W}^{a-1} A_am Tm_mW
// on fp32 MFMA 16x16x4 (step i contracts index 4*gq + i). The blocks Tm_mW of this
// column stay in registers in D layout (lane (gq, c), register j <-> row 4gq + j,
// column c), which is exactly the B operand of the next product.
template <int W>
__device__ __forceinline__ void solve_column_block(IntraSmem& sm, int lt, int gq) {
  f32x4 Tc[4 - W];
#pragma unroll
  for (int i = 0; i < 4; ++i) Tc[0][i] = sm.tm[tmi(16 * W + 4 * gq + i, 16 * W + lt)];
#pragma unroll
  for (int a = W + 1; a < 4; ++a) {
    f32x4 X = {0, 0, 0, 0};
#pragma unroll
    for (int m = W; m < a; ++m) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.r.A[16 * a + lt][16 * m + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) X = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], Tc[m - W][i], X, 0, 0, 0);
    }
    const f32x4 tv = *reinterpret_cast<const f32x4*>(&sm.tm[tmi(16 * a + lt, 16 * a + 4 * gq)]);
    f32x4 Y = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[i], X[i], Y, 0, 0, 0);
    Y = -Y;
    Tc[a - W] = Y;
#pragma unroll
    for (int j = 0; j < 4; ++j) sm.tm[tmi(16 * a + 4 * gq + j, 16 * W + lt)] = Y[j];
  }
}

// lane I of each 16-lane row, broadcast to the whole row (DPP row_newbcast)
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + I, 0xf, 0xf, false));
}

// Largest gate sum (log2 units) of one 8-token half of a sub-chunk for the split form of
// its diagonal block (split_diag), whose within-half entries are factorised about each
// channel's midpoint of that half: the factors then stay within 2^(+-100), finite and
// (for key or query components above 2^-26) clear of the subnormal range, and every kept
// entry, a product of the two for i <= r, is at most 1. Entries above the diagonal or
// across the halves may overflow in that product; the selects that merge and mask the
// blocks discard them.
constexpr float DIAG_RANGE2_MID = 200.0f;

// Diagonal 16x16 gram block entries of one sub-chunk over one channel per lane, for
// gates of any size. Lane (gq, r) holds token r's k^, q^ and decay alpha = exp(g~) (log2
// units folded in) of one channel; for every token i of the sub-chunk it adds
//   PA[i] += k^_r . k^_i E,   PQ[i] += q^_r . k^_i E,   E = exp(G_r - G_i) (i <= r).
// E is a running product of the decays of tokens i+1..r, restarted at 1 where i >= r, so
// it never overflows; entries i > r are masked by the caller. It serves the channels that
// the split form leaves out (split_diag<true>).
template <int I>
__device__ __forceinline__ void pair_step1(float kn, float qn, float al, int lt, float& E, float* PA, float* PQ) {
  if constexpr (I < 15) {   // broadcast first: a cross-lane read must not sit under a lane condition
    const float a = row_bcast<I + 1>(al);
    E = (I >= lt) ? 1.0f : E * a;
  }
  const float kb = row_bcast<I>(kn) * E;
  PA[I] = fmaf(kn, kb, PA[I]);
  PQ[I] = fmaf(qn, kb, PQ[I]);
  if constexpr (I > 0) pair_step1<I - 1>(kn, qn, al, lt, E, PA, PQ);
}

// A channel of one sub-chunk that the split form cannot take: an 8-token half of its gate
// sum spans more than DIAG_RANGE2_MID (g7, g15: the channel's cumulative sums at tokens 7
// and 15, in log2 units). Both users evaluate it on the same values, so they agree.
__device__ __forceinline__ bool split_excluded(float g7, float g15) {
  return fmaxf(-g7, g7 - g15) > DIAG_RANGE2_MID;
}

// Sums of 16 per-lane values over the four lane groups {l, l^16, l^32, l^48}, leaving
// lane group gq with the sums of values 4gq..4gq+3 (a reduce-scatter on the gfx950
// cross-half lane swaps: lanes 0-31 keep values 0..7 and lanes 32-63 values 8..15,
// then the even 16-lane rows keep the first four of those and the odd rows the rest).
__device__ __forceinline__ f32x4 reduce_scatter16(const float* P) {
  float t[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[m]), __float_as_uint(P[8 + m]), false, false);
    t[m] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  f32x4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(t[m]), __float_as_uint(t[4 + m]), false, false);
    r[m] = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  return r;
}

// Diagonal 16x16 gram blocks of one sub-chunk in the split form, for gate sums too large
// for one reference point per channel (unbounded gate):
//   - entries within one 8-token half: factors 2^(Gs - m) (rows) and 2^(m - Gs) (columns)
//     about that half's per-channel midpoint m (g7 / 2 for the first half, (g7 + g15) / 2
//     for the second, with g7, g15 the channel's sums at tokens 7 and 15), each within
//     2^(+-span / 2) for a half whose gate sum spans at most span;
//   - entries of a second-half row against a first-half column: factors 2^(Gs - g7)
//     (rows) and 2^(g7 - Gs) (columns), both <= 1.
// One product holds every within-half entry (each lane's token takes its own half's
// midpoint), another the cross entries (rows of the first half and columns of the second
// half are zero there); the entries are merged by half here, and the caller masks those
// above the diagonal. Lane (gq, lt) holds token lt and the 32 channels of kraw / qraw /
// Gs (log2 units).
// MASK: leave out the channels split_excluded() names (their factors may overflow; the
// caller adds them entry by entry).
// WHOLE: a sub-chunk whose gate sums all stay within DIAG_RANGE2_MID: every token takes the
// midpoint g15 / 2 of its channel, so each factor is within 2^(+-100) and one product holds
// every kept entry (no cross product, no merge).
template <bool MASK, bool WHOLE = false>
__device__ __forceinline__ void split_diag(const u32x4* qraw, const u32x4* kraw, const float* Gs, float rq, float rk,
                                           int lt, int gq, f32x4& aD, f32x4& qD) {
  const bool hi = lt >= 8;
  f32x4 aX = {0, 0, 0, 0}, qX = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float qf[8], kf[8];
    unpack8(qraw[s], qf);
    unpack8(kraw[s], kf);
    uint32_t a1[4], q1[4], c1[4], a2[4], q2[4], c2[4];   // bf16 pairs, packed as formed
#pragma unroll
    for (int e2i = 0; e2i < 4; ++e2i) {
      float v[2][6];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = 2 * e2i + u;
        const float G = Gs[8 * s + e];
        const float g7 = row_bcast<7>(G), g15 = row_bcast<15>(G);   // broadcasts first, selects after
        const float m = WHOLE ? 0.5f * g15 : (hi ? 0.5f * (g7 + g15) : 0.5f * g7);
        const float up = fast_exp2(G - m), dn = fast_exp2(m - G);
        const float ex = WHOLE ? 0.0f : fast_exp2(hi ? G - g7 : g7 - G);   // <= 1
        const float kn = kf[e] * rk, qn = qf[e] * rq;
        v[u][0] = kn * up;
        v[u][1] = qn * up;
        v[u][2] = kn * dn;
        v[u][3] = (!WHOLE && hi) ? kn * ex : 0.0f;
        v[u][4] = (!WHOLE && hi) ? qn * ex : 0.0f;
        v[u][5] = (WHOLE || hi) ? 0.0f : kn * ex;
        if constexpr (MASK) {
          const bool out = split_excluded(g7, g15);
#pragma unroll
          for (int c = 0; c < 6; ++c) v[u][c] = out ? 0.0f : v[u][c];
        }
      }
      a1[e2i] = pack_bf16x2(v[0][0], v[1][0]);
      q1[e2i] = pack_bf16x2(v[0][1], v[1][1]);
      c1[e2i] = pack_bf16x2(v[0][2], v[1][2]);
      a2[e2i] = pack_bf16x2(v[0][3], v[1][3]);
      q2[e2i] = pack_bf16x2(v[0][4], v[1][4]);
      c2[e2i] = pack_bf16x2(v[0][5], v[1][5]);
    }
    const u32x4 C1 = {c1[0], c1[1], c1[2], c1[3]}, C2 = {c2[0], c2[1], c2[2], c2[3]};
    aD = mfma_bf16(u32x4{a1[0], a1[1], a1[2], a1[3]}, C1, aD);
    qD = mfma_bf16(C1, u32x4{q1[0], q1[1], q1[2], q1[3]}, qD);
    if constexpr (!WHOLE) {
      aX = mfma_bf16(u32x4{a2[0], a2[1], a2[2], a2[3]}, C2, aX);
      qX = mfma_bf16(C2, u32x4{q2[0], q2[1], q2[2], q2[3]}, qX);
    }
  }
  if constexpr (WHOLE) return;
  // aD[j] = D[4gq + j][lt] (row, column); qD[j] = D[key 4gq + j][query lt]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool same = (4 * gq + j >= 8) == hi;
    aD[j] = same ? aD[j] : aX[j];
    qD[j] = same ? qD[j] : qX[j];
  }
}

// Largest sub-chunk gate sum (log2 units) for which the factorised diagonal blocks
// stay finite: their column factor 2^-Gs is at most 2^118, and a 32-channel MFMA
// step then sums at most 128 * 2^118 = 2^125 < FLT_MAX.
constexpr float DIAG_RANGE2 = 118.0f;

// UB = false: the safe gate, g~ in [lower_bound, 0] with lower_bound >= -5, so a
//             16-token sub-chunk spans at most 80 natural-log units and every diagonal
//             block is formed from the factorised operands on MFMA.
// UB = true : the gate without the safe bound. Sub-chunks whose gate sums stay within
//             DIAG_RANGE2 take the same MFMA path; those within DIAG_RANGE2_MID take the
//             split form about one midpoint per channel (split_diag<false, true>); those
//             whose 8-token halves each stay within DIAG_RANGE2_MID take the split form
//             (split_diag); in the others the split form takes the channels within that
//             range and pair_step1 the rest, entry by entry (wave-uniform choices, per
//             sub-chunk and channel slot).
template <bool UB>
__global__ __launch_bounds__(256, 3) void kda_intra_kernel(FwdParams p) {
  __shared__ IntraSmem sm;
  const int H = p.H;
  const int slot = blockIdx.x;
  const int h = slot % H;
  // chunks are launched last-first: the records of a sequence's first chunks are then
  // the most recently written, still in the last-level cache when the chain starts there
  const int ci = p.map.max_chunks - 1 - slot / H;

  int t0, L;
  if (p.map.chunk_tab) {
    const int2 e = p.map.chunk_tab[p.map.jb + ci];   // (jb: the window's first slot)
    t0 = e.x;
    L = e.y;
  } else {
    const int row = ci / p.map.nc_win, j = p.map.jb + (ci - row * p.map.nc_win);
    t0 = row * p.map.T + j * CH;
    L = min(CH, p.map.T - j * CH);
  }
  if (L <= 0) return;   // unused varlen slot (uniform over the block)
  uint8_t* rec = p.rec + ((size_t)ci * H + h) * REC_BYTES;

  const int tid = threadIdx.x, l = tid & 63, lt = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index = sub-chunk, uniform
  const int tok = w * SUB + lt;
  const bool valid = tok < L;
  const size_t rowoff = ((size_t)(t0 + (valid ? tok : 0)) * H + h) * KD;

  // ---------------- phase A: loads, gate, sub-chunk cumulative sums, norms ----
  u32x4 qraw[4], kraw[4];
  // V rows: with the safe gate they are loaded with q, k and g (the kernel then needs 154
  // VGPRs, still three workgroups per compute unit) and wait in registers until phase F;
  // the unbounded-gate kernel has no registers to spare and loads them after the solve
  u32x4 vr[4];
  float Gs[32];   // sub-chunk cumulative gates in log2 units (exp2(Gs) = exp of the natural sums)
  float rq, rk;
  bool slow = false;   // (UB only) this sub-chunk's diagonal block is formed entry by entry
  bool split = false;  // (UB only) ... on MFMA, in the split form (split_diag)
  bool whole = false;  // (UB only) ... about one midpoint per channel (with split set)
  // diagonal gram block of this sub-chunk: D[r][i] = k^_r.k^_i exp(Gs_r - Gs_i) and
  // D[i][r] = k^_i.q^_r exp(Gs_r - Gs_i) in D layout (MFMA path, phase B); on the
  // entry-by-entry path (phase A) aD holds the first transposed, see phase D
  f32x4 aD = {0, 0, 0, 0}, qD = {0, 0, 0, 0};
  {
    // fused safe gate: gate * log2(e) = (lb log2 e) / (1 + 2^(-exp(A_log) log2(e) (g + dt_bias)));
    // fused unbounded gate: gate * log2(e) = -exp(A_log) log2(1 + 2^((g + dt_bias) log2 e));
    // pre-activated gate (switch off): g clamped into [lb, 0] (unbounded: min(g, 0)), times log2(e)
    const bool fuse_gate = (p.flags & FUSE_GATE) != 0;
    const float lb = p.lower_bound, lb2 = lb * LOG2E;
    const float rate2 = fuse_gate ? -__expf(p.A_log[h]) * (UB ? 1.0f : LOG2E) : 0.0f;
    // every load of the phase is issued before the first use, without a per-lane branch
    // (tokens past the chunk end read the chunk's first row and are zeroed below), so the
    // phase waits for memory once
    u32x4 graw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qraw[s] = load_row8(p.q + rowoff, s, gq, true);
      kraw[s] = load_row8(p.k + rowoff, s, gq, true);
      graw[s] = load_row8(p.g + rowoff, s, gq, true);
    }
    if constexpr (!UB) {
#pragma unroll
      for (int s = 0; s < 4; ++s) vr[s] = load_row8(p.v + rowoff, s, gq, true);
    }
    float dtf[32];
    if (fuse_gate) {
      const float* dt = p.dt_bias + (size_t)h * KD;
#pragma unroll
      for (int s = 0; s < 4; ++s) ld8f(dt + 32 * s + 4 * gq, &dtf[8 * s]);
    }
    const float braw = bf16_to_f32(p.beta[(size_t)(t0 + (valid ? tok : 0)) * H + h]);
    if (L < CH && !valid) {   // partial chunk: rows past its end are zero
#pragma unroll
      for (int s = 0; s < 4; ++s) qraw[s] = kraw[s] = graw[s] = u32x4{0u, 0u, 0u, 0u};
    }
    float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float gf[8];
      unpack8(graw[s], gf);
      if (fuse_gate) {
        // rows past the chunk end take gate 0 through the outer factor (the inner terms are
        // finite and >= 0 there), so no per-element select is needed
        const float lb2v = valid ? lb2 : 0.0f, rate2v = valid ? rate2 : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Gs[8 * s + e] = UB ? rate2v * softplus_log2((gf[e] + dtf[8 * s + e]) * LOG2E)
                             : lb2v * fast_rcp(1.0f + fast_exp2(rate2 * (gf[e] + dtf[8 * s + e])));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Gs[8 * s + e] = valid ? (UB ? fminf(gf[e], 0.0f) : fminf(fmaxf(gf[e], lb), 0.0f)) * LOG2E : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // squared norms straight from the packed bf16 pairs
        ssq = dot2_bf16(qraw[s][i], qraw[s][i], ssq);
        ssk = dot2_bf16(kraw[s][i], kraw[s][i], ssk);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) Gs[i] = row16_inclusive_scan(Gs[i]);
    if (UB) {   // the gates are <= 0, so the smallest cumulative sum is the sub-chunk total
      float mn = Gs[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) mn = fminf(mn, Gs[i]);
      const float wmn = wave_min(mn);
      slow = __builtin_amdgcn_readfirstlane(wmn < -DIAG_RANGE2 ? 1 : 0) != 0;
      whole = slow && __builtin_amdgcn_readfirstlane(wmn >= -DIAG_RANGE2_MID ? 1 : 0) != 0;
      if (whole) {
        split = true;
        slow = false;
      } else if (slow) {   // the split form applies when each 8-token half spans at most DIAG_RANGE2_MID
        // largest gate span of an 8-token half: the lanes at each half's end take the sum 8
        // lanes back (0 past the row start) minus their own
        float d2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float b8 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(Gs[i]), 0x118, 0xf, 0xf, true));
          d2 = fmaxf(d2, b8 - Gs[i]);
        }
        d2 = (lt & 7) == 7 ? d2 : 0.0f;
        split = __builtin_amdgcn_readfirstlane(wave_max(d2) <= DIAG_RANGE2_MID ? 1 : 0) != 0;
        slow = !split;
      }
    }
    if (lt == 15) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<f32x4*>(&sm.r.g.tot[w][32 * s + 4 * gq]) = f32x4{Gs[8 * s], Gs[8 * s + 1], Gs[8 * s + 2], Gs[8 * s + 3]};
        *reinterpret_cast<f32x4*>(&sm.r.g.tot[w][32 * s + 16 + 4 * gq]) =
            f32x4{Gs[8 * s + 4], Gs[8 * s + 5], Gs[8 * s + 6], Gs[8 * s + 7]};
      }
    }
    // the four lane groups of a token hold disjoint channels: sum over them
    ssq += __shfl_xor(ssq, 16, 64);
    ssq += __shfl_xor(ssq, 32, 64);
    ssk += __shfl_xor(ssk, 16, 64);
    ssk += __shfl_xor(ssk, 32, 64);
    const bool fuse_norm = (p.flags & FUSE_QK_L2NORM) != 0;
    rq = fuse_norm ? rsqrtf(ssq + 1e-6f) : 1.0f;
    rk = fuse_norm ? rsqrtf(ssk + 1e-6f) : 1.0f;
    if (gq == 0) sm.beta[tok] = valid ? ((p.flags & FUSE_BETA_SIGMOID) ? sigmoidf_fast(braw) : braw) : 0.0f;
    if (UB && slow) {
      // the channels the split form leaves out (split_excluded), entry by entry; a channel
      // slot (s, e) holds one channel per lane group and is skipped when none of its four
      // channels is excluded (a wave-uniform test)
      float PA[16], PQ[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) PA[i] = PQ[i] = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float qf[8], kf[8];
        unpack8(qraw[s], qf);
        unpack8(kraw[s], kf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float G = Gs[8 * s + e];
          // this token's decay: the step of the cumulative sum from the previous token
          const float prev = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(G), 0x111, 0xf, 0xf, true));
          const float g7 = row_bcast<7>(G), g15 = row_bcast<15>(G);
          const bool out = split_excluded(g7, g15);
          if (__builtin_amdgcn_ballot_w64(out) != 0) {
            float E = 1.0f;
            pair_step1<15>(out ? kf[e] * rk : 0.0f, out ? qf[e] * rq : 0.0f, fast_exp2(G - prev), lt, E, PA, PQ);
          }
        }
      }
      // lane (gq, r) now holds, for columns i = 4gq + j: gram row r (aD) and Aqk of
      // query r, key i (qD, already the MFMA layout), over the excluded channels
      aD = reduce_scatter16(PA);
      qD = reduce_scatter16(PQ);
    }
  }
  lds_barrier();

  // ---------------- phase C: per-channel constants of the chunk -------------
  {
    const int c = tid & (KD - 1);
    const int wa = tid >> 7;   // this thread fills sub-chunks wa and wa + 2
    const float t0v = sm.r.g.tot[0][c], t1v = sm.r.g.tot[1][c], t2v = sm.r.g.tot[2][c], t3v = sm.r.g.tot[3][c];
    const float GL = t0v + t1v + t2v + t3v;
    const float rA = wa ? t0v : 0.0f, rA1 = wa ? t0v + t1v : t0v;                  // ref_wa, ref_wa+1
    const float rB = wa ? t0v + t1v + t2v : t0v + t1v, rB1 = wa ? GL : t0v + t1v + t2v;   // ref_wa+2, ref_wa+3
    const float eA = fast_exp2(rA1 - rA), eB = fast_exp2(rB1 - rB);   // the totals are in log2 units
    sm.r.g.eend[wa][c] = eA;
    sm.r.g.eend[wa + 2][c] = eB;
    sm.r.g.eend_h[wa][c] = (_Float16)eA;
    sm.r.g.eend_h[wa + 2][c] = (_Float16)eB;
    sm.r.g.exref_h[wa][c] = (_Float16)fast_exp2(rA);
    sm.r.g.exref_h[wa + 2][c] = (_Float16)fast_exp2(rB);
    sm.r.g.c2_h[wa][c] = (_Float16)fast_exp2(GL - rA1);
    sm.r.g.c2_h[wa + 2][c] = (_Float16)fast_exp2(GL - rB1);
    if (tid < KD) reinterpret_cast<float*>(rec + OFF_GAML)[c] = fast_exp2(GL);
  }
  lds_barrier();

  // ---------------- phase B: operands, diagonal grams, permuted copies -------
  f32x4 aS = {0, 0, 0, 0};   // (UB, slow sub-chunk) gram block over the channels of the split form
  if (UB && whole) split_diag<false, true>(qraw, kraw, Gs, rq, rk, lt, gq, aD, qD);
  else if (UB && split) split_diag<false>(qraw, kraw, Gs, rq, rk, lt, gq, aD, qD);
  if (UB && slow) {
    f32x4 qS = {0, 0, 0, 0};
    split_diag<true>(qraw, kraw, Gs, rq, rk, lt, gq, aS, qS);
    qD += qS;
  }
  const u32x4 idh0 = perm_operand(lt, gq, 0, 0x3C00u), idh1 = perm_operand(lt, gq, 1, 0x3C00u);
  const int half = (w & 1) * 8;   // byte offset of this sub-chunk's tokens inside a 32-token fragment
  u32x4 Rkh[4], Rqh[4];            // off-diagonal gram rows (fp16), kept for phase D
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float qf[8], kf[8];
    unpack8(qraw[s], qf);
    unpack8(kraw[s], kf);
    const u32x4 exh = ld8h(&sm.r.g.exref_h[w][32 * s + 4 * gq]);   // exp(ref_w) in fp16
    const u32x4 c2h = ld8h(&sm.r.g.c2_h[w][32 * s + 4 * gq]);      // exp(G_L - ref_w+1) in fp16
    // exp(sub-chunk total) for the factorised path; (UB only) the total itself for a
    // sub-chunk past DIAG_RANGE2 (diagonal block entry by entry in phase A, or in the
    // split form), where exp(-G) may be out of fp32 range and exp(end_w - G) is taken directly
    const bool direct = UB && (slow || split);
    float en[8];
    ld8f(direct ? &sm.r.g.tot[w][32 * s + 4 * gq] : &sm.r.g.eend[w][32 * s + 4 * gq], en);
    float rke[8], rqe[8], cki[8], tk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kn = kf[e] * rk, qn = qf[e] * rq;
      const float ee = fast_exp2(Gs[8 * s + e]);  // <= 1 (may underflow to 0 on the entry-by-entry path)
      const float ie = fast_rcp(ee);              // <= e^80 (2^118 with an unbounded gate)
      rke[e] = kn * ee;
      rqe[e] = qn * ee;
      cki[e] = kn * ie;
      tk[e] = kn * (direct ? fast_exp2(en[e] - Gs[8 * s + e]) : ie * en[e]);   // K^ exp(end_w - G) <= 1
    }
    if (!(UB && (slow || split))) {   // diagonal gram blocks from the factorised operands
      const u32x4 rkd = pk_bf16(rke), ckd = pk_bf16(cki), rqd = pk_bf16(rqe);
      aD = mfma_bf16(rkd, ckd, aD);                 // D[r][i] = k^_r.k^_i exp(Gs_r - Gs_i)
      qD = mfma_bf16(ckd, rqd, qD);                 // D[i][r] = k^_i.q^_r exp(Gs_r - Gs_i)
    }
    Rkh[s] = pk_f16(rke);
    Rqh[s] = pk_f16(rqe);
    const u32x4 tkh = pk_f16(tk);
    if (w < 3) sm.r.g.tk[w][s][l] = tkh;
    // the operands scaled by per-channel factors <= 1, as packed fp16 products:
    //   Q^ exp(G) = (Q^ exp(Gs)) exp(ref_w),  K^ exp(G) likewise,  K^ exp(G_L - G) = tk exp(G_L - ref_w+1)
    *reinterpret_cast<u32x4*>(rec + OFF_QG + ((w * 4 + s) * 64 + l) * 16) = mul_f16x8(Rqh[s], exh);
    const u32x4 kph = mul_f16x8(tkh, c2h), kgh = mul_f16x8(Rkh[s], exh);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int ct = 2 * s + par;
      const f32x4 z = {0, 0, 0, 0};
      // K'^T tile ct of this sub-chunk -> chain fragment (channel tile ct, token k-step w/2), half w&1
      const f32x4 dk = mfma_f16(kph, par ? idh1 : idh0, z);
      *reinterpret_cast<u32x2*>(rec + OFF_KP + ((ct * 2 + (w >> 1)) * 64 + l) * 16 + half) = pk4_f16(dk);
      const f32x4 dg = mfma_f16(kgh, par ? idh1 : idh0, z);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(&sm.kgt[ct][w >> 1][l]) + half) = pk4_f16(dg);
    }
  }
  lds_barrier();

  // ---------------- phase D: off-diagonal grams, A to LDS, Aqk out ----------
  {
    f32x4 aO[3], qO[3];   // by distance 1..3
#pragma unroll
    for (int d = 0; d < 3; ++d) aO[d] = qO[d] = f32x4{0, 0, 0, 0};
    if (w >= 1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 tb = sm.r.g.tk[w - 1][s][l];
        aO[0] = mfma_f16(Rkh[s], tb, aO[0]);
        qO[0] = mfma_f16(tb, Rqh[s], qO[0]);
      }
    }
    if (w >= 2) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 dh = ld8h(&sm.r.g.eend_h[w - 1][32 * s + 4 * gq]);   // exp(ref_w - ref_{w-1})
        const u32x4 tb = sm.r.g.tk[w - 2][s][l];
        aO[1] = mfma_f16(mul_f16x8(Rkh[s], dh), tb, aO[1]);
        qO[1] = mfma_f16(tb, mul_f16x8(Rqh[s], dh), qO[1]);
      }
    }
    if (w >= 3) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 dh = mul_f16x8(ld8h(&sm.r.g.eend_h[2][32 * s + 4 * gq]),
                                   ld8h(&sm.r.g.eend_h[1][32 * s + 4 * gq]));   // exp(ref_3 - ref_1)
        const u32x4 tb = sm.r.g.tk[0][s][l];
        aO[2] = mfma_f16(mul_f16x8(Rkh[s], dh), tb, aO[2]);
        qO[2] = mfma_f16(tb, mul_f16x8(Rqh[s], dh), qO[2]);
      }
    }
    lds_barrier();   // every wave is past its reads of the gram fragments and constants: A may overwrite them
    // rows r = 16w + 4gq + j, columns i = 16b + lt
    const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[16 * w + 4 * gq]);
    if (UB && slow) {   // aS[j] = gram[4gq + j][lt] (split-form channels), aD[j] = gram[lt][4gq + j] (the rest)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * gq + j;
        sm.r.A[16 * w + r][16 * w + lt] = (r > lt) ? br[j] * aS[j] : 0.0f;
      }
      // then the excluded channels' part, added by the same wave (its LDS accesses stay in order)
      const float b = sm.beta[16 * w + lt];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lt > 4 * gq + j) sm.r.A[16 * w + lt][16 * w + 4 * gq + j] += b * aD[j];
    } else {            // aD[j] = gram[4gq + j][lt]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * gq + j;
        sm.r.A[16 * w + r][16 * w + lt] = (r > lt) ? br[j] * aD[j] : 0.0f;
      }
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      if (w >= d + 1) {
        const int b = w - 1 - d;
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.r.A[16 * w + 4 * gq + j][16 * b + lt] = br[j] * aO[d][j];
      }
    }
    // Aqk^T blocks: lane <-> query r = lt (tile w), registers <-> keys 16b + 4gq + j.
    // Fragment (tile w, k-step b>>1), half b&1. The diagonal block keeps keys <= query.
    {
      f32x4 dq;
#pragma unroll
      for (int j = 0; j < 4; ++j) dq[j] = (4 * gq + j <= lt) ? qD[j] : 0.0f;
      uint8_t* fr = rec + OFF_AQK + ((w * 2 + (w >> 1)) * 64 + l) * 16 + half;
      *reinterpret_cast<u32x2*>(fr) = pk4_f16(dq);
      if ((w & 1) == 0) *reinterpret_cast<u32x2*>(fr + 8) = u32x2{0u, 0u};   // keys above the diagonal
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      if (w >= d + 1) {
        const int b = w - 1 - d;
        uint8_t* fr = rec + OFF_AQK + ((w * 2 + (b >> 1)) * 64 + l) * 16 + (b & 1) * 8;
        *reinterpret_cast<u32x2*>(fr) = pk4_f16(qO[d]);
      }
    }
  }
  lds_barrier();

  // ---------------- phase E: Tm = (I + A)^-1 (fp32) ----------------------------
  {
    // diagonal block w by forward substitution; every lane group solves column lt
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == lt) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int m4 = 0; m4 < i; m4 += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.r.A[16 * w + i][16 * w + m4]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m4 + u < i) acc += a4[u] * x[m4 + u];
      }
      if (i > lt) x[i] = -acc;
    }
    if (gq == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.tm[tmi(16 * w + i, 16 * w + lt)] = x[i];
    }
  }
  lds_barrier();
  if (w == 0) solve_column_block<0>(sm, lt, gq);
  else if (w == 1) solve_column_block<1>(sm, lt, gq);
  else if (w == 2) solve_column_block<2>(sm, lt, gq);
  lds_barrier();
  {
    // A is no longer needed: V^T takes its place.
    const u32x4 idb0 = perm_operand(lt, gq, 0, 0x3F80u), idb1 = perm_operand(lt, gq, 1, 0x3F80u);
    if constexpr (UB) {
#pragma unroll
      for (int s = 0; s < 4; ++s) vr[s] = load_row8(p.v + rowoff, s, gq, true);
    }
    if (L < CH && !valid) {
#pragma unroll
      for (int s = 0; s < 4; ++s) vr[s] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const f32x4 dv = mfma_bf16(vr[s], par ? idb1 : idb0, f32x4{0, 0, 0, 0});
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(&sm.r.vt[2 * s + par][w >> 1][l]) + half) = pk4_bf16(dv);
      }
    }
  }
  lds_barrier();

  // ---------------- phase F: W = Tm diag(beta) K^.Gamma,  U~ = Tm diag(beta) V -
  {
    const int t = 16 * w + lt;
    const int smax = (w >= 2) ? 1 : 0;
    f32x4 accW[8], accU[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) accW[i] = accU[i] = f32x4{0, 0, 0, 0};
    for (int s = 0; s <= smax; ++s) {
      // Tm diag(beta) row t at tokens m(e) = 32s + 4gq + e (e < 4), 32s + 16 + 4gq + e - 4 (e >= 4)
      const int m0 = 32 * s + 4 * gq, m1 = m0 + 16;
      const f32x4 r0 = *reinterpret_cast<const f32x4*>(&sm.tm[tmi(t, m0)]);
      const f32x4 r1 = *reinterpret_cast<const f32x4*>(&sm.tm[tmi(t, m1)]);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&sm.beta[m0]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&sm.beta[m1]);
      float val[8], lo[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[e] = (m0 + e <= t) ? r0[e] * b0[e] : 0.0f;
        val[4 + e] = (m1 + e <= t) ? r1[e] * b1[e] : 0.0f;
      }
      const u32x4 tmh = pk_f16(val);
      const u32x4 hi = pk_bf16(val);
      {
        float hf[8];
        unpack8(hi, hf);
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = val[e] - hf[e];
      }
      const u32x4 lov = pk_bf16(lo);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) accW[ct] = mfma_f16(sm.kgt[ct][s][l], tmh, accW[ct]);   // D[c][t]
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) {
        const u32x4 vb = sm.r.vt[vt][s][l];
        accU[vt] = mfma_bf16(hi, vb, accU[vt]);                                            // D[t][v]
        accU[vt] = mfma_bf16(lov, vb, accU[vt]);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 a = -accW[2 * s], b = -accW[2 * s + 1];
      const u32x2 pa = pk4_f16(a), pb = pk4_f16(b);
      *reinterpret_cast<u32x4*>(rec + OFF_WNEG + ((w * 4 + s) * 64 + l) * 16) = u32x4{pa.x, pa.y, pb.x, pb.y};
    }
    // U~ in fp16, one power-of-two scale per (token tile w, value column)
#pragma unroll
    for (int vt = 0; vt < 8; ++vt) {
      const f32x4 u = accU[vt];
      float sc, inv;
      pow2_scale(max_over_groups(fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w)))), sc, inv);
      *reinterpret_cast<u32x2*>(rec + OFF_UT + ((vt * 4 + w) * 64 + l) * 8) = pk4_f16(u * sc);
      if (gq == 0) reinterpret_cast<float*>(rec + OFF_USC)[(vt * 4 + w) * 16 + lt] = inv;
    }
  }
}

}  // namespace

hipError_t launch_intra(const FwdParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.map.max_chunks * p.H;
  if (blocks <= 0) return hipSuccess;
  if (p.flags & GATE_UNBOUNDED)
    hipLaunchKernelGGL(kda_intra_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(kda_intra_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
