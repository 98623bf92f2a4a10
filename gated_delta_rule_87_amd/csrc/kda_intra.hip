// kda_intra.hip -- intra-chunk kernel of the chunked KDA forward (gfx950).
//
// One workgroup (4 waves) per (64-token chunk, head); all chunks run in
// parallel. Wave w owns sub-chunk w (tokens 16w..16w+15); in the elementwise
// phase lane l holds token 16w + (l & 15) and 32 of its 128 channels (lane
// group l >> 4, "D-compatible" channel order, see kda_device.h).
//
// For the chunk (L <= 64 tokens, start state S0 handled by the chain kernel):
//   fused prologue : g~ = lb * sigmoid(exp(A_log) (g + dt_bias)),  beta = sigmoid(b),
//                    q^, k^ = L2-normalised q, k (eps 1e-6 under the root)
//   cumulative gate: G_t = sum_{s<=t} g~_s, kept as sub-chunk-local sums Gs plus
//                    per-sub-chunk reference points (so every exponential below
//                    stays within fp32 range when lb >= -5: |16 * lb| <= 80)
//   A   = StrictLower(diag(beta) (K^.Gamma)(K^/Gamma)^T)       (gram on MFMA)
//   Aqk = Lower((Q^.Gamma)(K^/Gamma)^T)                        (gram on MFMA)
//   Tm  = (I + A)^-1                                           (fp32 block forward substitution)
//   W   = Tm diag(beta) (K^.Gamma),  U~ = Tm diag(beta) V       (MFMA)
//   K'  = K^ . Gamma_L / Gamma,  Qg = Q^ . Gamma,  Gamma_L = exp(G_L)
// and writes them in the fragment order the chain kernel loads (one 16-byte
// load per lane per 16x32 fragment).
//
// Precision: diagonal gram blocks use bf16 operands (their column factor
// exp(-Gs) reaches e^80, beyond fp16 range); every other MFMA operand that is
// bounded by 1 in magnitude (normalised keys/queries times decays <= 1, W,
// Tm diag(beta)) is fp16 for its 11-bit mantissa; U~ = Tm diag(beta) V uses a
// hi/lo bf16 split of Tm diag(beta) against the exact bf16 V and is stored in
// fp32.
//
// The pages describe the method only at the level of "fusion of gate
// activation, beta sigmoid and q/k L2 norm into the kernel, intermediates kept
// on chip" (page "FlashKDA：面向SM90+的高性能KDA CUDA内核库", Q1) and name the
// chunked form ("设计深度解析（分块、融合、精度）", 2kiu.com guide section 四);
// the chunk algebra here is the standard WY/UT form of the gated delta rule.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int TROW = 72;   // 16-bit elements per row of the channel-major [128][64] tiles (+8 pad)
constexpr int AROW = 68;   // floats per row of the 64x64 fp32 A / Tm matrix (+4 pad)

struct IntraSmem {
  float tot[4][KD];          // sub-chunk gate totals
  float exref[4][KD];        // exp(reference point of sub-chunk w)          <= 1
  float eend[4][KD];         // exp(total of sub-chunk w)                     <= 1
  float c2[4][KD];           // exp(G_L - reference point of sub-chunk w+1)   <= 1
  float beta[CH];            // sigmoid(beta logits), 0 for padded tokens
  u32x4 tk[4][4][64];        // off-diagonal gram column fragments [sub-chunk][k-step][lane];
                             // reused as fp32 scratch in the triangular solve
  uint16_t kgt[KD][TROW];    // (K^.Gamma)^T fp16, channel-major
  uint16_t vt[VD][TROW];     // V^T bf16, channel-major
  union {
    uint16_t kpt[KD][TROW];  // K'^T fp16, channel-major (until written out)
    float A[CH][AROW];       // then beta*gram (strict lower), inverted in place into Tm
  } u;
};

// channel held by (k-step s, register e) of lane group gq
__device__ __forceinline__ int chan(int s, int e, int gq) {
  return 32 * s + (e < 4 ? 4 * gq + e : 16 + 4 * gq + (e - 4));
}

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

// load channels chan(s, 0..7, gq) of one token row (8-byte loads), zeros when !valid
__device__ __forceinline__ u32x4 load_row8(const uint16_t* row, int s, int gq, bool valid) {
  if (!valid) return u32x4{0u, 0u, 0u, 0u};
  u32x2 a = *reinterpret_cast<const u32x2*>(row + 32 * s + 4 * gq);
  u32x2 b = *reinterpret_cast<const u32x2*>(row + 32 * s + 16 + 4 * gq);
  return u32x4{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ void ld8f(const float* p, float* f) {   // p -> channels 4gq.. and 16+4gq..
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__global__ __launch_bounds__(256, 2) void kda_intra_kernel(FwdParams p) {
  __shared__ IntraSmem sm;
  const int H = p.H;
  const int slot = blockIdx.x;
  const int h = slot % H;
  const int ci = slot / H;

  int t0, L;
  if (p.map.chunk_tab) {
    const int2 e = p.map.chunk_tab[ci];
    t0 = e.x;
    L = e.y;
  } else {
    const int row = ci / p.map.nc_row, j = ci - row * p.map.nc_row;
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

  // ---------------- phase A: loads, gate, sub-chunk cumulative sums ---------
  u32x4 qraw[4], kraw[4], vraw[4];
  float Gs[32];
  {
    const float rate = expf(p.A_log[h]);
    const float lb = p.lower_bound;
    const float* dt = p.dt_bias + (size_t)h * KD;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qraw[s] = load_row8(p.q + rowoff, s, gq, valid);
      kraw[s] = load_row8(p.k + rowoff, s, gq, valid);
      vraw[s] = load_row8(p.v + rowoff, s, gq, valid);
      const u32x4 graw = load_row8(p.g + rowoff, s, gq, valid);
      float gf[8], dtf[8];
      unpack8(graw, gf);
      ld8f(dt + 32 * s + 4 * gq, dtf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gate = lb * sigmoidf_fast(rate * (gf[e] + dtf[e]));
        Gs[8 * s + e] = valid ? gate : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) Gs[i] = row16_inclusive_scan(Gs[i]);
    if (lt == 15) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<f32x4*>(&sm.tot[w][32 * s + 4 * gq]) = f32x4{Gs[8 * s], Gs[8 * s + 1], Gs[8 * s + 2], Gs[8 * s + 3]};
        *reinterpret_cast<f32x4*>(&sm.tot[w][32 * s + 16 + 4 * gq]) =
            f32x4{Gs[8 * s + 4], Gs[8 * s + 5], Gs[8 * s + 6], Gs[8 * s + 7]};
      }
    }
    if (gq == 0) {
      const float b = valid ? bf16_to_f32(p.beta[(size_t)(t0 + tok) * H + h]) : 0.0f;
      sm.beta[tok] = valid ? sigmoidf_fast(b) : 0.0f;
    }
  }
  __syncthreads();

  // ---------------- phase C: per-channel constants of the chunk -------------
  {
    const int c = tid & (KD - 1);
    const float t0v = sm.tot[0][c], t1v = sm.tot[1][c], t2v = sm.tot[2][c], t3v = sm.tot[3][c];
    const float ref[5] = {0.0f, t0v, t0v + t1v, t0v + t1v + t2v, t0v + t1v + t2v + t3v};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int wa = (tid >> 7) + 2 * k2;
      sm.exref[wa][c] = expf(ref[wa]);
      sm.eend[wa][c] = expf(sm.tot[wa][c]);
      sm.c2[wa][c] = expf(ref[4] - ref[wa + 1]);
    }
    if (tid < KD) reinterpret_cast<float*>(rec + OFF_GAML)[c] = expf(ref[4]);
  }
  __syncthreads();

  // ---------------- phase B: normalise, form operands -----------------------
  u32x4 Rkd[4], Ckd[4], Rqd[4];        // diagonal gram blocks (bf16)
  u32x4 Rkh[4], Rqh[4];                // off-diagonal rows, distance 1 (fp16)
  u32x4 Rkh2[4], Rqh2[4];              // distance 2 (sub-chunks 2, 3)
  u32x4 Rkh3[4], Rqh3[4];              // distance 3 (sub-chunk 3)
  {
    float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float qf[8], kf[8];
      unpack8(qraw[s], qf);
      unpack8(kraw[s], kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ssq += qf[e] * qf[e];
        ssk += kf[e] * kf[e];
      }
    }
    ssq += __shfl_xor(ssq, 16, 64);
    ssq += __shfl_xor(ssq, 32, 64);
    ssk += __shfl_xor(ssk, 16, 64);
    ssk += __shfl_xor(ssk, 32, 64);
    const float rq = rsqrtf(ssq + 1e-6f), rk = rsqrtf(ssk + 1e-6f);

#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float qf[8], kf[8], vf[8], exr[8], een[8], cc2[8], d2[8], d3[8];
      unpack8(qraw[s], qf);
      unpack8(kraw[s], kf);
      ld8f(&sm.exref[w][32 * s + 4 * gq], exr);
      ld8f(&sm.eend[w][32 * s + 4 * gq], een);
      ld8f(&sm.c2[w][32 * s + 4 * gq], cc2);
      if (w >= 2) ld8f(&sm.eend[w - 1][32 * s + 4 * gq], d2);
      if (w >= 3) {
        float e2[8];
        ld8f(&sm.eend[w - 2][32 * s + 4 * gq], e2);
#pragma unroll
        for (int e = 0; e < 8; ++e) d3[e] = d2[e] * e2[e];
      }
      float rke[8], rqe[8], cki[8], tk[8], kp[8], kg[8], qg[8], t2[8], t3[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kn = kf[e] * rk, qn = qf[e] * rq;
        const float ee = fast_exp(Gs[8 * s + e]);     // <= 1
        const float ie = fast_rcp(ee);                // <= e^80
        rke[e] = kn * ee;
        rqe[e] = qn * ee;
        cki[e] = kn * ie;
        tk[e] = kn * (ie * een[e]);                   // K^ exp(end_w - G) <= 1
        kp[e] = tk[e] * cc2[e];                       // K^ exp(G_L - G)   <= 1
        kg[e] = rke[e] * exr[e];                      // K^ exp(G)         <= 1
        qg[e] = rqe[e] * exr[e];                      // Q^ exp(G)         <= 1
      }
      Rkd[s] = pk_bf16(rke);
      Ckd[s] = pk_bf16(cki);
      Rqd[s] = pk_bf16(rqe);
      Rkh[s] = pk_f16(rke);
      Rqh[s] = pk_f16(rqe);
      if (w >= 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { t2[e] = rke[e] * d2[e]; t3[e] = rqe[e] * d2[e]; }
        Rkh2[s] = pk_f16(t2);
        Rqh2[s] = pk_f16(t3);
      } else {
        Rkh2[s] = Rqh2[s] = u32x4{0u, 0u, 0u, 0u};
      }
      if (w >= 3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { t2[e] = rke[e] * d3[e]; t3[e] = rqe[e] * d3[e]; }
        Rkh3[s] = pk_f16(t2);
        Rqh3[s] = pk_f16(t3);
      } else {
        Rkh3[s] = Rqh3[s] = u32x4{0u, 0u, 0u, 0u};
      }
      sm.tk[w][s][l] = pk_f16(tk);
      *reinterpret_cast<u32x4*>(rec + OFF_QG + ((w * 4 + s) * 64 + l) * 16) = pk_f16(qg);
      unpack8(vraw[s], vf);
      (void)vf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = chan(s, e, gq);
        sm.u.kpt[c][tok] = to_f16(kp[e]);
        sm.kgt[c][tok] = to_f16(kg[e]);
      }
      const uint32_t vv[4] = {vraw[s].x, vraw[s].y, vraw[s].z, vraw[s].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = chan(s, e, gq);
        sm.vt[c][tok] = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu));
      }
    }
  }

  // diagonal gram blocks need only this wave's fragments
  f32x4 aD = {0, 0, 0, 0}, qD = {0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aD = mfma_bf16(Rkd[s], Ckd[s], aD);   // D[r][i] = k^_r.k^_i exp(Gs_r - Gs_i)
    qD = mfma_bf16(Ckd[s], Rqd[s], qD);   // D[i][r] = k^_i.q^_r exp(Gs_r - Gs_i)
  }
  __syncthreads();

  // ---------------- phase D: K'^T out, off-diagonal grams, A and Aqk --------
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int fi = 4 * w + f, mt = fi >> 1, s = fi & 1, c = 16 * mt + lt;
    const u32x2 a = *reinterpret_cast<const u32x2*>(&sm.u.kpt[c][32 * s + 4 * gq]);
    const u32x2 b = *reinterpret_cast<const u32x2*>(&sm.u.kpt[c][32 * s + 16 + 4 * gq]);
    *reinterpret_cast<u32x4*>(rec + OFF_KP + (fi * 64 + l) * 16) = u32x4{a.x, a.y, b.x, b.y};
  }
  f32x4 aO[3], qO[3];   // off-diagonal blocks by distance 1..3
#pragma unroll
  for (int d = 0; d < 3; ++d) aO[d] = qO[d] = f32x4{0, 0, 0, 0};
  if (w >= 1) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 tb = sm.tk[w - 1][s][l];
      aO[0] = mfma_f16(Rkh[s], tb, aO[0]);
      qO[0] = mfma_f16(tb, Rqh[s], qO[0]);
    }
  }
  if (w >= 2) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 tb = sm.tk[w - 2][s][l];
      aO[1] = mfma_f16(Rkh2[s], tb, aO[1]);
      qO[1] = mfma_f16(tb, Rqh2[s], qO[1]);
    }
  }
  if (w >= 3) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 tb = sm.tk[0][s][l];
      aO[2] = mfma_f16(Rkh3[s], tb, aO[2]);
      qO[2] = mfma_f16(tb, Rqh3[s], qO[2]);
    }
  }
  __syncthreads();   // all reads of kpt and tk are done: A may overwrite kpt

  {
    // rows r = 16w + 4gq + j, columns i = 16b + lt
    const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.beta[16 * w + 4 * gq]);
    const float bj[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * gq + j;
      sm.u.A[16 * w + r][16 * w + lt] = (r > lt) ? bj[j] * aD[j] : 0.0f;
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      if (w >= d + 1) {
        const int b = w - 1 - d;
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.u.A[16 * w + 4 * gq + j][16 * b + lt] = bj[j] * aO[d][j];
      }
    }
    // Aqk^T blocks: lane <-> query r = lt (tile w), registers <-> keys 16b + 4gq + j.
    // Fragment (tile w, k-step b>>1) half (b&1). Diagonal block keeps keys <= query.
    const float s0 = 0.0f;
    {
      float dq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) dq[j] = (4 * gq + j <= lt) ? qD[j] : s0;
      uint8_t* fr = rec + OFF_AQK + ((w * 2 + (w >> 1)) * 64 + l) * 16 + (w & 1) * 8;
      *reinterpret_cast<u32x2*>(fr) = u32x2{pack_f16x2(dq[0], dq[1]), pack_f16x2(dq[2], dq[3])};
      if ((w & 1) == 0) {   // keys of sub-chunk w+1 lie above the diagonal: zero half
        *reinterpret_cast<u32x2*>(fr + 8) = u32x2{0u, 0u};
      }
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      if (w >= d + 1) {
        const int b = w - 1 - d;
        uint8_t* fr = rec + OFF_AQK + ((w * 2 + (b >> 1)) * 64 + l) * 16 + (b & 1) * 8;
        *reinterpret_cast<u32x2*>(fr) = u32x2{pack_f16x2(qO[d][0], qO[d][1]), pack_f16x2(qO[d][2], qO[d][3])};
      }
    }
  }
  __syncthreads();

  // ---------------- phase E: Tm = (I + A)^-1 in place (fp32) -----------------
  {
    // (a) diagonal 16x16 blocks: lane (any group) solves column lt of block w
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == lt) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int m4 = 0; m4 < i; m4 += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.u.A[16 * w + i][16 * w + m4]);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m4 + u < i) acc += av[u] * x[m4 + u];
      }
      if (i > lt) x[i] = -acc;
    }
    if (gq == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.u.A[16 * w + i][16 * w + lt] = x[i];
    }
  }
  __syncthreads();
  {
    float* X = reinterpret_cast<float*>(&sm.tk[0][0][0]);   // [3][16][16] scratch
    // (b) block rows a = 1..3: X_b = sum_{m=b}^{a-1} A_am Tm_mb ; Tm_ab = -Tm_aa X_b
    for (int a = 1; a < 4; ++a) {
      if (w < a) {
        const int b = w;
        float xr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int m = b; m < a; ++m) {
#pragma unroll
          for (int k4 = 0; k4 < 16; k4 += 4) {
            const float t0v = sm.u.A[16 * m + k4 + 0][16 * b + lt];
            const float t1v = sm.u.A[16 * m + k4 + 1][16 * b + lt];
            const float t2v = sm.u.A[16 * m + k4 + 2][16 * b + lt];
            const float t3v = sm.u.A[16 * m + k4 + 3][16 * b + lt];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.u.A[16 * a + 4 * gq + rr][16 * m + k4]);
              xr[rr] += a4.x * t0v + a4.y * t1v + a4.z * t2v + a4.w * t3v;
            }
          }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) X[(b * 16 + 4 * gq + rr) * 16 + lt] = xr[rr];
      }
      __syncthreads();
      if (w < a) {
        const int b = w;
        float tr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k4 = 0; k4 < 16; k4 += 4) {
          const float x0 = X[(b * 16 + k4 + 0) * 16 + lt];
          const float x1 = X[(b * 16 + k4 + 1) * 16 + lt];
          const float x2 = X[(b * 16 + k4 + 2) * 16 + lt];
          const float x3 = X[(b * 16 + k4 + 3) * 16 + lt];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.u.A[16 * a + 4 * gq + rr][16 * a + k4]);
            tr[rr] += a4.x * x0 + a4.y * x1 + a4.z * x2 + a4.w * x3;
          }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sm.u.A[16 * a + 4 * gq + rr][16 * b + lt] = -tr[rr];
      }
      __syncthreads();
    }
  }

  // ---------------- phase F: W = Tm diag(beta) K^.Gamma,  U~ = Tm diag(beta) V
  {
    const int t = 16 * w + lt;
    const int smax = (w >= 2) ? 1 : 0;
    f32x4 accW[8], accU[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) accW[i] = accU[i] = f32x4{0, 0, 0, 0};
    for (int s = 0; s <= smax; ++s) {
      const int m0 = 32 * s + 8 * gq;
      const f32x4 r0 = *reinterpret_cast<const f32x4*>(&sm.u.A[t][m0]);
      const f32x4 r1 = *reinterpret_cast<const f32x4*>(&sm.u.A[t][m0 + 4]);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&sm.beta[m0]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&sm.beta[m0 + 4]);
      const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float val[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = (m0 + e <= t) ? rv[e] * bv[e] : 0.0f;
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
      for (int mt = 0; mt < 8; ++mt) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&sm.kgt[16 * mt + lt][m0]);
        accW[mt] = mfma_f16(ka, tmh, accW[mt]);          // D[c][t]
      }
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) {
        const u32x4 vb = *reinterpret_cast<const u32x4*>(&sm.vt[16 * vt + lt][m0]);
        accU[vt] = mfma_bf16(hi, vb, accU[vt]);          // D[t][v]
        accU[vt] = mfma_bf16(lov, vb, accU[vt]);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 a = accW[2 * s], b = accW[2 * s + 1];
      *reinterpret_cast<u32x4*>(rec + OFF_WNEG + ((w * 4 + s) * 64 + l) * 16) =
          u32x4{pack_f16x2(-a.x, -a.y), pack_f16x2(-a.z, -a.w), pack_f16x2(-b.x, -b.y), pack_f16x2(-b.z, -b.w)};
    }
#pragma unroll
    for (int vt = 0; vt < 8; ++vt)
      *reinterpret_cast<f32x4*>(rec + OFF_UT + ((vt * 4 + w) * 64 + l) * 16) = accU[vt];
  }
}

}  // namespace

hipError_t launch_intra(const FwdParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.map.max_chunks * p.H;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(kda_intra_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
