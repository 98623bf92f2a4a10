/*
 * kda_oracle.c -- plain fp64 CPU reference for the Kimi Delta Attention (KDA)
 * forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this code. The GPU product path never
 * links, imports or calls it, and it shares no code, header or table with the
 * GPU path: the only thing both sides share is the seeded input generator.
 *
 * What it computes (one independent chain per sequence n and head h):
 *
 *   KDA is Gated DeltaNet with a finer, per-channel gate ("FlashKDA ... CUDA
 *   加速實作", section 背景).  The pages print no equation, so this file takes
 *   the plain gated delta-rule recurrence with a per-key-channel decay:
 *
 *     S      : V x K state, row v, column c (K contiguous), fp64
 *     q^, k^ = q / sqrt(sum q^2 + 1e-6), k / sqrt(sum k^2 + 1e-6)   (over K)
 *     beta_t = 1 / (1 + exp(-b_t))                 (beta logits, sigmoid in-kernel)
 *     gt[c]  = lower_bound * sigmoid(exp(A_log[h]) * (g_t[c] + dt_bias[h][c]))
 *     S      = S * Diag(exp(gt))                    (decay the K columns)
 *     S      = S - beta_t * (S k^ - v_t) k^^T       (delta update)
 *     o_t    = scale * S q^                         (read the updated state)
 *
 *   Parameter roles, shapes and dtypes follow the "Kernel API" table of the
 *   FlashKDA README digest (aiwatch.icu page): q, k, g [B,T,H,K] bf16,
 *   v [B,T,H,V] bf16, beta [B,T,H] bf16 logits with the sigmoid applied
 *   inside, A_log fp32 [H] (log of the gate rate), dt_bias fp32 [H,K] (an
 *   offset added to g), lower_bound in [-5, 0] (the gate's floor), state [B|N,H,V,K],
 *   cu_seqlens int64 [N+1] with B = 1 and T the packed total length; without
 *   cu_seqlens every batch row is an independent sequence.
 *
 *   Readings where the pages are silent: the gate form above (the pages name
 *   only its three parameters), natural exp, an L2-norm epsilon of 1e-6 inside
 *   the square root, scale applied to the read-out, and decay -> delta update
 *   -> read-out in that order.
 *
 *   Fusion switches (the use_gate_in_kernel, use_qk_l2norm_in_kernel and
 *   use_beta_sigmoid_in_kernel switches of page "FlashKDA：面向SM90+的高性能KDA
 *   CUDA内核库", Q4). With a switch off the kernel takes that input already
 *   processed (our reading, the plainest one):
 *     gate off : gt[c] = g_t[c] itself, clamped into [lower_bound, 0] (the range
 *                the safe gate bound guarantees for the in-kernel activation);
 *                A_log and dt_bias are unused
 *     norm off : q^, k^ = q, k as given
 *     beta off : beta_t = b_t as given
 *
 *   Gate without the safe bound (the safe_gate switch of the same page, Q4,
 *   turned off). Our reading: the gate is then the plain softplus log-decay,
 *   not bounded below, and lower_bound is not used:
 *     gate on  : gt[c] = -exp(A_log[h]) * softplus(g_t[c] + dt_bias[h][c]),
 *                softplus(x) = log(1 + exp(x))
 *     gate off : gt[c] = min(g_t[c], 0)
 *
 * Inputs are taken in their storage formats (bf16 as raw uint16 bits, fp32) and
 * widened exactly to fp64; every operation is done in fp64.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* switch bits (fusion bits all set and the unbounded bit clear: the fully fused kernel) */
enum { ORACLE_FUSE_GATE = 1, ORACLE_FUSE_QK_L2NORM = 2, ORACLE_FUSE_BETA_SIGMOID = 4,
       ORACLE_GATE_UNBOUNDED = 8 };

/* log(1 + exp(x)) without overflow for large x */
static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* state dtype codes for initial_state */
enum { ORACLE_STATE_NONE = 0, ORACLE_STATE_BF16 = 1, ORACLE_STATE_FP32 = 2, ORACLE_STATE_FP64 = 3 };

static double load_state(const void *p, int dtype, size_t i)
{
    switch (dtype) {
    case ORACLE_STATE_BF16: return bf16_bits_to_double(((const uint16_t *)p)[i]);
    case ORACLE_STATE_FP32: return (double)((const float *)p)[i];
    case ORACLE_STATE_FP64: return ((const double *)p)[i];
    default: return 0.0;
    }
}

/*
 * One chain: tokens [t_begin, t_end) of the packed token axis, head h.
 * S (V*K doubles) must hold the initial state on entry; it holds the final
 * state on return.  out_row(t) = out + (t*nh + hi)*V.
 */
static void run_chain(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *beta, double scale, const float *A_log, const float *dt_bias,
                      double lower_bound, int64_t H, int64_t K, int64_t V, int64_t h,
                      int64_t t_begin, int64_t t_end, int64_t nh, int64_t hi, int flags,
                      double *S, double *out, double *work)
{
    double *qh = work, *kh = work + K, *alpha = work + 2 * K;
    const double rate = (flags & ORACLE_FUSE_GATE) ? exp((double)A_log[h]) : 0.0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        const size_t row = (size_t)t * (size_t)H + (size_t)h;
        const uint16_t *qt = q + row * (size_t)K, *kt = k + row * (size_t)K;
        const uint16_t *gt = g + row * (size_t)K, *vt = v + row * (size_t)V;

        /* L2-normalise q and k over the K channels (norm switch on) */
        double qs = 0.0, ks = 0.0;
        for (int64_t c = 0; c < K; ++c) {
            qh[c] = bf16_bits_to_double(qt[c]);
            kh[c] = bf16_bits_to_double(kt[c]);
            qs += qh[c] * qh[c];
            ks += kh[c] * kh[c];
        }
        if (flags & ORACLE_FUSE_QK_L2NORM) {
            const double qn = sqrt(qs + 1e-6), kn = sqrt(ks + 1e-6);
            for (int64_t c = 0; c < K; ++c) {
                qh[c] /= qn;
                kh[c] /= kn;
            }
        }

        /* beta = sigmoid(logit) (beta switch on) or the given value */
        const double braw = bf16_bits_to_double(beta[row]);
        const double b = (flags & ORACLE_FUSE_BETA_SIGMOID) ? sigmoid(braw) : braw;

        /* per-channel gate, then the decay factor exp(gate) */
        for (int64_t c = 0; c < K; ++c) {
            double gate;
            const int unbounded = (flags & ORACLE_GATE_UNBOUNDED) != 0;
            if (flags & ORACLE_FUSE_GATE) {
                const double x = bf16_bits_to_double(gt[c]) + (double)dt_bias[h * K + c];
                gate = unbounded ? -rate * softplus(x) : lower_bound * sigmoid(rate * x);
            } else {
                gate = bf16_bits_to_double(gt[c]);
                gate = gate > 0.0 ? 0.0 : gate;
                if (!unbounded && gate < lower_bound)
                    gate = lower_bound;
            }
            alpha[c] = exp(gate);
        }

        /* S = S Diag(alpha);  S = S - b (S k^ - v) k^^T;  o = scale S q^ */
        for (int64_t r = 0; r < V; ++r) {
            double *Sr = S + (size_t)r * (size_t)K;
            for (int64_t c = 0; c < K; ++c)
                Sr[c] *= alpha[c];
            double sk = 0.0;
            for (int64_t c = 0; c < K; ++c)
                sk += Sr[c] * kh[c];
            const double u = b * (sk - bf16_bits_to_double(vt[r]));
            for (int64_t c = 0; c < K; ++c)
                Sr[c] -= u * kh[c];
            double o = 0.0;
            for (int64_t c = 0; c < K; ++c)
                o += Sr[c] * qh[c];
            out[((size_t)t * (size_t)nh + (size_t)hi) * (size_t)V + (size_t)r] = scale * o;
        }
    }
}

/*
 * kda_oracle_fwd -- returns 0 on success, nonzero on bad arguments.
 *
 *   q, k, g      : bf16 bits, [B*T][H][K]
 *   v            : bf16 bits, [B*T][H][V]
 *   beta         : bf16 bits, [B*T][H]
 *   A_log        : fp32 [H];  dt_bias : fp32 [H][K]
 *   initial_state: NULL or [nseq][H][V][K] in dtype state_dtype (codes above)
 *   final_state  : NULL or fp64 [nseq][nh][V][K]
 *   out          : fp64 [B*T][nh][V]
 *   cu_seqlens   : NULL (nseq = B, rows of length T) or int64 [N+1] (B must be 1)
 *   heads        : NULL (all H heads, nh must equal H) or int32 [nh] head ids
 *   nthreads     : OpenMP threads (<= 0: runtime default)
 *   flags        : ORACLE_FUSE_* bits (7 = fully fused) and ORACLE_GATE_UNBOUNDED;
 *                  A_log and dt_bias may be NULL when ORACLE_FUSE_GATE is clear
 */
int kda_oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                   const uint16_t *beta, double scale, const float *A_log, const float *dt_bias,
                   double lower_bound, const void *initial_state, int state_dtype,
                   double *final_state, double *out, const int64_t *cu_seqlens, int64_t N,
                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, const int32_t *heads,
                   int64_t nh, int nthreads, int flags)
{
    if (!q || !k || !v || !g || !beta || !out)
        return 1;
    if ((flags & ~15) != 0)
        return 2;
    if ((flags & ORACLE_FUSE_GATE) && (!A_log || !dt_bias))
        return 1;
    if (B < 1 || T < 0 || H < 1 || K < 1 || V < 1 || nh < 1)
        return 2;
    if (cu_seqlens && (B != 1 || N < 1))
        return 2;
    if (!heads && nh != H)
        return 2;
    const int64_t nseq = cu_seqlens ? N : B;
    const int64_t nchains = nseq * nh;
    int bad = 0;

#pragma omp parallel num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(V * K));
        double *work = (double *)malloc(sizeof(double) * (size_t)(3 * K));
#pragma omp for schedule(dynamic, 1)
        for (int64_t idx = 0; idx < nchains; ++idx) {
            const int64_t n = idx / nh, hi = idx % nh;
            const int64_t h = heads ? (int64_t)heads[hi] : hi;
            if (h < 0 || h >= H || !S || !work) {
#pragma omp atomic write
                bad = 3;
                continue;
            }
            int64_t t0, t1;
            if (cu_seqlens) {
                t0 = cu_seqlens[n];
                t1 = cu_seqlens[n + 1];
                if (t0 < 0 || t1 < t0 || t1 > T) {
#pragma omp atomic write
                    bad = 4;
                    continue;
                }
            } else {
                t0 = n * T;
                t1 = t0 + T;
            }
            for (int64_t i = 0; i < V * K; ++i)
                S[i] = initial_state
                           ? load_state(initial_state, state_dtype,
                                        ((size_t)n * (size_t)H + (size_t)h) * (size_t)(V * K) + (size_t)i)
                           : 0.0;
            run_chain(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, H, K, V, h, t0, t1, nh,
                      hi, flags, S, out, work);
            if (final_state)
                memcpy(final_state + ((size_t)n * (size_t)nh + (size_t)hi) * (size_t)(V * K), S,
                       sizeof(double) * (size_t)(V * K));
        }
        free(S);
        free(work);
    }
    return bad;
}
