/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library
 * (libkda.so).
 *
 * The operation (per sequence n and head h, state S of V x K, K contiguous):
 *   q^, k^ = L2-normalised q, k over K (x / sqrt(sum x^2 + 1e-6))
 *   beta   = sigmoid(beta logit)
 *   g~[c]  = lower_bound * sigmoid(exp(A_log[h]) * (g[c] + dt_bias[h][c]))
 *   S      = S * Diag(exp(g~));  S = S - beta (S k^ - v) k^^T;  o = scale * S q^
 * KDA is Gated DeltaNet with a per-channel gate (page "FlashKDA：基於 CUTLASS
 * 的 Kimi Delta Attention CUDA 加速實作", section 背景). The pages print no
 * equation; the gate form, natural exp, the 1e-6 epsilon and the order
 * decay -> delta update -> read-out are this library's stated readings.
 *
 * The argument list mirrors flash_kda.fwd(q, k, v, g, beta, scale, out,
 * A_log, dt_bias, lower_bound, initial_state, final_state, cu_seqlens) and its
 * parameter table ("Kernel API" of the FlashKDA README digest, aiwatch.icu
 * page), with the caller-owned, written-in-place `out` of the 2kiu.com guide
 * (sections 一 and 三).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or from a caching
 *     allocator), row-major and contiguous, aligned to 16 bytes (the state
 *     and fp32 parameters to 16 bytes as well).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are stream-ordered and asynchronous: they return as soon as the
 *     work is enqueued. The library allocates nothing per call and keeps no
 *     pointer after it returns; it is reentrant.
 *   - Errors are detected on the host before anything is launched; on error
 *     nothing is written. cu_seqlens CONTENTS live on the device and are a
 *     caller precondition (cu[0] = 0, non-decreasing, cu[N] = T); the kernels
 *     clamp every sequence into [0, T] so malformed contents cannot make them
 *     access memory out of bounds (results are then unspecified). Setting the
 *     environment variable KDA_VALIDATE=1 makes kda_fwd synchronise the stream
 *     and check the contents on the host (KDA_ERR_VALUE if violated).
 *   - Other environment variables: KDA_LOG=1 prints each kda_fwd call's sizes
 *     and chain segment count to stderr; KDA_CHAIN_SEGMENTS=n caps the number
 *     of segments of the segment-parallel state chain (see
 *     kda_fwd_workspace_size; 1 keeps the plain chain).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,      /* a required pointer is NULL                           */
    KDA_ERR_SHAPE = 2,     /* K != 128, V != 128, H < 1, T < 0, B < 1, B != 1 with
                              cu_seqlens, N < 1 with cu_seqlens, size overflow      */
    KDA_ERR_DTYPE = 3,     /* unknown state dtype code, or initial and final state
                              given with different dtypes                           */
    KDA_ERR_VALUE = 4,     /* lower_bound outside [-5, 0] or not finite (safe gate),
                              scale not finite, unknown flag bits, bad cu_seqlens
                              contents (KDA_VALIDATE=1 only)                        */
    KDA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                      */
    KDA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than kda_fwd_workspace_min */
    KDA_ERR_HIP = 7,       /* a HIP runtime call or kernel launch failed            */
    KDA_ERR_CAPACITY = 8   /* kda_fwd_noalloc: the call needs more workspace than
                              its fixed device array holds (KDA_NOALLOC_CAPACITY)   */
};

/*
 * Fusion switches of kda_fwd_ex / kda_fwd_recurrent_ex (the use_gate_in_kernel,
 * use_qk_l2norm_in_kernel and use_beta_sigmoid_in_kernel switches of page
 * "FlashKDA：面向SM90+的高性能KDA CUDA内核库", Q4). A set bit runs that input
 * processing inside the kernels; with a bit clear the input is taken as
 * already processed (this library's reading):
 *   KDA_FUSE_GATE clear          g holds the log-decay g~ itself (bf16), which
 *                                is clamped into [lower_bound, 0]; A_log and
 *                                dt_bias are unused and may be NULL
 *   KDA_FUSE_QK_L2NORM clear     q and k are used as given (expected unit norm)
 *   KDA_FUSE_BETA_SIGMOID clear  beta holds beta itself (expected in [0, 1])
 * KDA_GATE_UNBOUNDED is the safe_gate switch of the same page turned off. The
 * safe gate (bit clear) is the lower_bound form documented at kda_fwd; with the
 * bit set the gate is the plain softplus log-decay, not bounded below, and
 * lower_bound is neither used nor checked (this library's reading):
 *   KDA_FUSE_GATE set            g~ = -exp(A_log[h]) * log(1 + exp(g + dt_bias[h]))
 *   KDA_FUSE_GATE clear          g~ = min(g, 0)
 * Chunks whose 16-token gate sums stay above -80 (natural log) take the same
 * kernel path as the safe gate; others compute their diagonal 16x16 decay
 * blocks pairwise, which costs extra vector work for those chunks only.
 * kda_fwd and kda_fwd_recurrent are the KDA_FUSE_ALL case (safe gate).
 */
enum kda_fuse_flags {
    KDA_FUSE_GATE = 1,
    KDA_FUSE_QK_L2NORM = 2,
    KDA_FUSE_BETA_SIGMOID = 4,
    KDA_FUSE_ALL = 7,
    KDA_GATE_UNBOUNDED = 8,
    KDA_PATH_CHUNKED = 16   /* kda_fwd_ex only: never hand a short call to the
                               token-recurrent kernel (see kda_fwd)             */
};

/* State dtype codes for initial_state / final_state. */
enum kda_state_dtype {
    KDA_STATE_NONE = 0,    /* pointer must be NULL (stateless)  */
    KDA_STATE_BF16 = 1,    /* bfloat16, rounded to nearest-even */
    KDA_STATE_FP32 = 2     /* float32                           */
};

/*
 * kda_fwd_workspace_size -- bytes of device workspace kda_fwd needs.
 *   B, T, H: as for kda_fwd;  N: number of sequences when cu_seqlens is used,
 *   0 otherwise. Returns 0 for invalid sizes (B < 1, T < 0, H < 1, N < 0).
 * The workspace holds the per-chunk intermediates of the chunked (WY) form
 * (74.5 KiB per 64-token chunk and head) and the varlen chunk tables. With few
 * (row or sequence, head) pairs on long rows it also holds the buffers of the
 * segment-parallel state chain: each row's or sequence's chunks are cut into s
 * segments (s chosen from B or N, T and H), with 192 KiB per (row or sequence,
 * segment, head) for the segments' affine maps and initial states.
 * Calls whose full workspace would exceed 4 GiB and that use the plain chain
 * get the size of a windowed run within 4 GiB instead (see
 * kda_fwd_workspace_min; at B = 4, T = 32768, H = 64 that takes the same time
 * as the full 9.5 GiB).
 */
size_t kda_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t N);

/*
 * kda_fwd_workspace_min -- the smallest workspace kda_fwd / kda_fwd_ex accept for
 * the same call (same arguments and invalid-size rule as kda_fwd_workspace_size).
 * Calls given less than kda_fwd_workspace_size run in windows, each the
 * intra-chunk pass and the state chain over part of the chunks:
 *   - fixed length (N = 0): chunk columns jb .. jb + w - 1 of every row, with
 *     each row's state carried to the next window in fp32 (in final_state itself
 *     when that is fp32, else in the workspace: 64 KiB per (row, head)); the
 *     minimum holds one chunk column (B * H records of 74.5 KiB) and the carry;
 *   - varlen (N > 0): w consecutive chunk slots of the packed sequences, a
 *     sequence that crosses a window boundary carrying its state in fp32 through
 *     one of two carry slots (64 KiB per head each); the minimum holds the
 *     scheduler's tables, the carry slots and one slot of H records.
 * Windowed calls return the same bits as unwindowed ones; they take more kernel
 * launches and skip the segment-parallel chain.
 */
size_t kda_fwd_workspace_min(int64_t B, int64_t T, int64_t H, int64_t N);

/*
 * kda_fwd -- chunked KDA prefill forward (64-token chunks).
 *
 *   q, k, g      bf16 [B, T, H, K]   query, key, raw gate input (activated inside)
 *   v            bf16 [B, T, H, V]   value
 *   beta         bf16 [B, T, H]      beta logits (sigmoid applied inside)
 *   scale        float               read-out scaling factor (finite)
 *   out          bf16 [B, T, H, V]   OUTPUT, written in place; every element
 *                                    is written, none is read (no need to
 *                                    pre-zero it)
 *   A_log        fp32 [H]            log of each head's gate rate
 *   dt_bias      fp32 [H, K]         per-channel offset added to g
 *   lower_bound  float in [-5, 0]    most negative value the gate can take
 *   initial_state, initial_dtype     NULL/KDA_STATE_NONE (zeros) or
 *                                    [B|N, H, V, K] bf16/fp32
 *   final_state, final_dtype         NULL/KDA_STATE_NONE (not written) or
 *                                    [B|N, H, V, K] bf16/fp32, written for every
 *                                    (sequence, head), zero-length sequences
 *                                    included. May alias initial_state.
 *   cu_seqlens   int64 [N+1] or NULL packed sequence boundaries; requires
 *                                    B == 1 and T the total packed length.
 *                                    Without it, each of the B rows is an
 *                                    independent sequence of length T.
 *   N            number of sequences (ignored without cu_seqlens)
 *   B, T, H, K, V                    sizes; K and V must be 128. T may be 0:
 *                                    then q, k, v, g, beta and out hold no
 *                                    element and may be NULL, and the call
 *                                    only writes final_state (the initial
 *                                    state, or zeros, for every sequence)
 *   workspace, workspace_bytes       caller-owned device scratch of at least
 *                                    kda_fwd_workspace_min(B, T, H, N) bytes
 *                                    (run in windows when below
 *                                    kda_fwd_workspace_size), 256-byte aligned;
 *                                    its contents need no initialisation and
 *                                    are clobbered
 *   stream       hipStream_t as void*
 * Returns a kda_status.
 *
 * Decode-sized calls run on the token-recurrent kernel of kda_fwd_recurrent,
 * which computes the same operation without the chunked form's fixed cost of
 * one 64-token chunk per (sequence, head): fixed-length calls with T <= 8, and
 * varlen calls with T <= 2 N (at most two tokens per sequence on average; the
 * lengths themselves stay on the device). The workspace rules are unchanged.
 * kda_fwd_ex with KDA_PATH_CHUNKED keeps such calls on the chunked kernels.
 */
int kda_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
            float scale, void *out, const float *A_log, const float *dt_bias, float lower_bound,
            const void *initial_state, int initial_dtype, void *final_state, int final_dtype,
            const int64_t *cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K,
            int64_t V, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_fwd_recurrent -- the same operation computed token by token (one
 * workgroup per sequence and head, fp32 state in registers). Same arguments
 * and rules as kda_fwd, without a workspace. It is the path for online
 * generation with state passing (decode-sized T; page "FlashKDA：面向SM90+的
 * 高性能KDA CUDA内核库", Q2 on stateful/streaming use) and a reference for the
 * chunked path on long inputs.
 */
int kda_fwd_recurrent(const void *q, const void *k, const void *v, const void *g,
                      const void *beta, float scale, void *out, const float *A_log,
                      const float *dt_bias, float lower_bound, const void *initial_state,
                      int initial_dtype, void *final_state, int final_dtype,
                      const int64_t *cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H,
                      int64_t K, int64_t V, void *stream);

/*
 * kda_fwd_ex, kda_fwd_recurrent_ex -- kda_fwd / kda_fwd_recurrent with the
 * switches in `flags` (KDA_FUSE_* bits, KDA_GATE_UNBOUNDED and, for kda_fwd_ex,
 * KDA_PATH_CHUNKED; other bits: KDA_ERR_VALUE). Every other argument and rule is that of the plain entry
 * point, except that A_log and dt_bias may be NULL when KDA_FUSE_GATE is
 * clear, and lower_bound is ignored when KDA_GATE_UNBOUNDED is set.
 */
int kda_fwd_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
               float scale, void *out, const float *A_log, const float *dt_bias, float lower_bound,
               const void *initial_state, int initial_dtype, void *final_state, int final_dtype,
               const int64_t *cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K,
               int64_t V, uint32_t flags, void *workspace, size_t workspace_bytes, void *stream);
int kda_fwd_recurrent_ex(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, float scale, void *out, const float *A_log,
                         const float *dt_bias, float lower_bound, const void *initial_state,
                         int initial_dtype, void *final_state, int final_dtype,
                         const int64_t *cu_seqlens, int64_t N, int64_t B, int64_t T, int64_t H,
                         int64_t K, int64_t V, uint32_t flags, void *stream);

/*
 * kda_fwd_noalloc -- kda_fwd_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The same operation, arguments, switches, rules and errors as
 * kda_fwd_ex, without the workspace arguments: the workspace is a fixed array
 * of KDA_NOALLOC_CAPACITY bytes in device memory that the library holds on
 * every GPU it runs on, from its first use there until the process ends. The
 * call itself allocates nothing and issues no memset or copy.
 *   - Calls whose full workspace exceeds the capacity run in windows (see
 *     kda_fwd_workspace_min); calls whose kda_fwd_workspace_min(B, T, H, N)
 *     exceeds it (fixed length: B * H beyond about 1,890; varlen: H beyond
 *     about 1,300 at moderate T and N) are rejected on the host with
 *     KDA_ERR_CAPACITY, before anything is launched. Decode-sized calls need
 *     no workspace at all.
 *   - The array of the CURRENT device is used: `stream` must belong to it.
 *     The array's device address is looked up once per device, on the first
 *     call there (KDA_ERR_HIP if that fails).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind; nothing in it needs clearing (each call writes every word it
 *     reads). Calls that overlap on one device (several streams or host
 *     threads) RACE on the array: the caller must serialise them.
 * kda_noalloc_capacity() returns KDA_NOALLOC_CAPACITY.
 */
#define KDA_NOALLOC_CAPACITY ((size_t)256 << 20)
int kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    float scale, void *out, const float *A_log, const float *dt_bias,
                    float lower_bound, const void *initial_state, int initial_dtype,
                    void *final_state, int final_dtype, const int64_t *cu_seqlens, int64_t N,
                    int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, uint32_t flags,
                    void *stream);
size_t kda_noalloc_capacity(void);

/* kda_status_string -- static description of a status code (never NULL). */
const char *kda_status_string(int status);

/* kda_version -- library version string, e.g. "0.1.0 gfx950". */
const char *kda_version(void);

/*
 * Per-kernel timing of kda_fwd (a measurement hook; results are unchanged).
 *
 * kda_profile_start(max_calls): from now on, each of the next max_calls
 *   kda_fwd calls records HIP events on its stream before its first kernel and
 *   after each kernel (the events are created here, not per call, with
 *   hipEventDisableSystemFence: they only measure time and add no cache
 *   write-back to the timed work, so they must not be used to order anything
 *   with the host or other devices). Calls
 *   beyond max_calls are not timed. Starting again discards earlier recordings.
 *   Returns KDA_ERR_VALUE unless 1 <= max_calls <= 65536, KDA_ERR_HIP if an
 *   event cannot be created.
 * kda_profile_stop(total_ms, launches, n_kernels): waits for the recorded
 *   events and writes, for each kernel i < kda_profile_kernel_count(), the
 *   summed milliseconds over the timed calls into total_ms[i] and the number
 *   of timed calls that launched it into launches[i] (host arrays of
 *   n_kernels >= the kernel count); then stops timing and frees the events.
 *   Returns KDA_ERR_NULL, KDA_ERR_SHAPE (n_kernels too small), KDA_ERR_VALUE
 *   (timing not started) or KDA_ERR_HIP.
 * kda_profile_kernel_name(i): static name of kernel i ("" when out of range).
 * One interval runs from one event to the next on the same stream: the
 * kernel's execution plus its launch gap.
 */
int kda_profile_start(int max_calls);
int kda_profile_stop(double *total_ms, int *launches, int n_kernels);
int kda_profile_kernel_count(void);
const char *kda_profile_kernel_name(int i);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
