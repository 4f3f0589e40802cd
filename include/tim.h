/*
 * tim.h — batch-invariant selected-token log-probabilities and
 * training/rollout mismatch ("TIM") statistics for AMD Instinct MI355X
 * (gfx950).  C ABI of libtim.so.
 *
 * What is computed (sources are the pages this library follows; each entry
 * point below names the passage that defines it):
 *
 *   logits  z[t,v] = sum_k h[t,k] * W[v,k]           (LM head, no bias)
 *   logp[t]        = z[t, a_t] - log sum_v exp z[t,v] (log-softmax + gather)
 *
 *     "RL: Training Inference Mismatch", section "log p": the chain
 *     final hidden states -> LM head -> logits -> log-softmax -> gather of
 *     the realised token id, and its PyTorch rendering with log_softmax and
 *     gather along the vocabulary axis.
 *
 *   delta_t = logp_train[t] - logp_rollout[t],  r_t = exp(delta_t),
 *   k1 = -delta, k2 = delta^2 / 2, k3 = (r - 1) - delta,
 *   token-level truncated IS weight, per-sequence geometric-mean-ratio
 *   rejection and the batch monitoring aggregates.
 *
 *     "Diagnosing Training Inference Mismatch in LLM Reinforcement Learning
 *     (VeXact)", eq. (1) (token-level TIM), the K1/K3 estimators and the
 *     "Algorithmic TIM Compensation Results" table (TIS and r_corr-based
 *     sequence rejection); "训推一致性与 determinism" (LLM Infra Atlas),
 *     section 2 (Delta_t and r_t = e^Delta_t); "RL: Training Inference
 *     Mismatch", section on the three KL estimators and the monitoring
 *     flow (per-token KL, mean per completion, mean over the batch);
 *     "Train-Inference Consistency" (LoongSage), section 5 (metric names
 *     is_approx_k3_kl, is_clip_ratio, is_nan_ratio) and section 4 (IS
 *     correction clips out-of-bound weights).
 *
 * Determinism contract.  For one build and one device, every output bit of
 * tim_logprob_forward for row t depends only on (h[t,:], W, a_t, V, D,
 * dtype, flags): not on N, not on the row's position in the batch and not
 * on the other rows ("训推一致性与 determinism", section 1.2, batch
 * invariance).  Repeated calls return identical bits (same page, 1.1).
 * The per-sequence outputs of tim_mismatch_stats depend only on that
 * sequence's tokens; batch aggregates are reduced in a fixed order.
 *
 * Memory.  Every pointer is DEVICE memory unless marked (host).  The caller
 * owns every buffer; no call allocates device memory and none keeps a
 * pointer after it returns.  Scratch memory is passed in as a workspace
 * whose size is returned by the *_workspace_bytes query.  The one exception,
 * tim_logprob_forward_noalloc, uses a static device array instead, of
 * TIM_NOALLOC_SCRATCH_BYTES on each device the library's kernels are loaded
 * on, held until the process ends.
 *
 * Execution.  Calls enqueue kernels on `stream` (a hipStream_t; NULL means
 * the null stream) and return without synchronising.  They are re-entrant;
 * two calls may share a workspace only if they are ordered on one stream.
 *
 * Errors.  Argument problems found on the host are reported before any
 * launch, and then no output is written.  Data anomalies never fail a call:
 * they are counted (out-of-range ids, non-finite log-ratios).
 */
#ifndef TIM_H
#define TIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TIM_ABI_VERSION 5

typedef enum {
    TIM_OK = 0,
    TIM_EINVAL = 1,        /* null required pointer, negative size, ld < d,
                              bad dtype/flags, bad stats parameters        */
    TIM_EUNSUPPORTED = 2,  /* d % 64 != 0, misaligned pointer or leading
                              dimension (see tim_logprob_forward)          */
    TIM_EWORKSPACE = 3,    /* workspace null or smaller than the query    */
    TIM_EHIP = 4,          /* a HIP launch or runtime call failed          */
    TIM_ESCRATCH = 5       /* tim_logprob_forward_noalloc: the request
                              needs more than TIM_NOALLOC_SCRATCH_BYTES    */
} tim_status;

/* Element type shared by h and W. */
typedef enum {
    TIM_BF16 = 0,          /* bfloat16 inputs, fp32 MFMA accumulation      */
    TIM_F32 = 1            /* fp32 inputs, fp32 MFMA ("FP32 LM head":
                              "Train-Inference Consistency", section 3)    */
} tim_dtype;

/* Schedule flags for tim_logprob_forward. */
enum {
    TIM_SCHED_INVARIANT = 0u, /* vocabulary split and tile order are functions
                                 of (V, D, dtype) only: batch invariant      */
    TIM_SCHED_FREE = 1u,      /* the fastest configuration this library has
                                 for the given N, allowed to depend on N
                                 (deterministic for a fixed N, not promised
                                 batch invariant).  On gfx950 that is the
                                 invariant one at every N measured (the K
                                 split below is slower).  Exists to price
                                 invariance.                                 */
    TIM_SCHED_SPLIT_K = 2u    /* bf16, 33..256 tokens, no entropy: K split in
                                 two halves over twice the workgroups, the
                                 partial logits added, then folded.  Depends
                                 on N (not batch invariant); an N-dependent
                                 schedule against which invariance is priced.
                                 Other sizes: as TIM_SCHED_FREE.             */
};

/* Library version of this header (TIM_ABI_VERSION). */
int tim_abi_version(void);

/* Static, never-freed description of a status code; unknown codes give a
 * generic string. */
const char* tim_status_string(int status);

/* ------------------------------------------------------------------------
 * Selected-token log-probabilities.
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace tim_logprob_forward needs for these sizes.
 * Returns 0 for sizes the library rejects (negative sizes, unknown dtype or
 * flags).  Pure host function; never touches the device. */
size_t tim_logprob_workspace_bytes(int64_t n, int64_t d, int64_t v,
                                   int dtype, unsigned flags);

/*
 * logp[t] = log softmax(h[t,:] . W^T)[ids[t]]   for t in [0, n).
 *
 * Defined by "RL: Training Inference Mismatch", section "log p" (the
 * hidden -> LM head -> log-softmax -> gather chain).  The caller passes the
 * rows already shifted so that h[t] is the state whose next token is
 * ids[t] (same page, section on shift and mask alignment).  No bias, no
 * temperature, no logits processors: raw logits at temperature 1 (same
 * page, section on logits processors, which asks for all processors off).
 *
 *  h          [n, d] row-major, leading dimension ldh (elements), dtype.
 *  ldh        >= d; ldh % 8 == 0 (bf16) or % 4 == 0 (fp32).
 *  w          [v, d] row-major (the nn.Linear [out, in] layout), ldw >= d,
 *             same alignment rule as ldh.  h and w 16-byte aligned.
 *  ids        [n] int32 target token ids.  An id outside [0, v) is not an
 *             error: its logp is NaN and it is counted in *n_bad_ids.
 *  n          rows, >= 0.  n == 0 returns TIM_OK without a launch.
 *  d          hidden size, > 0, d % 64 == 0 (else TIM_EUNSUPPORTED).
 *  v          vocabulary size, 1 <= v <= 2^31 - 1.
 *  dtype      TIM_BF16 or TIM_F32.
 *  flags      TIM_SCHED_INVARIANT, TIM_SCHED_FREE or TIM_SCHED_SPLIT_K.
 *  logp       [n] fp32 out.
 *  lse        [n] fp32 out, nullable: log sum_v exp z[t,v].
 *  n_bad_ids  [1] int32 out, nullable: number of ids outside [0, v).
 *  workspace  device scratch of at least tim_logprob_workspace_bytes(...)
 *             bytes (null or smaller: TIM_EWORKSPACE), 256-byte aligned
 *             (else TIM_EUNSUPPORTED).
 *  stream     hipStream_t to enqueue on (NULL = null stream).
 *
 * Arithmetic: products of bf16 (or fp32) inputs accumulate in fp32 in a
 * fixed K order with no split-K; the log-sum-exp is carried in fp32 over
 * vocabulary tiles in a fixed order and merged across vocabulary chunks in
 * ascending chunk order.  The logits are never written to memory.
 */
int tim_logprob_forward(const void* h, int64_t ldh,
                        const void* w, int64_t ldw,
                        const int32_t* ids,
                        int64_t n, int64_t d, int64_t v,
                        int dtype, unsigned flags,
                        float* logp, float* lse, int32_t* n_bad_ids,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* Bytes of the static device scratch behind tim_logprob_forward_noalloc,
 * per device (64 MiB). */
#define TIM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * tim_logprob_forward without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that must not
 * call hipMalloc, harnesses that forbid allocation.
 *
 * Arguments, results, checks and errors are those of tim_logprob_forward
 * (same kernels, same schedule, bit-identical outputs), minus `workspace`
 * and `workspace_bytes`.  The scratch is a file-scope device array of
 * TIM_NOALLOC_SCRATCH_BYTES: a request whose tim_logprob_workspace_bytes(
 * n, d, v, dtype, flags) exceeds it returns TIM_ESCRATCH before any launch
 * (bf16 at V = 151936: up to about 14000 rows with the invariant schedule;
 * the K-split schedule's partial logits rarely fit).  The call allocates
 * nothing: the first call on a device looks up that device's copy of the
 * array (the device of `stream`, made current for the lookup).
 *
 * Every call on one device shares that device's array, and the array keeps
 * the last call's contents (nothing in it has to start at zero).  Calls
 * that can overlap on one device — on streams not ordered with each other,
 * or from several host threads — race on it and give wrong results; calls
 * ordered on one stream do not.
 */
int tim_logprob_forward_noalloc(const void* h, int64_t ldh,
                                const void* w, int64_t ldw,
                                const int32_t* ids,
                                int64_t n, int64_t d, int64_t v,
                                int dtype, unsigned flags,
                                float* logp, float* lse, int32_t* n_bad_ids,
                                void* stream);

/* ------------------------------------------------------------------------
 * RMSNorm in front of the head, and scoring at a sampling temperature.
 * ---------------------------------------------------------------------- */

/*
 * y[t, k] = gamma[k] * x[t, k] / sqrt(mean_k x[t, k]^2 + eps),  t in [0, n).
 *
 * The batch-invariant RMSNorm of "训推一致性与 determinism", section 6
 * kernel table (a fixed per-row reduction), and of the VeXact methodology
 * (its batch-invariant kernel list).  Each row is reduced on its own in a
 * fixed order that depends only on d, in fp64; y is formed in fp64 and
 * rounded once to dtype (bf16: nearest, ties to even).  A row's output bits
 * depend only on that row, gamma, d, eps and dtype.
 *
 *  x       [n, d] row-major, ldx >= d elements, dtype (any alignment).
 *  gamma   [d], dtype.
 *  n       rows, >= 0 (0: TIM_OK, no launch).  d > 0.
 *  dtype   TIM_BF16 (x, gamma, y bf16) or TIM_F32 (all fp32).
 *  eps     >= 0, finite.
 *  y       [n, d] out, ldy >= d; may not overlap x.
 *  rstd    [n] fp32 out, nullable: 1 / sqrt(mean x^2 + eps).
 */
int tim_rmsnorm(const void* x, int64_t ldx, const void* gamma,
                int64_t n, int64_t d, int dtype, double eps,
                void* y, int64_t ldy, float* rstd, void* stream);

/* (host) options of tim_logprob_forward_ex. */
typedef struct {
    double temperature;       /* tau > 0, finite.  The distribution scored is
                                 softmax(z / tau): the rollout engine samples
                                 from it at temperature tau, and its
                                 log-probabilities must be compared with the
                                 trainer's at the same tau ("RL: Training
                                 Inference Mismatch", logits-processor
                                 section).  1 = raw logits.                  */
    const void* norm_gamma;   /* device [d] of dtype, or NULL.  Non-NULL: the
                                 input rows are the pre-norm states x and the
                                 call first applies tim_rmsnorm(x, gamma, eps)
                                 into the workspace, then scores the
                                 normalised rows.                            */
    double norm_eps;          /* >= 0, finite; used with norm_gamma.         */
} tim_forward_params;

/* Workspace bytes for tim_logprob_forward_ex with these options;
 * with_entropy != 0 when the entropy output will be requested.  0 for
 * arguments the library rejects.  Pure host function. */
size_t tim_logprob_ex_workspace_bytes(int64_t n, int64_t d, int64_t v, int dtype,
                                      unsigned flags, const tim_forward_params* params,
                                      int with_entropy);

/*
 * tim_logprob_forward with a temperature, an optional RMSNorm in front and
 * an optional entropy output:
 *   z       = W . norm(x_t)   (or W . h_t without norm_gamma)
 *   logp[t] = log softmax(z / tau)[ids[t]]
 *   lse[t]  = log sum_v exp(z_v / tau)
 *   ent[t]  = - sum_v p_v log p_v,  p = softmax(z / tau)
 * (entropy: one of the quantities a train-rollout mismatch disturbs,
 * "训推一致性与 determinism", section 2).  Arguments as tim_logprob_forward;
 * with norm_gamma the rows of h need no particular alignment (they are read
 * by the norm, the head reads the normalised copy).  entropy [n] fp32 out,
 * nullable.  params NULL: TIM_EINVAL.
 *
 * Arithmetic: as tim_logprob_forward, with the exponent scale log2(e) / tau
 * and 1 / tau each rounded once to fp32 (both exact at tau = 1, where the
 * results are bitwise those of tim_logprob_forward).  The entropy carries,
 * next to the running maximum and sum, the running sum of p-weighted
 * exponent arguments, merged in the same fixed order; it is batch
 * invariant and deterministic like logp.
 */
int tim_logprob_forward_ex(const void* h, int64_t ldh,
                           const void* w, int64_t ldw,
                           const int32_t* ids,
                           int64_t n, int64_t d, int64_t v,
                           int dtype, unsigned flags,
                           const tim_forward_params* params,
                           float* logp, float* lse, float* entropy, int32_t* n_bad_ids,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * Mismatch statistics between trainer and rollout log-probabilities.
 * ---------------------------------------------------------------------- */

/* (host) parameters of tim_mismatch_stats. */
typedef struct {
    double tis_clip_c; /* C > 0.  Token-level truncated IS weight
                          w = min(e^delta, C); a token is "clipped" iff
                          delta > log(C) (log(C) evaluated once, in fp64).
                          "Train-Inference Consistency", section 4, and the
                          TIS rows of the VeXact compensation table.       */
    double seq_lo;     /* reject sequence iff mean delta < seq_lo ...      */
    double seq_hi;     /* ... or mean delta > seq_hi; seq_lo <= seq_hi.
                          Log-domain bounds: the geometric mean of r over a
                          sequence's tokens is exp(mean delta), so a ratio
                          window [a, b] is passed as [log a, log b].      */
    double seq_k3_hi;  /* K3-rejects a sequence iff its mean k3 > seq_k3_hi
                          (not NaN; +inf never rejects).  The K3 form of the
                          r_corr sequence rejection: VeXact compensation
                          table, srs-k3 rows.                              */
} tim_stats_params;

/* (host struct) optional per-token outputs, each [n], each nullable.
 * A position with mask == 0 is not scored: delta = 0, ratio = 1,
 * k1 = k2 = k3 = 0, tis_w = 0, clipped = 0.  A scored position whose delta
 * is not finite gets delta/ratio/k's as computed (NaN/inf), tis_w = 0 and
 * clipped = 0. */
typedef struct {
    float* delta;      /* logp_train - logp_rollout (computed in fp64)     */
    float* ratio;      /* exp(delta)                                       */
    float* k1;         /* -delta                                           */
    float* k2;         /* delta^2 / 2                                      */
    float* k3;         /* exp(delta) - 1 - delta                           */
    float* tis_w;      /* clipped ? C : exp(delta)                         */
    uint8_t* clipped;  /* 1 iff delta > log C                              */
} tim_token_out;

/* (host struct) optional per-sequence outputs, each [s], each nullable.
 * Means are over the sequence's valid tokens (mask != 0 and finite delta);
 * a sequence with no valid token has means 0 and is never rejected. */
typedef struct {
    int32_t* n_valid;
    int32_t* n_clipped;
    int32_t* n_nan;        /* mask != 0 but delta not finite               */
    double* mean_delta;
    double* mean_k1;
    double* mean_k2;
    double* mean_k3;
    double* mean_tis_w;
    uint8_t* reject;       /* 1 iff mean_delta < seq_lo || > seq_hi        */
    uint8_t* reject_k3;    /* 1 iff mean_k3 > seq_k3_hi                    */
} tim_seq_out;

/* Indices of the batch aggregate vector (fp64).  Token means are over all
 * valid tokens of the batch; sequence means are the mean, over sequences
 * with at least one valid token, of the per-sequence means ("RL: Training
 * Inference Mismatch", monitoring flow: mean per completion, then mean
 * over completions).  Ratios with a zero denominator are 0. */
enum {
    TIM_B_TOK_MEAN_DELTA = 0,
    TIM_B_TOK_MEAN_K1 = 1,
    TIM_B_TOK_MEAN_K2 = 2,
    TIM_B_TOK_MEAN_K3 = 3,     /* train/is_approx_k3_kl                    */
    TIM_B_SEQ_MEAN_DELTA = 4,
    TIM_B_SEQ_MEAN_K1 = 5,
    TIM_B_SEQ_MEAN_K2 = 6,
    TIM_B_SEQ_MEAN_K3 = 7,
    TIM_B_TOK_MEAN_TIS_W = 8,
    TIM_B_CLIP_RATIO = 9,      /* train/is_clip_ratio = n_clipped / n_valid */
    TIM_B_NAN_RATIO = 10,      /* train/is_nan_ratio = n_nan / n_masked_in  */
    TIM_B_REJECT_FRAC = 11,    /* rejected / sequences with a valid token  */
    TIM_B_MEAN_ABS_DELTA = 12,
    TIM_B_MAX_ABS_DELTA = 13,
    TIM_B_N_VALID = 14,
    TIM_B_N_NAN = 15,
    TIM_B_N_CLIPPED = 16,
    TIM_B_N_SEQ_NONEMPTY = 17,
    TIM_B_N_SEQ_REJECTED = 18,
    TIM_B_REJECT_K3_FRAC = 19, /* K3-rejected / sequences with a valid token */
    TIM_B_N_SEQ_REJECTED_K3 = 20,
    TIM_B_NFIELDS = 21
};

/* Bytes of device workspace tim_mismatch_stats needs; 0 for negative
 * sizes.  Pure host function. */
size_t tim_stats_workspace_bytes(int64_t n, int64_t s);

/*
 * Per-token log-ratio statistics, per-sequence means and rejection flags,
 * and batch aggregates.
 *
 *  logp_train    [n] fp32: trainer-side log pi_old^train(a_t|s_t).
 *  logp_rollout  [n] fp32: log pi_old^rollout(a_t|s_t) recorded at rollout.
 *  mask          [n] uint8, nullable (= every token scored).  Tokens with
 *                mask == 0 (prompt, padding) are left out of every sum.
 *  cu_seqlens    [s+1] int32, 0 = c0 <= c1 <= ... <= cs = n (precondition,
 *                not checked on the device): sequence j is [c_j, c_{j+1}).
 *  n, s          tokens and sequences; n >= 0, s >= 1 unless n == 0.
 *  p             (host) clip constant and rejection window.
 *  tok, seq      (host structs) nullable; their members are nullable.
 *  batch         [TIM_B_NFIELDS] fp64 out, nullable.
 *  workspace     >= tim_stats_workspace_bytes(n, s) bytes (else
 *                TIM_EWORKSPACE), 256-byte aligned (else TIM_EUNSUPPORTED).
 *  Errors: TIM_EINVAL for n < 0, s < 0, n > 0 with s == 0, null p, C not a
 *  finite positive number, seq_lo > seq_hi or a NaN bound (seq_k3_hi
 *  included), null lt/lr when
 *  n > 0, null cu_seqlens; TIM_EUNSUPPORTED for n or s beyond int32.
 *  n == 0 and s == 0 returns TIM_OK without a launch; TIM_EUNSUPPORTED also
 *  when floor(n / 1024) + s + 1 reaches 2^31.
 *
 * delta is computed in fp64 from the fp32 inputs, so both signs and the
 * clip decision are exact; exp/expm1 are evaluated in fp64.
 */
int tim_mismatch_stats(const float* logp_train, const float* logp_rollout,
                       const uint8_t* mask, const int32_t* cu_seqlens,
                       int64_t n, int64_t s, const tim_stats_params* p,
                       const tim_token_out* tok, const tim_seq_out* seq,
                       double* batch,
                       void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * Extra mismatch metrics: extreme-token rate, relative difference and
 * quantiles of the ratio and of |delta|.
 * ---------------------------------------------------------------------- */

#define TIM_X_MAX_Q 4      /* probabilities per call, both kinds together */

/* (host) parameters of tim_mismatch_extras. */
typedef struct {
    double tok_tau;        /* a valid token is "extreme" iff |delta| > tok_tau
                              (not NaN; +inf counts none)                   */
    int32_t n_ratio_q;     /* number of quantiles of r = exp(delta) ...     */
    int32_t n_abs_q;       /* ... and of |delta|; n_ratio_q + n_abs_q <=
                              TIM_X_MAX_Q, both >= 0                        */
    double ratio_q[TIM_X_MAX_Q];   /* probabilities in [0, 1]               */
    double abs_q[TIM_X_MAX_Q];     /* probabilities in [0, 1]               */
} tim_extras_params;

/* Indices of the fp64 output vector of tim_mismatch_extras. */
enum {
    TIM_X_N_VALID = 0,         /* valid tokens: mask != 0, finite delta     */
    TIM_X_N_EXTREME = 1,       /* valid tokens with |delta| > tok_tau       */
    TIM_X_EXTREME_FRAC = 2,    /* n_extreme / n_valid                       */
    TIM_X_MEAN_REL_DIFF = 3,   /* mean of |delta| / (|logp_train| + 1e-8)   */
    TIM_X_RATIO_Q = 4,         /* 4 slots: quantile ratio_q[i] of r         */
    TIM_X_ABS_Q = 8,           /* 4 slots: quantile abs_q[i] of |delta|     */
    TIM_X_NFIELDS = 12
};

/* Bytes of device workspace tim_mismatch_extras needs; 0 for n < 0 or
 * n > 2^31 - 1.  Pure host function. */
size_t tim_extras_workspace_bytes(int64_t n);

/*
 * Batch metrics over the valid tokens (mask != 0 and a finite
 * delta = logp_train - logp_rollout, computed in fp64):
 *
 *   - the extreme-token rate, the share of valid tokens with
 *     |delta| > tok_tau ("训推一致性与 determinism", section 7, metric
 *     table, the fraction of tokens above a threshold);
 *   - the mean of |delta| / (|logp_train| + 1e-8) ("RL: Training Inference
 *     Mismatch", training/inference consistency section, rel_diff and its
 *     masked mean);
 *   - quantiles of r = exp(delta) and of |delta| (same Atlas table: ratio
 *     quantiles 0.01 / 0.5 / 0.99 and the p95 of the absolute difference).
 *     Quantile q of m sorted values x is x[lo] + (x[hi] - x[lo]) * f with
 *     pos = q (m - 1), lo = floor(pos), hi = min(lo + 1, m - 1),
 *     f = pos - lo, each operation rounded in fp64.
 *
 *  logp_train, logp_rollout  [n] fp32;  mask [n] uint8, nullable (= all).
 *  n          tokens, 0 <= n <= 2^31 - 1.
 *  p          (host) threshold and probabilities.
 *  out        [TIM_X_NFIELDS] fp64 out, nullable (then nothing is written).
 *             With no valid token every ratio and quantile is 0.  Unused
 *             quantile slots are 0.
 *  workspace  >= tim_extras_workspace_bytes(n) bytes (else TIM_EWORKSPACE),
 *             256-byte aligned (else TIM_EUNSUPPORTED).
 *  Errors: TIM_EINVAL for n < 0, null p, a NaN tok_tau, a probability
 *  outside [0, 1], a negative count or more than TIM_X_MAX_Q of them, null
 *  logp_train / logp_rollout when n > 0; TIM_EUNSUPPORTED for n > 2^31 - 1.
 *
 * The order statistics are selected exactly (a radix select over 64-bit
 * keys of the fp64 deltas, integer histograms), so the |delta| quantiles
 * are correctly rounded functions of the inputs and every output is
 * deterministic; the relative-difference sum is reduced in an order that
 * depends only on n.
 */
int tim_mismatch_extras(const float* logp_train, const float* logp_rollout,
                        const uint8_t* mask, int64_t n, const tim_extras_params* p,
                        double* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * Backward of the selected-token log-probability.
 * ---------------------------------------------------------------------- */

enum {
    TIM_BWD_ACCUMULATE_DW = 1u  /* dw is read and the sum over this batch's
                                   tokens continues from it (see below)      */
};

/* Bytes of device workspace tim_logprob_backward needs; 0 for sizes or a
 * dtype it does not accept.  Pure host function. */
size_t tim_logprob_backward_workspace_bytes(int64_t n, int64_t d, int64_t v, int dtype);

/*
 * Gradients of L through logp[t] = log softmax(h[t,:] . W^T)[ids[t]], given
 * grad_logp[t] = dL/dlogp[t]:
 *     dz[t, v] = grad_logp[t] ([v == ids[t]] - softmax(z_t)[v])
 *     dh[t, :] = sum_v dz[t, v] W[v, :]          (v ascending)
 *     dw[v, :] = sum_t dz[t, v] h[t, :]          (t ascending)
 * ("RL: Training Inference Mismatch", the "log p" chain differentiated; the
 * policy-gradient term g_t grad log q_t of its importance-sampling section.)
 *
 *  h, ldh, w, ldw, ids, n, d, v, dtype  as for tim_logprob_forward
 *             (TIM_F32: the FP32 LM head of "Train-Inference Consistency",
 *             section 3, which keeps the output layer's weights and compute
 *             in FP32 during training).
 *  lse        [n] fp32: the lse output of tim_logprob_forward on the same
 *             inputs (the softmax is exp(z - lse)).
 *  grad_logp  [n] fp32.  A token with grad 0, or an id outside [0, v),
 *             contributes nothing.
 *  dh         [n, d] fp32 out (row stride d), nullable; 16-byte aligned
 *             (else TIM_EUNSUPPORTED).
 *  dw         [v, d] fp32 out (row stride d), nullable; 16-byte aligned
 *             (else TIM_EUNSUPPORTED).  With TIM_BWD_ACCUMULATE_DW its
 *             incoming values start the sums.
 *  flags      0 or TIM_BWD_ACCUMULATE_DW.
 *  workspace  >= tim_logprob_backward_workspace_bytes(...) bytes,
 *             256-byte aligned.
 *
 * Arithmetic: the logits are recomputed exactly as tim_logprob_forward does
 * (same K order and instructions).  TIM_BF16: dz is rounded to bf16 once;
 * dh and dw are bf16 x bf16 products accumulated in fp32.  TIM_F32: dz stays
 * fp32; dh and dw are fp32 products accumulated in fp32.  One chain per
 * output element in ascending K, no split-K and no atomics.  dh[t] depends
 * only on token t.
 * dw's chain over tokens continues across calls in accumulate mode, so
 * accumulating batches whose sizes are multiples of 64 tokens reproduces
 * the bits of one call over their concatenation.
 * Errors as tim_logprob_forward, plus TIM_EINVAL for null lse / grad_logp
 * when n > 0 and for flags other than 0 and TIM_BWD_ACCUMULATE_DW.
 */
int tim_logprob_backward(const void* h, int64_t ldh, const void* w, int64_t ldw,
                         const int32_t* ids, const float* lse, const float* grad_logp,
                         int64_t n, int64_t d, int64_t v, int dtype, unsigned flags,
                         float* dh, float* dw, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * PPO / GRPO clipped surrogate with truncated importance weights.
 * ---------------------------------------------------------------------- */

/* (host) parameters of tim_ppo_loss. */
typedef struct {
    double eps_low;    /* ratios below 1 - eps_low are clipped (>= 0)        */
    double eps_high;   /* ratios above 1 + eps_high are clipped (>= 0)       */
    int32_t bypass;    /* 0: ratio over the trainer's recomputed old logp
                          ("recompute"); 1: over the rollout's ("bypass")
                          (VeXact eq. (3))                                   */
    double tis_c;      /* > 0: weight w = min(exp(old_train - old_rollout),
                          tis_c), the truncated r_corr of the VeXact
                          compensation table's TIS rows; <= 0: w = 1.  Not
                          NaN.                                               */
    double grad_scale; /* 0: grad is the derivative of the token mean over
                          this call's valid tokens (a second pass divides by
                          n_valid once it is known); > 0 (finite): of
                          grad_scale * (sum of the token losses), written in
                          one pass, e.g. 1 / (valid tokens over every
                          data-parallel rank).  Other outputs do not depend
                          on it.                                             */
} tim_ppo_params;

/* (host struct) optional per-token outputs, each [n] fp32 (clipped uint8),
 * each nullable.  Tokens left out (mask 0, non-finite) get loss 0, grad 0,
 * ratio 1, contrib 0, clipped 0. */
typedef struct {
    float* loss;       /* -w min(r A, clip(r, 1 - eps_low, 1 + eps_high) A)
                          (VeXact eq. (2))                                   */
    float* grad;       /* -w [not clipped] r A / n_valid (d mean loss / d logp[t]),
                          or times grad_scale instead of / n_valid           */
    float* ratio;      /* r = exp(logp - logp_old)                           */
    float* contrib;    /* -(r - 1) A, the zero-centred contribution (VeXact
                          eq. (5))                                           */
    uint8_t* clipped;  /* 1 iff A > 0 and r > 1 + eps_high, or A < 0 and
                          r < 1 - eps_low (the gradient is dropped)          */
} tim_ppo_token_out;

/* Indices of the fp64 batch vector of tim_ppo_loss (means over valid
 * tokens: mask != 0 and finite r, w and A; 0 when there is none). */
enum {
    TIM_P_MEAN_LOSS = 0,
    TIM_P_CLIP_FRAC = 1,
    TIM_P_MEAN_RATIO = 2,
    TIM_P_MEAN_TIS_W = 3,
    TIM_P_MEAN_CONTRIB = 4,
    TIM_P_N_VALID = 5,
    TIM_P_N_CLIPPED = 6,
    TIM_P_N_NAN = 7,
    TIM_P_NFIELDS = 8
};

/* Bytes of device workspace tim_ppo_loss needs (independent of n; 0 for
 * n < 0).  Pure host function. */
size_t tim_ppo_workspace_bytes(int64_t n);

/*
 * The token-level clipped surrogate of VeXact eq. (2) with the ratios of
 * eq. (3), the truncated importance weight of its TIS rows and the
 * contribution of eq. (5), and the gradient of the token-mean loss by the
 * current log-probabilities.  The clip test follows "RL: Training Inference
 * Mismatch" (clipped importance ratios: the gradient is dropped once the
 * ratio leaves the interval on the side the advantage favours).
 *
 *  logp              [n] fp32: current policy log pi_theta(a_t|s_t).
 *  logp_old_train    [n] fp32: log pi_old^train (trainer recompute).
 *  logp_old_rollout  [n] fp32: log pi_old^rollout (rollout engine).
 *  advantages        [n] fp32.
 *  mask              [n] uint8, nullable (= all tokens).
 *  p                 (host) parameters.
 *  tok               (host struct) nullable; members nullable.
 *  batch             [TIM_P_NFIELDS] fp64 out, nullable.
 *  workspace         >= tim_ppo_workspace_bytes(n) bytes, 256-byte aligned.
 *  Errors: TIM_EINVAL for n < 0, null p, negative or NaN eps, NaN tis_c,
 *  bypass not 0/1, grad_scale negative, NaN or infinite, null inputs when
 *  n > 0; TIM_EWORKSPACE, TIM_EUNSUPPORTED
 *  (alignment) as elsewhere.  n == 0 writes the batch vector (zeros).
 * Per-token arithmetic is fp64 from the fp32 inputs; the sums are reduced in
 * a fixed order that depends only on n.
 */
int tim_ppo_loss(const float* logp, const float* logp_old_train, const float* logp_old_rollout,
                 const float* advantages, const uint8_t* mask, int64_t n,
                 const tim_ppo_params* p, const tim_ppo_token_out* tok, double* batch,
                 void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TIM_H */
