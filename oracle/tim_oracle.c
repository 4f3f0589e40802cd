/*
 * tim_oracle.c — plain, slow, fp64 CPU reference ("the oracle").
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this file's library.  The HIP
 * library never links, calls or includes it, and it includes nothing of the
 * HIP library: the two share no code, headers, tables or constants.
 *
 * Everything here is the textbook definition written out in double
 * precision, in the order the definitions state, with no blocking or fusion
 * that changes the arithmetic:
 *
 *   or_logprob_rows     z_v = sum_k h_k W_vk (k ascending, fp64),
 *                       lse = m + log sum_v exp(z_v - m) (v ascending),
 *                       logp = z_a - lse.
 *                       "RL: Training Inference Mismatch", section "log p"
 *                       (hidden -> LM head -> log-softmax -> gather).
 *   or_logprob_rows_ex  the same for softmax(z / tau), with its entropy
 *                       ("RL: Training Inference Mismatch", logits-processor
 *                       section).
 *   or_rmsnorm          y = gamma x / sqrt(mean x^2 + eps) per row
 *                       ("训推一致性与 determinism", section 6 kernel table).
 *   or_mismatch_stats   delta = train - rollout ("Diagnosing Training
 *                       Inference Mismatch ... (VeXact)", eq. (1)),
 *                       r = exp(delta) ("训推一致性与 determinism", section 2),
 *                       k1 = -log r, k2 = (log r)^2 / 2, k3 = (r-1) - log r
 *                       ("RL: Training Inference Mismatch", KL-estimator
 *                       table; VeXact K1/K3), truncated IS weight and
 *                       clip flag ("Train-Inference Consistency", section 4),
 *                       per-sequence mean then batch mean ("RL: Training
 *                       Inference Mismatch", monitoring flow, steps 2-3),
 *                       geometric-mean-ratio sequence rejection and its
 *                       K3 form, mean k3 above a bound (VeXact
 *                       compensation table, srs-k1 / srs-k3 rows).
 *   or_mismatch_extras  over the valid tokens of a batch: extreme-token
 *                       rate |delta| > tau, quantiles of r and of |delta|
 *                       ("训推一致性与 determinism", section 7, metric
 *                       table), and the masked mean of
 *                       |lt - lr| / (|lt| + 1e-8) ("RL: Training Inference
 *                       Mismatch", training/inference consistency).
 *   or_bf16_decode /    exact bf16 -> double, and double -> bf16 with
 *   or_bf16_round_rne   round-to-nearest, ties-to-even ("Train-infer
 *                       mismatch for Open-weight MoE RL", figure "Rounding
 *                       depends on the order of additions").
 *
 * Readings where the pages leave a step open (sign of delta, clip form,
 * NaN handling, empty sequences, log-domain rejection bounds) are the ones
 * documented with the C ABI: delta = train - rollout; clipped iff
 * delta > log C; non-finite delta is counted and left out of every sum;
 * a sequence with no valid token has means 0 and is never rejected.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared -pthread -lm
 * (no -ffast-math: IEEE semantics and the written summation order are kept).
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ */
/* bfloat16                                                            */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32: decode by placing the 16
 * bits in the high half of a float.  Exact (every bf16 is a float, every
 * float is a double). */
double or_bf16_decode(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, and return its
 * bits.  Written from the definition: find the two bf16 neighbours of |x|
 * on the grid of its binade and pick the nearer, the even one on a tie. */
uint16_t or_bf16_round_rne(double x)
{
    if (isnan(x)) return (uint16_t)0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    /* bf16: 8 exponent bits (bias 127), 7 stored fraction bits.
     * Normal numbers span [2^-126, (2 - 2^-7) 2^127]; the subnormal grid
     * spacing is 2^-133. */
    int e;
    frexp(a, &e);               /* a = m 2^e, m in [0.5, 1) */
    int unit_exp = e - 8;       /* 8 significant bits: spacing 2^(e-8) */
    if (unit_exp < -133) unit_exp = -133;   /* subnormal range */
    double scaled = ldexp(a, -unit_exp);    /* exact: power-of-two scale */
    double q = floor(scaled);
    double rem = scaled - q;                /* exact */
    if (rem > 0.5 || (rem == 0.5 && fmod(q, 2.0) != 0.0)) q += 1.0;
    double r = ldexp(q, unit_exp);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);  /* inf */
    float f = (float)r;         /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

void or_bf16_round_rne_n(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_round_rne(x[i]);
}

/* ------------------------------------------------------------------ */
/* RMSNorm                                                             */
/* ------------------------------------------------------------------ */

static double load_elem(const void* base, int dtype, int64_t idx);

/*
 * Root-mean-square normalisation of each row of x [n, ldx] with the gain
 * gamma [d]: rstd_t = 1 / sqrt(mean_k x[t, k]^2 + eps) and
 * y[t, k] = gamma[k] x[t, k] rstd_t, in fp64, the row sum in ascending k
 * ("训推一致性与 determinism", section 6 kernel table, and "Diagnosing
 * Training Inference Mismatch ... (VeXact)", its methodology: RMSNorm as
 * one of the kernels made batch invariant by a fixed per-row reduction).
 * x and gamma are both bf16 or both fp32 (dtype); y [n, d] and rstd [n]
 * are fp64 (rstd nullable).  Returns 0, or -1 on bad arguments.
 */
int or_rmsnorm(const void* x, int64_t ldx, const void* gamma, int dtype, int64_t n,
               int64_t d, double eps, double* y, double* rstd)
{
    if (n < 0 || d <= 0 || ldx < d || !(eps >= 0.0) || isinf(eps) ||
        (n > 0 && (!x || !gamma || !y)))
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        double ss = 0.0;
        for (int64_t k = 0; k < d; ++k) {
            const double xv = load_elem(x, dtype, t * ldx + k);
            ss += xv * xv;
        }
        const double r = 1.0 / sqrt(ss / (double)d + eps);
        if (rstd) rstd[t] = r;
        for (int64_t k = 0; k < d; ++k)
            y[t * d + k] = load_elem(gamma, dtype, k) * load_elem(x, dtype, t * ldx + k) * r;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Selected-token log-probability                                      */
/* ------------------------------------------------------------------ */

enum { OR_BF16 = 0, OR_F32 = 1 };

static double load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == OR_BF16) return or_bf16_decode(((const uint16_t*)base)[idx]);
    return (double)((const float*)base)[idx];
}

typedef struct {
    const void* h; int64_t ldh;
    const void* w; int64_t ldw;
    const int32_t* ids;
    int dtype; int64_t d, v;
    const int64_t* rows;   /* NULL: rows 0..nrows-1 */
    int64_t nrows;
    double* logp; double* lse; double* zsel;
    double tau;            /* temperature: the softmax is taken of z / tau */
    double* ent;           /* entropy of softmax(z / tau); nullable */
    int64_t begin, end;    /* slice of the row list owned by one thread */
} lp_job;

/* Rows handled together share one pass over W (cache reuse only: each
 * logit is still one sequential fp64 sum over k). */
#define OR_ROW_BLOCK 8

static void* lp_worker(void* arg)
{
    lp_job* j = (lp_job*)arg;
    const int64_t d = j->d, v = j->v;
    double* hd = (double*)malloc(sizeof(double) * (size_t)(OR_ROW_BLOCK * d));
    double* wd = (double*)malloc(sizeof(double) * (size_t)d);
    double* z = (double*)malloc(sizeof(double) * (size_t)(OR_ROW_BLOCK * v));
    if (!hd || !wd || !z) {
        for (int64_t i = j->begin; i < j->end; ++i) j->logp[i] = NAN;
        free(hd); free(wd); free(z);
        return NULL;
    }
    for (int64_t i0 = j->begin; i0 < j->end; i0 += OR_ROW_BLOCK) {
        int64_t nb = j->end - i0 < OR_ROW_BLOCK ? j->end - i0 : OR_ROW_BLOCK;
        for (int64_t r = 0; r < nb; ++r) {
            int64_t t = j->rows ? j->rows[i0 + r] : i0 + r;
            for (int64_t k = 0; k < d; ++k)
                hd[r * d + k] = load_elem(j->h, j->dtype, t * j->ldh + k);
        }
        /* logits: z[t, v] = sum_k h[t, k] W[v, k] */
        for (int64_t c = 0; c < v; ++c) {
            for (int64_t k = 0; k < d; ++k)
                wd[k] = load_elem(j->w, j->dtype, c * j->ldw + k);
            for (int64_t r = 0; r < nb; ++r) {
                const double* hr = hd + r * d;
                double acc = 0.0;
                for (int64_t k = 0; k < d; ++k) acc += hr[k] * wd[k];
                z[r * v + c] = acc;
            }
        }
        /* log-softmax of z / tau and gather (tau = 1: z / 1 is z itself) */
        for (int64_t r = 0; r < nb; ++r) {
            int64_t t = j->rows ? j->rows[i0 + r] : i0 + r;
            double* zr = z + r * v;
            for (int64_t c = 0; c < v; ++c) zr[c] = zr[c] / j->tau;
            double m = -INFINITY;
            for (int64_t c = 0; c < v; ++c)
                if (zr[c] > m) m = zr[c];
            double s = 0.0;
            for (int64_t c = 0; c < v; ++c) s += exp(zr[c] - m);
            double l = m + log(s);
            int32_t a = j->ids[t];
            int ok = a >= 0 && (int64_t)a < v;
            if (j->lse) j->lse[i0 + r] = l;
            if (j->zsel) j->zsel[i0 + r] = ok ? zr[a] : NAN;
            j->logp[i0 + r] = ok ? zr[a] - l : NAN;
            if (j->ent) {
                /* H = -sum_v p_v log p_v = sum_v p_v (lse - z_v), p_v = exp(z_v - lse);
                 * every term is >= 0 */
                double hsum = 0.0;
                for (int64_t c = 0; c < v; ++c) {
                    const double lp = zr[c] - l;
                    hsum += -exp(lp) * lp;
                }
                j->ent[i0 + r] = hsum;
            }
        }
    }
    free(hd); free(wd); free(z);
    return NULL;
}

/* Number of CPUs this process may run on. */
int or_available_cpus(void)
{
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}

/*
 * logp[i], lse[i], zsel[i] for token row t = rows[i] (rows == NULL: t = i),
 * i in [0, nrows).  h: [*, ldh], W: [v, ldw], ids indexed by t.
 * An id outside [0, v) gives NaN logp and zsel.  lse/zsel nullable.
 * nthreads <= 0: all available CPUs.  Returns the thread count used, or -1
 * on bad arguments.
 */
int or_logprob_rows_ex(const void* h, int64_t ldh, const void* w, int64_t ldw,
                       const int32_t* ids, int dtype, int64_t d, int64_t v,
                       const int64_t* rows, int64_t nrows, double tau,
                       double* logp, double* lse, double* zsel, double* entropy,
                       int nthreads);

int or_logprob_rows(const void* h, int64_t ldh, const void* w, int64_t ldw,
                    const int32_t* ids, int dtype, int64_t d, int64_t v,
                    const int64_t* rows, int64_t nrows,
                    double* logp, double* lse, double* zsel, int nthreads)
{
    return or_logprob_rows_ex(h, ldh, w, ldw, ids, dtype, d, v, rows, nrows, 1.0,
                              logp, lse, zsel, NULL, nthreads);
}

/*
 * The same with a sampling temperature tau > 0: logp, lse and the entropy
 * H = -sum_v p_v log p_v of p = softmax(z / tau) ("RL: Training Inference
 * Mismatch", logits-processor section: at temperature tau the sampler draws
 * from softmax(z / tau), so a trainer that scores the sampler's tokens must
 * use the same tau; "训推一致性与 determinism", section 2, names entropy
 * among the quantities a mismatch disturbs).  zsel is z_a / tau.  entropy
 * nullable.
 */
int or_logprob_rows_ex(const void* h, int64_t ldh, const void* w, int64_t ldw,
                       const int32_t* ids, int dtype, int64_t d, int64_t v,
                       const int64_t* rows, int64_t nrows, double tau,
                       double* logp, double* lse, double* zsel, double* entropy,
                       int nthreads)
{
    if (!h || !w || !ids || !logp || d <= 0 || v <= 0 || nrows < 0 ||
        ldh < d || ldw < d || (dtype != OR_BF16 && dtype != OR_F32) ||
        !(tau > 0.0) || isinf(tau))
        return -1;
    if (nthreads <= 0) nthreads = or_available_cpus();
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    lp_job* jobs = (lp_job*)calloc((size_t)nthreads, sizeof(lp_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    for (int i = 0; i < nthreads; ++i) {
        lp_job* j = &jobs[i];
        j->h = h; j->ldh = ldh; j->w = w; j->ldw = ldw; j->ids = ids;
        j->dtype = dtype; j->d = d; j->v = v; j->rows = rows;
        j->nrows = nrows; j->logp = logp; j->lse = lse; j->zsel = zsel;
        j->tau = tau; j->ent = entropy;
        j->begin = nrows * i / nthreads;
        j->end = nrows * (i + 1) / nthreads;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, lp_worker, &jobs[i]);
    lp_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(jobs); free(th);
    return nthreads;
}

/* ------------------------------------------------------------------ */
/* Mismatch statistics                                                 */
/* ------------------------------------------------------------------ */

/* Batch vector layout (same meaning as the library's, restated here). */
enum {
    OB_TOK_MEAN_DELTA, OB_TOK_MEAN_K1, OB_TOK_MEAN_K2, OB_TOK_MEAN_K3,
    OB_SEQ_MEAN_DELTA, OB_SEQ_MEAN_K1, OB_SEQ_MEAN_K2, OB_SEQ_MEAN_K3,
    OB_TOK_MEAN_TIS_W, OB_CLIP_RATIO, OB_NAN_RATIO, OB_REJECT_FRAC,
    OB_MEAN_ABS_DELTA, OB_MAX_ABS_DELTA, OB_N_VALID, OB_N_NAN, OB_N_CLIPPED,
    OB_N_SEQ_NONEMPTY, OB_N_SEQ_REJECTED, OB_REJECT_K3_FRAC,
    OB_N_SEQ_REJECTED_K3, OB_NFIELDS
};

int or_batch_nfields(void) { return OB_NFIELDS; }

static double safe_div(double a, double b) { return b != 0.0 ? a / b : 0.0; }

/*
 * Token outputs (each [n], nullable), sequence outputs (each [s],
 * nullable) and batch[OB_NFIELDS] (nullable).  mask nullable = all scored.
 * cu: [s+1] with 0 = cu[0] <= ... <= cu[s] = n.  Returns 0, or -1 on bad
 * arguments.  A sequence is rejected (s_reject) when its mean delta lies
 * outside [seq_lo, seq_hi], and K3-rejected (s_reject_k3) when its mean k3
 * exceeds seq_k3_hi (+inf: never); empty sequences are never rejected.
 */
int or_mismatch_stats(const float* lt, const float* lr, const uint8_t* mask,
                      const int32_t* cu, int64_t n, int64_t s,
                      double clip_c, double seq_lo, double seq_hi,
                      double seq_k3_hi,
                      double* t_delta, double* t_ratio, double* t_k1,
                      double* t_k2, double* t_k3, double* t_w,
                      uint8_t* t_clipped,
                      int32_t* s_n_valid, int32_t* s_n_clipped,
                      int32_t* s_n_nan, double* s_mean_delta,
                      double* s_mean_k1, double* s_mean_k2, double* s_mean_k3,
                      double* s_mean_w, uint8_t* s_reject,
                      uint8_t* s_reject_k3, double* batch)
{
    if (n < 0 || s < 0 || (n > 0 && (!lt || !lr || !cu || s < 1)) ||
        !(clip_c > 0.0) || !(seq_lo <= seq_hi) || isnan(seq_k3_hi))
        return -1;
    for (int64_t j = 0; j < s; ++j)
        if (cu[j] > cu[j + 1]) return -1;
    if (s > 0 && (cu[0] != 0 || cu[s] != n)) return -1;

    const double log_c = log(clip_c);

    /* batch token sums, accumulated over tokens in index order */
    double b_delta = 0, b_k1 = 0, b_k2 = 0, b_k3 = 0, b_w = 0, b_abs = 0;
    double b_max = 0;
    int64_t b_valid = 0, b_nan = 0, b_clip = 0, b_in = 0;
    /* batch sequence sums, accumulated over sequences in index order */
    double bs_delta = 0, bs_k1 = 0, bs_k2 = 0, bs_k3 = 0;
    int64_t bs_nonempty = 0, bs_rejected = 0, bs_rejected_k3 = 0;

    for (int64_t j = 0; j < s; ++j) {
        double q_delta = 0, q_k1 = 0, q_k2 = 0, q_k3 = 0, q_w = 0;
        int64_t q_valid = 0, q_nan = 0, q_clip = 0;
        for (int64_t t = cu[j]; t < cu[j + 1]; ++t) {
            int scored = mask ? mask[t] != 0 : 1;
            double delta = 0, ratio = 1, k1 = 0, k2 = 0, k3 = 0, w = 0;
            int clipped = 0;
            if (scored) {
                b_in++;
                delta = (double)lt[t] - (double)lr[t];
                ratio = exp(delta);
                k1 = -delta;                  /* -log r            */
                k2 = 0.5 * delta * delta;     /* (log r)^2 / 2     */
                k3 = expm1(delta) - delta;    /* (r - 1) - log r   */
                if (!isfinite(delta)) {
                    q_nan++;
                    b_nan++;
                    w = 0;
                } else {
                    clipped = delta > log_c;
                    w = clipped ? clip_c : ratio;
                    q_valid++; q_delta += delta; q_k1 += k1; q_k2 += k2;
                    q_k3 += k3; q_w += w; q_clip += clipped;
                    b_valid++; b_delta += delta; b_k1 += k1; b_k2 += k2;
                    b_k3 += k3; b_w += w; b_clip += clipped;
                    b_abs += fabs(delta);
                    if (fabs(delta) > b_max) b_max = fabs(delta);
                }
            }
            if (t_delta) t_delta[t] = delta;
            if (t_ratio) t_ratio[t] = ratio;
            if (t_k1) t_k1[t] = k1;
            if (t_k2) t_k2[t] = k2;
            if (t_k3) t_k3[t] = k3;
            if (t_w) t_w[t] = w;
            if (t_clipped) t_clipped[t] = (uint8_t)clipped;
        }
        double m_delta = safe_div(q_delta, (double)q_valid);
        double m_k1 = safe_div(q_k1, (double)q_valid);
        double m_k2 = safe_div(q_k2, (double)q_valid);
        double m_k3 = safe_div(q_k3, (double)q_valid);
        double m_w = safe_div(q_w, (double)q_valid);
        int reject = q_valid > 0 && (m_delta < seq_lo || m_delta > seq_hi);
        /* K3 form of the sequence rejection: the sequence's mean k3 (its
         * sampled estimate of the rollout-to-trainer KL) above a bound */
        int reject_k3 = q_valid > 0 && m_k3 > seq_k3_hi;
        if (q_valid > 0) {
            bs_nonempty++;
            bs_rejected += reject;
            bs_rejected_k3 += reject_k3;
            bs_delta += m_delta; bs_k1 += m_k1; bs_k2 += m_k2; bs_k3 += m_k3;
        }
        if (s_n_valid) s_n_valid[j] = (int32_t)q_valid;
        if (s_n_clipped) s_n_clipped[j] = (int32_t)q_clip;
        if (s_n_nan) s_n_nan[j] = (int32_t)q_nan;
        if (s_mean_delta) s_mean_delta[j] = m_delta;
        if (s_mean_k1) s_mean_k1[j] = m_k1;
        if (s_mean_k2) s_mean_k2[j] = m_k2;
        if (s_mean_k3) s_mean_k3[j] = m_k3;
        if (s_mean_w) s_mean_w[j] = m_w;
        if (s_reject) s_reject[j] = (uint8_t)reject;
        if (s_reject_k3) s_reject_k3[j] = (uint8_t)reject_k3;
    }
    if (batch) {
        double nv = (double)b_valid, ns = (double)bs_nonempty;
        batch[OB_TOK_MEAN_DELTA] = safe_div(b_delta, nv);
        batch[OB_TOK_MEAN_K1] = safe_div(b_k1, nv);
        batch[OB_TOK_MEAN_K2] = safe_div(b_k2, nv);
        batch[OB_TOK_MEAN_K3] = safe_div(b_k3, nv);
        batch[OB_SEQ_MEAN_DELTA] = safe_div(bs_delta, ns);
        batch[OB_SEQ_MEAN_K1] = safe_div(bs_k1, ns);
        batch[OB_SEQ_MEAN_K2] = safe_div(bs_k2, ns);
        batch[OB_SEQ_MEAN_K3] = safe_div(bs_k3, ns);
        batch[OB_TOK_MEAN_TIS_W] = safe_div(b_w, nv);
        batch[OB_CLIP_RATIO] = safe_div((double)b_clip, nv);
        batch[OB_NAN_RATIO] = safe_div((double)b_nan, (double)b_in);
        batch[OB_REJECT_FRAC] = safe_div((double)bs_rejected, ns);
        batch[OB_MEAN_ABS_DELTA] = safe_div(b_abs, nv);
        batch[OB_MAX_ABS_DELTA] = b_max;
        batch[OB_N_VALID] = nv;
        batch[OB_N_NAN] = (double)b_nan;
        batch[OB_N_CLIPPED] = (double)b_clip;
        batch[OB_N_SEQ_NONEMPTY] = ns;
        batch[OB_N_SEQ_REJECTED] = (double)bs_rejected;
        batch[OB_REJECT_K3_FRAC] = safe_div((double)bs_rejected_k3, ns);
        batch[OB_N_SEQ_REJECTED_K3] = (double)bs_rejected_k3;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Extra mismatch metrics: quantiles, extreme tokens, relative diff    */
/* ------------------------------------------------------------------ */

/* Output layout of or_mismatch_extras (restated from the definitions). */
enum {
    OX_N_VALID, OX_N_EXTREME, OX_EXTREME_FRAC, OX_MEAN_REL_DIFF,
    OX_RATIO_Q0, OX_ABS_Q0 = OX_RATIO_Q0 + 4, OX_NFIELDS = OX_ABS_Q0 + 4
};
#define OX_MAX_Q 4

int or_extras_nfields(void) { return OX_NFIELDS; }

static int cmp_double(const void* a, const void* b)
{
    double x = *(const double*)a, y = *(const double*)b;
    return (x > y) - (x < y);
}

/* Ascending sort of x[0..m): up to nthreads pieces sorted by qsort, each in
 * its own thread, then merged (at every step the smallest head of the
 * pieces, the first piece on a tie).  Sorting fixes the sequence, so the
 * result is the one a single qsort gives; the pieces only spread the work
 * of a few hundred million keys over the host's cores. */
typedef struct { double* a; size_t n; } sort_job;

static void* sort_worker(void* arg)
{
    sort_job* j = (sort_job*)arg;
    qsort(j->a, j->n, sizeof(double), cmp_double);
    return NULL;
}

#define OX_MAX_SORT_PIECES 16

static int sort_doubles(double* x, int64_t m, int nthreads)
{
    if (nthreads > OX_MAX_SORT_PIECES) nthreads = OX_MAX_SORT_PIECES;
    if (nthreads < 2 || m < (int64_t)1 << 20) {
        qsort(x, (size_t)m, sizeof(double), cmp_double);
        return 0;
    }
    sort_job jobs[OX_MAX_SORT_PIECES];
    pthread_t th[OX_MAX_SORT_PIECES];
    size_t pos[OX_MAX_SORT_PIECES], end[OX_MAX_SORT_PIECES];
    const int64_t per = (m + nthreads - 1) / nthreads;
    int np = 0;
    for (int64_t b = 0; b < m; b += per, ++np) {
        const int64_t e = b + per < m ? b + per : m;
        jobs[np].a = x + b;
        jobs[np].n = (size_t)(e - b);
        pos[np] = (size_t)b;
        end[np] = (size_t)e;
    }
    for (int i = 0; i < np; ++i) pthread_create(&th[i], NULL, sort_worker, &jobs[i]);
    for (int i = 0; i < np; ++i) pthread_join(th[i], NULL);
    double* out = (double*)malloc(sizeof(double) * (size_t)m);
    if (!out) return -1;
    for (int64_t k = 0; k < m; ++k) {
        int best = -1;
        for (int i = 0; i < np; ++i)
            if (pos[i] < end[i] && (best < 0 || x[pos[i]] < x[pos[best]])) best = i;
        out[k] = x[pos[best]++];
    }
    memcpy(x, out, sizeof(double) * (size_t)m);
    free(out);
    return 0;
}

/* Quantile q of the ascending array x[0..m) with linear interpolation
 * between order statistics: position q (m - 1), lower index its floor,
 * upper index one above (capped at m - 1), weight the fractional part.
 * Empty array: 0. */
static double quantile_sorted(const double* x, int64_t m, double q)
{
    if (m == 0) return 0.0;
    double pos = q * (double)(m - 1);
    double fl = floor(pos);
    int64_t lo = (int64_t)fl;
    int64_t hi = lo + 1 < m ? lo + 1 : lo;
    double frac = pos - fl;
    return x[lo] + (x[hi] - x[lo]) * frac;
}

/*
 * Batch metrics over the valid tokens (mask != 0 and a finite
 * delta = lt - lr computed in double):
 *   out[OX_N_VALID]        number of valid tokens;
 *   out[OX_N_EXTREME]      valid tokens with |delta| > tok_tau, and
 *   out[OX_EXTREME_FRAC]   their share of the valid tokens ("训推一致性与
 *                          determinism", section 7: the extreme-token rate);
 *   out[OX_MEAN_REL_DIFF]  mean of |lt - lr| / (|lt| + 1e-8) ("RL: Training
 *                          Inference Mismatch", training/inference
 *                          consistency section: masked mean of rel_diff);
 *   out[OX_RATIO_Q0 + i]   quantile ratio_q[i] of r = exp(delta), and
 *   out[OX_ABS_Q0 + i]     quantile abs_q[i] of |delta| (same Atlas section:
 *                          ratio quantiles and the p95 of the absolute
 *                          difference), each by sorting the values and
 *                          interpolating linearly; unused slots are 0.
 * With no valid token every ratio and quantile is 0.  Returns 0, or -1 on
 * bad arguments (probabilities outside [0, 1], NaN tok_tau, more than
 * OX_MAX_Q probabilities of a kind, null required pointer).
 */
int or_mismatch_extras(const float* lt, const float* lr, const uint8_t* mask,
                       int64_t n, double tok_tau,
                       const double* ratio_q, int n_ratio_q,
                       const double* abs_q, int n_abs_q, double* out)
{
    if (n < 0 || (n > 0 && (!lt || !lr)) || !out || isnan(tok_tau) ||
        n_ratio_q < 0 || n_ratio_q > OX_MAX_Q || n_abs_q < 0 ||
        n_abs_q > OX_MAX_Q || (n_ratio_q > 0 && !ratio_q) ||
        (n_abs_q > 0 && !abs_q))
        return -1;
    for (int i = 0; i < n_ratio_q; ++i)
        if (!(ratio_q[i] >= 0.0 && ratio_q[i] <= 1.0)) return -1;
    for (int i = 0; i < n_abs_q; ++i)
        if (!(abs_q[i] >= 0.0 && abs_q[i] <= 1.0)) return -1;

    double* ratio = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* absd = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!ratio || !absd) { free(ratio); free(absd); return -1; }

    int64_t m = 0, n_ext = 0;
    double rel_sum = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        if (mask && mask[t] == 0) continue;
        double delta = (double)lt[t] - (double)lr[t];
        if (!isfinite(delta)) continue;
        ratio[m] = exp(delta);
        absd[m] = fabs(delta);
        if (fabs(delta) > tok_tau) n_ext++;
        rel_sum += fabs(delta) / (fabs((double)lt[t]) + 1e-8);
        m++;
    }
    const int nsort = or_available_cpus();
    if (sort_doubles(ratio, m, nsort) != 0 || sort_doubles(absd, m, nsort) != 0) {
        free(ratio);
        free(absd);
        return -1;
    }

    for (int i = 0; i < OX_NFIELDS; ++i) out[i] = 0.0;
    out[OX_N_VALID] = (double)m;
    out[OX_N_EXTREME] = (double)n_ext;
    out[OX_EXTREME_FRAC] = safe_div((double)n_ext, (double)m);
    out[OX_MEAN_REL_DIFF] = safe_div(rel_sum, (double)m);
    for (int i = 0; i < n_ratio_q; ++i)
        out[OX_RATIO_Q0 + i] = quantile_sorted(ratio, m, ratio_q[i]);
    for (int i = 0; i < n_abs_q; ++i)
        out[OX_ABS_Q0 + i] = quantile_sorted(absd, m, abs_q[i]);
    free(ratio);
    free(absd);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Backward of the selected-token log-probability                      */
/* ------------------------------------------------------------------ */

/*
 * With logp_t = z_t[a_t] - log sum_v exp z_t[v] and z_t = W h_t, the
 * derivative of logp_t by the logit z_t[v] is [v == a_t] - p_t[v], p_t the
 * softmax of z_t.  For an upstream gradient g_t = dL/dlogp_t:
 *   dz_t[v]  = g_t ([v == a_t] - p_t[v])
 *   dh_t[k]  = sum_v dz_t[v] W[v, k]            (v ascending)
 *   dW[v, k] = sum_t dz_t[v] h[t, k]            (t ascending)
 * ("RL: Training Inference Mismatch", "log p" chain, differentiated; the
 * policy-gradient term grad log q of its importance-sampling section.)
 *
 * Only tokens with g_t != 0 contribute.  dh is written for the token rows
 * dh_rows[0..n_dh) ([n_dh, d]), dW for the vocabulary rows dw_rows[0..n_dw)
 * ([n_dw, d]).  An out-of-range id contributes nothing (its logp is NaN in
 * the forward).  nthreads <= 0: all CPUs.  Returns 0, or -1 on bad
 * arguments or memory.
 */
typedef struct {
    const void* h; int64_t ldh; const void* w; int64_t ldw;
    const int32_t* ids; const double* g; int dtype; int64_t d, v;
    const int64_t* tok; int64_t ntok;     /* tokens with g != 0 */
    double* dz;                           /* [ntok, v] */
    int64_t begin, end;
} bw_job;

static void* bw_dz_worker(void* arg)
{
    bw_job* j = (bw_job*)arg;
    const int64_t d = j->d, v = j->v;
    double* hd = (double*)malloc(sizeof(double) * (size_t)d);
    double* z = (double*)malloc(sizeof(double) * (size_t)v);
    if (!hd || !z) { free(hd); free(z); return (void*)1; }
    for (int64_t i = j->begin; i < j->end; ++i) {
        const int64_t t = j->tok[i];
        double* dz = j->dz + i * v;
        const int32_t a = j->ids[t];
        if (!(a >= 0 && (int64_t)a < v)) {
            for (int64_t c = 0; c < v; ++c) dz[c] = 0.0;
            continue;
        }
        for (int64_t k = 0; k < d; ++k) hd[k] = load_elem(j->h, j->dtype, t * j->ldh + k);
        double m = -INFINITY;
        for (int64_t c = 0; c < v; ++c) {
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k) acc += hd[k] * load_elem(j->w, j->dtype, c * j->ldw + k);
            z[c] = acc;
            if (acc > m) m = acc;
        }
        double s = 0.0;
        for (int64_t c = 0; c < v; ++c) s += exp(z[c] - m);
        const double lse = m + log(s);
        const double g = j->g[t];
        for (int64_t c = 0; c < v; ++c) {
            const double p = exp(z[c] - lse);
            dz[c] = g * ((c == a ? 1.0 : 0.0) - p);
        }
    }
    free(hd); free(z);
    return NULL;
}

typedef struct {
    const void* h; int64_t ldh; const void* w; int64_t ldw; int dtype; int64_t d, v;
    const int64_t* tok; int64_t ntok; const double* dz;
    const int64_t* rows; double* out; int64_t begin, end;
    int which;                            /* 0: dh rows (tokens), 1: dW rows (vocab) */
    const int64_t* tok_index;             /* dh: position of a token in tok, or -1 */
} bw_out_job;

static void* bw_out_worker(void* arg)
{
    bw_out_job* j = (bw_out_job*)arg;
    const int64_t d = j->d, v = j->v;
    for (int64_t i = j->begin; i < j->end; ++i) {
        double* o = j->out + i * d;
        for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
        if (j->which == 0) {
            const int64_t pos = j->tok_index[i];
            if (pos < 0) continue;                       /* g_t == 0: dh_t = 0 */
            const double* dz = j->dz + pos * v;
            for (int64_t c = 0; c < v; ++c) {
                const double f = dz[c];
                for (int64_t k = 0; k < d; ++k) o[k] += f * load_elem(j->w, j->dtype, c * j->ldw + k);
            }
        } else {
            const int64_t c = j->rows[i];
            for (int64_t q = 0; q < j->ntok; ++q) {
                const int64_t t = j->tok[q];
                const double f = j->dz[q * v + c];
                for (int64_t k = 0; k < d; ++k) o[k] += f * load_elem(j->h, j->dtype, t * j->ldh + k);
            }
        }
    }
    return NULL;
}

static int run_threads(void* jobs, size_t job_size, int nthreads, void* (*fn)(void*))
{
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!th) return -1;
    int bad = 0;
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, fn, (char*)jobs + i * job_size);
    if (fn((char*)jobs) != NULL) bad = 1;
    for (int i = 1; i < nthreads; ++i) {
        void* r = NULL;
        pthread_join(th[i], &r);
        if (r != NULL) bad = 1;
    }
    free(th);
    return bad ? -1 : 0;
}

int or_logprob_backward(const void* h, int64_t ldh, const void* w, int64_t ldw,
                        const int32_t* ids, const double* g, int dtype,
                        int64_t n, int64_t d, int64_t v,
                        const int64_t* dh_rows, int64_t n_dh, double* dh,
                        const int64_t* dw_rows, int64_t n_dw, double* dw, int nthreads)
{
    if (!h || !w || !ids || !g || n < 0 || d <= 0 || v <= 0 || ldh < d || ldw < d ||
        (dtype != OR_BF16 && dtype != OR_F32) || n_dh < 0 || n_dw < 0 ||
        (n_dh > 0 && (!dh_rows || !dh)) || (n_dw > 0 && (!dw_rows || !dw)))
        return -1;
    for (int64_t i = 0; i < n_dh; ++i) if (dh_rows[i] < 0 || dh_rows[i] >= n) return -1;
    for (int64_t i = 0; i < n_dw; ++i) if (dw_rows[i] < 0 || dw_rows[i] >= v) return -1;
    if (nthreads <= 0) nthreads = or_available_cpus();

    /* tokens that contribute, ascending */
    int64_t ntok = 0;
    for (int64_t t = 0; t < n; ++t) ntok += g[t] != 0.0;
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)(ntok > 0 ? ntok : 1));
    double* dz = (double*)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok * v : 1));
    int64_t* tok_index = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_dh > 0 ? n_dh : 1));
    if (!tok || !dz || !tok_index) { free(tok); free(dz); free(tok_index); return -1; }
    for (int64_t t = 0, q = 0; t < n; ++t) if (g[t] != 0.0) tok[q++] = t;
    for (int64_t i = 0; i < n_dh; ++i) {
        tok_index[i] = -1;
        for (int64_t q = 0; q < ntok; ++q) if (tok[q] == dh_rows[i]) { tok_index[i] = q; break; }
    }
    int rc = 0;
    {
        int nt = nthreads < ntok ? nthreads : (int)(ntok > 0 ? ntok : 1);
        bw_job* jobs = (bw_job*)calloc((size_t)nt, sizeof(bw_job));
        if (!jobs) rc = -1;
        for (int i = 0; rc == 0 && i < nt; ++i) {
            bw_job* j = &jobs[i];
            j->h = h; j->ldh = ldh; j->w = w; j->ldw = ldw; j->ids = ids; j->g = g;
            j->dtype = dtype; j->d = d; j->v = v; j->tok = tok; j->ntok = ntok; j->dz = dz;
            j->begin = ntok * i / nt; j->end = ntok * (i + 1) / nt;
        }
        if (rc == 0) rc = run_threads(jobs, sizeof(bw_job), nt, bw_dz_worker);
        free(jobs);
    }
    for (int which = 0; rc == 0 && which < 2; ++which) {
        const int64_t nrows = which == 0 ? n_dh : n_dw;
        if (nrows == 0) continue;
        int nt = nthreads < nrows ? nthreads : (int)nrows;
        bw_out_job* jobs = (bw_out_job*)calloc((size_t)nt, sizeof(bw_out_job));
        if (!jobs) { rc = -1; break; }
        for (int i = 0; i < nt; ++i) {
            bw_out_job* j = &jobs[i];
            j->h = h; j->ldh = ldh; j->w = w; j->ldw = ldw; j->dtype = dtype; j->d = d; j->v = v;
            j->tok = tok; j->ntok = ntok; j->dz = dz; j->which = which;
            j->rows = which == 0 ? dh_rows : dw_rows; j->out = which == 0 ? dh : dw;
            j->tok_index = tok_index;
            j->begin = nrows * i / nt; j->end = nrows * (i + 1) / nt;
        }
        rc = run_threads(jobs, sizeof(bw_out_job), nt, bw_out_worker);
        free(jobs);
    }
    free(tok); free(dz); free(tok_index);
    return rc;
}

/* ------------------------------------------------------------------ */
/* PPO / GRPO clipped surrogate with truncated importance weights      */
/* ------------------------------------------------------------------ */

enum {
    OP_MEAN_LOSS, OP_CLIP_FRAC, OP_MEAN_RATIO, OP_MEAN_TIS_W, OP_MEAN_CONTRIB,
    OP_N_VALID, OP_N_CLIPPED, OP_N_NAN, OP_NFIELDS
};

int or_ppo_nfields(void) { return OP_NFIELDS; }

/*
 * Per token (mask != 0): the PPO ratio r = exp(logp - logp_old), with
 * logp_old the trainer's recomputed old log-probability ("recompute") or
 * the rollout's ("bypass") (VeXact eq. (3)); the clipped surrogate
 * loss = -w min(r A, clip(r, 1 - eps_lo, 1 + eps_hi) A) (VeXact eq. (2)),
 * w = min(exp(old_train - old_rollout), C) the truncated r_corr weight when
 * tis_c > 0, else 1 (VeXact compensation table, TIS rows: TIS moves the
 * ratio from the trainer's to the rollout's denominator); the zero-centred
 * contribution -(r - 1) A (VeXact eq. (5)); and d loss / d logp =
 * -w [unclipped] r A, where the clip is active iff A > 0 and r > 1 + eps_hi
 * or A < 0 and r < 1 - eps_lo ("RL: Training Inference Mismatch", clipped
 * importance ratios: the gradient is dropped once the ratio leaves the
 * interval on the side that the advantage's sign favours).
 * A token whose inputs give a non-finite r, weight or advantage is counted
 * in n_nan and left out.  grad[t] is the derivative of the token mean of
 * loss over the valid tokens when grad_scale == 0, and of grad_scale times
 * the token sum when grad_scale > 0 (VeXact eq. (2) writes the surrogate per
 * token and leaves the normaliser of the sum open: a trainer divides by a
 * token count taken over all its data-parallel ranks, or by a constant);
 * 0 for tokens left out.  Outputs nullable.
 */
int or_ppo_loss(const float* logp, const float* old_train, const float* old_rollout,
                const float* adv, const uint8_t* mask, int64_t n,
                double eps_lo, double eps_hi, int bypass, double tis_c, double grad_scale,
                double* loss, double* grad, double* ratio, double* contrib,
                uint8_t* clipped, double* batch)
{
    if (n < 0 || (n > 0 && (!logp || !old_train || !old_rollout || !adv)) ||
        !(eps_lo >= 0.0) || !(eps_hi >= 0.0) || isnan(tis_c) ||
        !(grad_scale >= 0.0) || isinf(grad_scale))
        return -1;
    double s_loss = 0, s_r = 0, s_w = 0, s_c = 0;
    int64_t nv = 0, nclip = 0, nnan = 0;
    for (int64_t t = 0; t < n; ++t) {
        double l_t = 0, g_t = 0, r_t = 1, c_t = 0;
        int clip_t = 0;
        if (!mask || mask[t] != 0) {
            const double old = bypass ? (double)old_rollout[t] : (double)old_train[t];
            const double r = exp((double)logp[t] - old);
            const double w = tis_c > 0.0
                ? fmin(exp((double)old_train[t] - (double)old_rollout[t]), tis_c) : 1.0;
            const double a = (double)adv[t];
            if (!isfinite(r) || !isfinite(w) || !isfinite(a)) {
                nnan++;
            } else {
                const double rc = r < 1.0 - eps_lo ? 1.0 - eps_lo : (r > 1.0 + eps_hi ? 1.0 + eps_hi : r);
                const double sur = fmin(r * a, rc * a);
                const int active = (a > 0.0 && r > 1.0 + eps_hi) || (a < 0.0 && r < 1.0 - eps_lo);
                l_t = -w * sur;
                g_t = active ? 0.0 : -w * r * a;
                r_t = r;
                c_t = -(r - 1.0) * a;
                clip_t = active;
                nv++; nclip += active;
                s_loss += l_t; s_r += r; s_w += w; s_c += c_t;
            }
        }
        if (loss) loss[t] = l_t;
        if (grad) grad[t] = g_t;        /* scaled below */
        if (ratio) ratio[t] = r_t;
        if (contrib) contrib[t] = c_t;
        if (clipped) clipped[t] = (uint8_t)clip_t;
    }
    if (grad && grad_scale > 0.0)
        for (int64_t t = 0; t < n; ++t) grad[t] *= grad_scale;
    else if (grad && nv > 0)
        for (int64_t t = 0; t < n; ++t) grad[t] /= (double)nv;
    if (batch) {
        const double dn = (double)nv;
        batch[OP_MEAN_LOSS] = safe_div(s_loss, dn);
        batch[OP_CLIP_FRAC] = safe_div((double)nclip, dn);
        batch[OP_MEAN_RATIO] = safe_div(s_r, dn);
        batch[OP_MEAN_TIS_W] = safe_div(s_w, dn);
        batch[OP_MEAN_CONTRIB] = safe_div(s_c, dn);
        batch[OP_N_VALID] = dn;
        batch[OP_N_CLIPPED] = (double)nclip;
        batch[OP_N_NAN] = (double)nnan;
    }
    return 0;
}
