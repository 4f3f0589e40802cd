// stats.hip — training/rollout mismatch statistics for gfx950.
//
// Per token (mask != 0): delta = lt - lr in fp64 ("Diagnosing Training
// Inference Mismatch ... (VeXact)", eq. (1), token-level TIM), r = e^delta
// ("训推一致性与 determinism", section 2), k1 = -delta, k2 = delta^2/2,
// k3 = (r - 1) - delta ("RL: Training Inference Mismatch", KL-estimator
// table; VeXact K1/K3), truncated IS weight w = min(r, C) with a clip flag
// ("Train-Inference Consistency", section 4).  Per sequence: means over the
// valid tokens and the geometric-mean-ratio rejection flag (VeXact
// compensation table, r_corr-based sequence rejection; exp(mean delta) is
// the geometric mean of r, tested in the log domain).  Per batch: token
// means and the mean of per-sequence means ("RL: Training Inference
// Mismatch", monitoring flow), and the is_* ratios named in
// "Train-Inference Consistency", section 5.
//
// The pass is HBM-bound: 9 bytes per token are read once.  Layout of the
// work:
//   1. window_map: for every window of kSubChunk tokens, the first sequence
//      starting at or after the window start (one thread per sequence).
//   2. stream: one wavefront per window.  It reduces every sub-chunk that
//      *starts* in its window (a sequence's first kSubChunk tokens, or a
//      continuation kSubChunk * k tokens into a sequence), so each wave
//      reads at most 2 * kSubChunk tokens and no search is needed.  A
//      sub-chunk is folded lane-locally in token order, then across the
//      wave with a fixed butterfly; its reduction order depends only on the
//      token offsets inside the sub-chunk, so per-sequence sums do not
//      depend on the rest of the batch.
//   3. seq_finalize: one thread per sequence folds its sub-chunks in
//      ascending order, writes means and flags, and each block folds its
//      sequences into a block partial with a fixed tree.
//   4. batch_finalize: one block folds the block partials in a fixed tree.

#include "tim_internal.h"

#include <math.h>

namespace tim {
namespace {

// Partial sums of one sub-chunk (64 bytes).
struct alignas(16) SubPartial {
    double sd, sk2, sk3, sw, sabs, maxabs;
    int32_t nvalid, nclip, nnan, pad;
};

// Contribution of one sequence to the batch, and the running fold of many.
struct alignas(16) BatchAcc {
    double sd, sk2, sk3, sw, sabs, maxabs;           // token sums
    double md, mk1, mk2, mk3;                        // sums of sequence means
    int64_t nvalid, nclip, nnan, nonempty, rejected;
};

constexpr int kWave = 64;
constexpr int kPerLane = kSubChunk / kWave;   // tokens per lane per sub-chunk
constexpr int kFinBlock = 256;

__device__ __forceinline__ double shfl_xor_d(double x, int m) {
    int lo = __double2loint(x), hi = __double2hiint(x);
    lo = __shfl_xor(lo, m);
    hi = __shfl_xor(hi, m);
    return __hiloint2double(hi, lo);
}

// e^d - 1 - d and e^d - 1 for finite d.  For |d| <= 1/32 a degree-8 Taylor
// polynomial evaluated as d^2 * P(d) (no cancellation; truncation error
// < 2^-60 relative); otherwise the library expm1.
__device__ __forceinline__ void k3_em1(double d, double& k3, double& em1) {
    if (fabs(d) <= 0.03125) {
        double p = 1.0 / 40320.0;
        p = fma(p, d, 1.0 / 5040.0);
        p = fma(p, d, 1.0 / 720.0);
        p = fma(p, d, 1.0 / 120.0);
        p = fma(p, d, 1.0 / 24.0);
        p = fma(p, d, 1.0 / 6.0);
        p = fma(p, d, 0.5);
        k3 = (d * d) * p;
        em1 = d + k3;
    } else {
        em1 = expm1(d);
        k3 = em1 - d;
    }
}

__global__ void __launch_bounds__(256)
window_map_kernel(const int32_t* __restrict__ cu, int64_t s, int64_t nwin,
                  int32_t* __restrict__ fmap) {
    // fmap[w] = first sequence j with cu[j] >= w * kSubChunk, for w < nwin.
    // Sequence j owns the windows w with cu[j-1] < w*SC <= cu[j].
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j > s) return;
    const int64_t hi = cu[j];
    const int64_t lo = j == 0 ? -1 : (int64_t)cu[j - 1];
    const int64_t w_begin = lo < 0 ? 0 : lo / kSubChunk + 1;
    const int64_t w_end = hi / kSubChunk;       // inclusive: w * SC <= hi
    for (int64_t wdx = w_begin; wdx <= w_end && wdx < nwin; ++wdx) fmap[wdx] = (int32_t)j;
}

struct TokOut {
    float *delta, *ratio, *k1, *k2, *k3, *tis_w;
    uint8_t* clipped;
};

// Reduce tokens [a, b) (b - a <= kSubChunk) with one wavefront.  All lanes
// return identical sums.
__device__ __forceinline__ SubPartial reduce_subchunk(
    int64_t a, int64_t b, int lane, const float* __restrict__ lt, const float* __restrict__ lr,
    const uint8_t* __restrict__ mask, const StatsParamsDev& prm, const TokOut& tok) {
    double sd = 0, sk2 = 0, sk3 = 0, sw = 0, sabs = 0, mx = 0;
    int nvalid = 0, nclip = 0, nnan = 0;
    const int iters = (int)((b - a + kWave - 1) / kWave);
    for (int i = 0; i < iters; ++i) {
        const int64_t t = a + lane + (int64_t)kWave * i;
        if (t >= b) continue;
        const bool scored = mask ? mask[t] != 0 : true;
        double d = 0, r = 1, k1 = 0, k2 = 0, k3 = 0, wgt = 0;
        bool clipped = false;
        if (scored) {
            d = (double)lt[t] - (double)lr[t];
            k1 = -d;
            k2 = 0.5 * d * d;
            if (isfinite(d)) {
                double em1;
                k3_em1(d, k3, em1);
                r = 1.0 + em1;
                clipped = d > prm.log_c;
                wgt = clipped ? prm.clip_c : r;
                nvalid += 1;
                nclip += clipped;
                sd += d; sk2 += k2; sk3 += k3; sw += wgt;
                const double ad = fabs(d);
                sabs += ad;
                mx = fmax(mx, ad);
            } else {
                nnan += 1;
                r = exp(d);
                k3 = expm1(d) - d;
            }
        }
        if (tok.delta) tok.delta[t] = (float)d;
        if (tok.ratio) tok.ratio[t] = (float)r;
        if (tok.k1) tok.k1[t] = (float)k1;
        if (tok.k2) tok.k2[t] = (float)k2;
        if (tok.k3) tok.k3[t] = (float)k3;
        if (tok.tis_w) tok.tis_w[t] = (float)wgt;
        if (tok.clipped) tok.clipped[t] = clipped ? 1 : 0;
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        sd += shfl_xor_d(sd, m);
        sk2 += shfl_xor_d(sk2, m);
        sk3 += shfl_xor_d(sk3, m);
        sw += shfl_xor_d(sw, m);
        sabs += shfl_xor_d(sabs, m);
        mx = fmax(mx, shfl_xor_d(mx, m));
        nvalid += __shfl_xor(nvalid, m);
        nclip += __shfl_xor(nclip, m);
        nnan += __shfl_xor(nnan, m);
    }
    SubPartial p;
    p.sd = sd; p.sk2 = sk2; p.sk3 = sk3; p.sw = sw; p.sabs = sabs; p.maxabs = mx;
    p.nvalid = nvalid; p.nclip = nclip; p.nnan = nnan; p.pad = 0;
    return p;
}

__global__ void __launch_bounds__(256)
stats_stream_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                    const uint8_t* __restrict__ mask, const int32_t* __restrict__ cu,
                    int64_t n, int64_t s, int64_t nwin, const int32_t* __restrict__ fmap,
                    StatsParamsDev prm, TokOut tok, SubPartial* __restrict__ first,
                    SubPartial* __restrict__ tail) {
    const int lane = threadIdx.x & 63;
    const int64_t wdx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (wdx >= nwin) return;
    const int64_t win0 = wdx * kSubChunk;
    const int64_t win1 = win0 + kSubChunk < n ? win0 + kSubChunk : n;
    // cu values are clamped to [0, n] and f to [0, s] so that a malformed
    // cu_seqlens (a documented precondition) can give wrong numbers but never
    // an out-of-range access
    auto cuc = [&](int64_t j) -> int64_t {
        const int64_t c = cu[j];
        return c < 0 ? 0 : (c > n ? n : c);
    };
    int64_t f = fmap[wdx];                          // first sequence starting >= win0
    f = f < 0 ? 0 : (f > s ? s : f);

    // continuation sub-chunk of the sequence that started before the window
    const int64_t cf = cuc(f);
    if (f > 0 && cf > win0) {
        const int64_t j = f - 1;
        const int64_t c0 = cuc(j);                  // c0 < win0 < cu[j+1] = cf
        const int64_t k = (win0 - c0 + kSubChunk - 1) / kSubChunk;
        const int64_t a = c0 + k * kSubChunk;
        if (a < win1 && a < cf) {
            const int64_t b = a + kSubChunk < cf ? a + kSubChunk : cf;
            const SubPartial p = reduce_subchunk(a, b, lane, lt, lr, mask, prm, tok);
            if (lane == 0) tail[wdx] = p;
        }
    }
    // first sub-chunk of every sequence that starts inside the window
    for (int64_t j = f; j < s; ++j) {
        const int64_t a = cuc(j);
        if (a >= win1) break;
        const int64_t e = cuc(j + 1);
        if (e <= a) continue;                       // empty sequence
        const int64_t b = a + kSubChunk < e ? a + kSubChunk : e;
        const SubPartial p = reduce_subchunk(a, b, lane, lt, lr, mask, prm, tok);
        if (lane == 0) first[j] = p;
    }
}

__device__ __forceinline__ void acc_add(BatchAcc& x, const BatchAcc& y) {
    x.sd += y.sd; x.sk2 += y.sk2; x.sk3 += y.sk3; x.sw += y.sw; x.sabs += y.sabs;
    x.maxabs = fmax(x.maxabs, y.maxabs);
    x.md += y.md; x.mk1 += y.mk1; x.mk2 += y.mk2; x.mk3 += y.mk3;
    x.nvalid += y.nvalid; x.nclip += y.nclip; x.nnan += y.nnan;
    x.nonempty += y.nonempty; x.rejected += y.rejected;
}

__device__ __forceinline__ BatchAcc acc_zero() {
    BatchAcc a;
    a.sd = a.sk2 = a.sk3 = a.sw = a.sabs = a.maxabs = 0;
    a.md = a.mk1 = a.mk2 = a.mk3 = 0;
    a.nvalid = a.nclip = a.nnan = a.nonempty = a.rejected = 0;
    return a;
}

// Fixed-shape tree over the kFinBlock entries of `buf`, result in buf[0].
__device__ void block_tree(BatchAcc* buf) {
    for (int stride = kFinBlock / 2; stride > 0; stride >>= 1) {
        if ((int)threadIdx.x < stride) acc_add(buf[threadIdx.x], buf[threadIdx.x + stride]);
        __syncthreads();
    }
}

struct SeqOut {
    int32_t *n_valid, *n_clipped, *n_nan;
    double *mean_delta, *mean_k1, *mean_k2, *mean_k3, *mean_tis_w;
    uint8_t* reject;
};

__global__ void __launch_bounds__(kFinBlock)
seq_finalize_kernel(const int32_t* __restrict__ cu, int64_t n, int64_t s, StatsParamsDev prm,
                    const SubPartial* __restrict__ first, const SubPartial* __restrict__ tail,
                    SeqOut so, BatchAcc* __restrict__ blk) {
    __shared__ BatchAcc buf[kFinBlock];
    const int64_t j = (int64_t)blockIdx.x * kFinBlock + threadIdx.x;
    BatchAcc c = acc_zero();
    if (j < s) {
        int64_t a = cu[j], e = cu[j + 1];
        a = a < 0 ? 0 : (a > n ? n : a);            // see stats_stream_kernel
        e = e < a ? a : (e > n ? n : e);
        double sd = 0, sk2 = 0, sk3 = 0, sw = 0, sabs = 0, mx = 0;
        int64_t nvalid = 0, nclip = 0, nnan = 0;
        if (e > a) {
            const int64_t nsub = (e - a + kSubChunk - 1) / kSubChunk;
            for (int64_t k = 0; k < nsub; ++k) {
                const SubPartial p = k == 0 ? first[j] : tail[(a + k * kSubChunk) / kSubChunk];
                sd += p.sd; sk2 += p.sk2; sk3 += p.sk3; sw += p.sw; sabs += p.sabs;
                mx = fmax(mx, p.maxabs);
                nvalid += p.nvalid; nclip += p.nclip; nnan += p.nnan;
            }
        }
        const double nv = (double)nvalid;
        const double md = nvalid ? sd / nv : 0.0;
        const double mk1 = nvalid ? (-sd) / nv : 0.0;
        const double mk2 = nvalid ? sk2 / nv : 0.0;
        const double mk3 = nvalid ? sk3 / nv : 0.0;
        const double mw = nvalid ? sw / nv : 0.0;
        const bool rej = nvalid > 0 && (md < prm.seq_lo || md > prm.seq_hi);
        if (so.n_valid) so.n_valid[j] = (int32_t)nvalid;
        if (so.n_clipped) so.n_clipped[j] = (int32_t)nclip;
        if (so.n_nan) so.n_nan[j] = (int32_t)nnan;
        if (so.mean_delta) so.mean_delta[j] = md;
        if (so.mean_k1) so.mean_k1[j] = mk1;
        if (so.mean_k2) so.mean_k2[j] = mk2;
        if (so.mean_k3) so.mean_k3[j] = mk3;
        if (so.mean_tis_w) so.mean_tis_w[j] = mw;
        if (so.reject) so.reject[j] = rej ? 1 : 0;
        c.sd = sd; c.sk2 = sk2; c.sk3 = sk3; c.sw = sw; c.sabs = sabs; c.maxabs = mx;
        c.nvalid = nvalid; c.nclip = nclip; c.nnan = nnan;
        if (nvalid > 0) {
            c.md = md; c.mk1 = mk1; c.mk2 = mk2; c.mk3 = mk3;
            c.nonempty = 1;
            c.rejected = rej ? 1 : 0;
        }
    }
    buf[threadIdx.x] = c;
    __syncthreads();
    block_tree(buf);
    if (threadIdx.x == 0) blk[blockIdx.x] = buf[0];
}

__global__ void __launch_bounds__(kFinBlock)
batch_finalize_kernel(const BatchAcc* __restrict__ blk, int64_t nblk, double* __restrict__ out) {
    __shared__ BatchAcc buf[kFinBlock];
    BatchAcc c = acc_zero();
    for (int64_t i = threadIdx.x; i < nblk; i += kFinBlock) acc_add(c, blk[i]);
    buf[threadIdx.x] = c;
    __syncthreads();
    block_tree(buf);
    if (threadIdx.x == 0) {
        const BatchAcc& a = buf[0];
        const double nv = (double)a.nvalid, ns = (double)a.nonempty;
        const double nin = (double)(a.nvalid + a.nnan);
        auto dv = [](double x, double y) { return y != 0.0 ? x / y : 0.0; };
        out[0] = dv(a.sd, nv);            // TIM_B_TOK_MEAN_DELTA
        out[1] = dv(-a.sd, nv);           // TIM_B_TOK_MEAN_K1
        out[2] = dv(a.sk2, nv);           // TIM_B_TOK_MEAN_K2
        out[3] = dv(a.sk3, nv);           // TIM_B_TOK_MEAN_K3
        out[4] = dv(a.md, ns);            // TIM_B_SEQ_MEAN_DELTA
        out[5] = dv(a.mk1, ns);           // TIM_B_SEQ_MEAN_K1
        out[6] = dv(a.mk2, ns);           // TIM_B_SEQ_MEAN_K2
        out[7] = dv(a.mk3, ns);           // TIM_B_SEQ_MEAN_K3
        out[8] = dv(a.sw, nv);            // TIM_B_TOK_MEAN_TIS_W
        out[9] = dv((double)a.nclip, nv); // TIM_B_CLIP_RATIO
        out[10] = dv((double)a.nnan, nin);  // TIM_B_NAN_RATIO
        out[11] = dv((double)a.rejected, ns);  // TIM_B_REJECT_FRAC
        out[12] = dv(a.sabs, nv);         // TIM_B_MEAN_ABS_DELTA
        out[13] = a.maxabs;               // TIM_B_MAX_ABS_DELTA
        out[14] = nv;
        out[15] = (double)a.nnan;
        out[16] = (double)a.nclip;
        out[17] = ns;
        out[18] = (double)a.rejected;
    }
}

}  // namespace

bool make_stats_plan(int64_t n, int64_t s, StatsPlan* p) {
    if (n < 0 || s < 0 || s > INT32_MAX - 1 || n > INT32_MAX) return false;
    p->n = n;
    p->s = s;
    p->nwin = (n + kSubChunk - 1) / kSubChunk;
    p->nblk_seq = (s + kFinBlock - 1) / kFinBlock;
    size_t off = 0;
    p->fmap_off = off;  off += align_up((size_t)(p->nwin + 1) * sizeof(int32_t), 256);
    p->first_off = off; off += align_up((size_t)s * sizeof(SubPartial), 256);
    p->tail_off = off;  off += align_up((size_t)p->nwin * sizeof(SubPartial), 256);
    p->blk_off = off;   off += align_up((size_t)(p->nblk_seq > 0 ? p->nblk_seq : 1) * sizeof(BatchAcc), 256);
    p->total_bytes = off;
    return true;
}

hipError_t launch_mismatch_stats(const StatsPlan& p, const float* lt, const float* lr,
                                 const uint8_t* mask, const int32_t* cu,
                                 const StatsParamsDev& prm, const TokenOutPtrs& tok,
                                 const SeqOutPtrs& seq, double* batch, void* workspace,
                                 hipStream_t st) {
    unsigned char* ws = (unsigned char*)workspace;
    int32_t* fmap = (int32_t*)(ws + p.fmap_off);
    SubPartial* first = (SubPartial*)(ws + p.first_off);
    SubPartial* tail = (SubPartial*)(ws + p.tail_off);
    BatchAcc* blk = (BatchAcc*)(ws + p.blk_off);
    TokOut to{tok.delta, tok.ratio, tok.k1, tok.k2, tok.k3, tok.tis_w, tok.clipped};
    SeqOut so{seq.n_valid, seq.n_clipped, seq.n_nan, seq.mean_delta, seq.mean_k1,
              seq.mean_k2, seq.mean_k3, seq.mean_tis_w, seq.reject};
    if (p.nwin > 0) {
        hipLaunchKernelGGL(window_map_kernel, dim3((unsigned)((p.s + 1 + 255) / 256)), dim3(256),
                           0, st, cu, p.s, p.nwin, fmap);
        const int64_t threads = p.nwin * 64;
        hipLaunchKernelGGL(stats_stream_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, st, lt, lr, mask, cu, p.n, p.s, p.nwin, fmap, prm, to, first, tail);
    }
    if (p.s > 0)
        hipLaunchKernelGGL(seq_finalize_kernel, dim3((unsigned)p.nblk_seq), dim3(kFinBlock), 0, st,
                           cu, p.n, p.s, prm, first, tail, so, blk);
    if (batch)
        hipLaunchKernelGGL(batch_finalize_kernel, dim3(1), dim3(kFinBlock), 0, st, blk,
                           p.nblk_seq, batch);
    return hipGetLastError();
}

}  // namespace tim
