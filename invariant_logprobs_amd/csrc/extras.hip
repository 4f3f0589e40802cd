// extras.hip — extra mismatch metrics over the valid tokens of a batch
// (mask != 0 and a finite delta = lt - lr computed in fp64):
//
//   * the extreme-token rate, |delta| > tau ("训推一致性与 determinism",
//     section 7, metric table: fraction of tokens above a threshold);
//   * the masked mean of |lt - lr| / (|lt| + 1e-8) ("RL: Training Inference
//     Mismatch", training/inference consistency section, rel_diff);
//   * quantiles of r = e^delta and of |delta| (same Atlas table: ratio
//     quantiles 0.01 / 0.5 / 0.99 and the p95 of the absolute difference),
//     with linear interpolation between the two order statistics around
//     position q (m - 1), m the number of valid tokens.
//
// Order statistics are found exactly by a radix select over 64-bit keys
// that order like the values: delta's key is its bit pattern with the sign
// bit set for positive values and every bit inverted for negative ones;
// |delta|'s key is its bit pattern (the sign bit is 0).  The first digit of
// |delta|'s key, [0, exponent, two fraction bits], therefore counts the two
// delta digits [1, e, m] and [0, ~e, ~m]: pass 0 histograms delta's keys
// only and derives the other.
// Each pass histograms one digit of the keys that share a target's prefix:
//
//   pass 0: top 14 bits; passes 1-4: 11 bits each; pass 5: the last 6.
//
// A slot is a distinct (kind, prefix) that some unresolved target lies in.
// After each pass a select step moves every unresolved target into the bin
// that holds its rank; a slot whose smallest and largest key are equal
// resolves its targets at once (ties, zero mismatch).  Pass 0 also folds
// the extreme count and the relative difference in a fixed order.
//
// Up to kXFusedMax tokens, one block does everything (xsel_fused): the
// tokens' keys and every histogram live in LDS.  Above,
// each pass is three launches:
//
//   xsel_pass    every block histograms its share in LDS and writes it with
//                plain stores, with its key range per slot.  Pass 0 also
//                copies the keys whose first digit lies in a predicted
//                window of some target into a region of the workspace owned
//                by the block (capped; an overflow is flagged), and passes
//                1-5 read those regions instead of the 9 bytes per token of
//                the inputs, so the inputs are read once.  The windows come
//                from a sample (below); whether they hold every target is
//                checked exactly after pass 0's select step, from the full
//                first-digit histogram.  If one does not (or a region
//                overflowed), pass 1 reads the inputs again and copies the
//                keys that lie in any slot, as it would without a sample,
//                and passes 2-5 read those.
//   xsel_reduce  sums the block histograms bin by bin (integers: the order
//                does not matter).
//   xsel_select  one block runs the select step.
//
// The sample (xsel_sample, xsel_predict): 16 consecutive tokens out of
// every 1024 (about 1.6 % of the tokens, each group most often a sequence of
// its own), their delta keys' first digits histogrammed; each target's
// window is the first-digit bins holding the sample ranks within
// 8 sqrt(m q (1 - q)) + 64 of q (m - 1), m the sample's valid tokens.  The
// sample only decides how much is copied: which keys are selected, and so
// every result, does not depend on it.
//
// Once every target is resolved the remaining launches return at once.
//
// Every step is exact integer work except the per-token relative
// difference (one fp64 division, as the definition states) and its sum,
// whose order depends only on n.  The results are therefore deterministic,
// and the selected order statistics are bit-exact.

#include "tim_internal.h"

#include <math.h>

namespace tim {
namespace {

constexpr int kXThreads = 1024;          // threads per block of the pass, select and fused kernels
constexpr int kXUnroll = 8;              // tokens per thread per loop trip
constexpr int kXMaxTargets = 2 * kXMaxQ;
constexpr int kXMaxSlots = kXMaxTargets;
constexpr int kXLdsBins = 16384;         // 2 slots x 2^13 or 8 slots x 2^11
constexpr int kXPerThreadFused = kXFusedMax / kXThreads;
constexpr int kXReduceBins = 64;         // bins per reduce block
constexpr int kXReduceGroups = 16;       // pass-block groups per bin
constexpr int kXReduceThreads = kXReduceBins * kXReduceGroups;
constexpr int kXFinThreads = 256;

__host__ __device__ constexpr int digit_bits(int pass) {
    return pass == 0 ? 14 : (pass < kXPasses - 1 ? 11 : 6);
}
__host__ __device__ constexpr int bits_before(int pass) {
    return pass == 0 ? 0 : 14 + 11 * (pass - 1);
}
static_assert(bits_before(kXPasses - 1) + digit_bits(kXPasses - 1) == 64, "64 key bits");
static_assert((1 << digit_bits(0)) <= kXLdsBins, "pass 0: delta's first digit");
static_assert(kXMaxSlots * (1 << digit_bits(1)) <= kXLdsBins, "later passes: one slot per target");
static_assert(kXFusedMax % kXThreads == 0, "whole tokens per thread in the fused kernel");

struct XTarget {
    uint64_t prefix;   // key bits fixed so far (the top bits_before(pass) bits)
    uint64_t rank;     // rank among the valid keys of its kind sharing the prefix
    uint64_t key;      // the order statistic's key, once resolved
    int32_t kind;      // 0: delta, 1: |delta|
    int32_t resolved;
    int32_t slot;      // histogram slot in the coming pass
    int32_t pad;
};

struct XSlot {
    uint64_t prefix;
    int32_t kind, pad;
};

struct XState {
    XTarget tgt[kXMaxTargets];
    XSlot slot[kXMaxSlots];
    int32_t ntgt, nslots, all_done, pad;
    uint64_t nvalid;
};

struct XPart {
    double rel;        // sum of |delta| / (|lt| + 1e-8)
    uint64_t next;     // tokens with |delta| > tau
    uint64_t nvalid;
    uint64_t pad;
};

__device__ __forceinline__ uint64_t key_delta(double d) {
    const uint64_t u = __builtin_bit_cast(uint64_t, d);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
// a / b for finite a >= 0 and b in [1e-8, 2^128]: the hardware reciprocal
// refined by two Newton steps, then one correction of the quotient
// (Markstein's sequence).  It is the compiler's IEEE division without the
// operand scaling and special-value fixup steps, which change nothing for
// such operands (no quotient or reciprocal can overflow, underflow or be
// special), so the result is the correctly rounded quotient.
__device__ __forceinline__ double div_in_range(double a, double b) {
    double y = __builtin_amdgcn_rcp(b);
    double e = fma(-b, y, 1.0);
    y = fma(y, e, y);
    e = fma(-b, y, 1.0);
    y = fma(y, e, y);
    const double q = a * y;
    return fma(fma(-b, q, a), y, q);
}
// min and max of finite doubles as single instructions (no NaN can reach
// them, so no canonicalisation)
__device__ __forceinline__ double min_fin(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ double max_fin(double a, double b) {
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// |delta|'s key from delta's key: the bit pattern of |delta|
__device__ __forceinline__ uint64_t key_abs_of(uint64_t k0) {
    return ((k0 >> 63) ? k0 : ~k0) & 0x7FFFFFFFFFFFFFFFull;
}

// Bin D of |delta|'s first-pass histogram from delta's (14-bit digits).
__device__ __forceinline__ uint32_t abs_root_bin(const uint32_t* h, int d) {
    return d < 0x2000 ? h[0x2000 | d] + h[0x1FFF ^ d] : 0u;
}
__device__ __forceinline__ double value_of(uint64_t k, int kind) {
    uint64_t u;
    if (kind == 0) u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    else u = k;
    return __builtin_bit_cast(double, u);
}

struct QPos {
    uint64_t lo, hi;   // the two order statistics' ranks
    double frac;       // interpolation weight
};

// Position q (m - 1) of probability q among m >= 1 sorted values.  Each
// operation is rounded on its own: no fused multiply-add may join the
// product and the subtraction.
__device__ __attribute__((noinline)) QPos quantile_pos(double q, uint64_t m) {
#pragma clang fp contract(off)
    const double pos = q * (double)(m - 1);
    const double fl = floor(pos);
    QPos r;
    r.lo = (uint64_t)fl;
    r.hi = r.lo + 1 < m ? r.lo + 1 : r.lo;
    r.frac = pos - fl;
    return r;
}

// a + (b - a) f with each of the three operations rounded on its own (no
// fused multiply-add), as the quantile definition is written.
__device__ __attribute__((noinline)) double interpolate(double a, double b, double f) {
#pragma clang fp contract(off)
    return a + (b - a) * f;
}

// Sum over a block of kT threads, in a fixed tree; every thread gets it.
template <int kT, typename T>
__device__ T block_sum(T x, T* sh) {
    sh[threadIdx.x] = x;
    __syncthreads();
    for (int s = kT / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
        __syncthreads();
    }
    const T r = sh[0];
    __syncthreads();
    return r;
}

// Exclusive prefix sum of integers over a block of kT threads: shuffle scans
// within each wave, then one wave scans the wave totals (sh holds them).
template <int kT>
__device__ uint64_t block_excl_scan(uint64_t x, uint64_t* sh) {
    static_assert(kT % 64 == 0 && kT / 64 <= 64, "whole waves, at most 64");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint64_t v = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    if (lane == 63) sh[w] = v;                           // inclusive wave total
    __syncthreads();
    if (w == 0) {
        uint64_t t = lane < kT / 64 ? sh[lane] : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t y = __shfl_up(t, o);
            if (lane >= o) t += y;
        }
        if (lane < kT / 64) sh[lane] = t;
    }
    __syncthreads();
    const uint64_t r = (w > 0 ? sh[w - 1] : 0) + v - x;
    __syncthreads();                                     // sh is free again
    return r;
}

// Targets (a lower and an upper order statistic per probability, delta's
// first) and one root slot per key kind present.  One thread.
__device__ void init_state(XState* st, const XParamsDev& prm) {
    const int root_abs = prm.nrq > 0 ? 1 : 0;
    st->ntgt = 2 * (prm.nrq + prm.naq);
    st->nslots = (prm.nrq > 0 ? 1 : 0) + (prm.naq > 0 ? 1 : 0);
    st->all_done = 0;
    st->pad = 0;
    st->nvalid = 0;
    for (int t = 0; t < kXMaxTargets; ++t) {
        const int kind = t < 2 * prm.nrq ? 0 : 1;
        st->tgt[t] = XTarget{0, 0, 0, kind, 0, kind == 0 ? 0 : root_abs, 0};
    }
    for (int k = 0; k < kXMaxSlots; ++k) st->slot[k] = XSlot{0, 0, 0};
    if (prm.naq > 0) st->slot[root_abs].kind = 1;
}

// Pass 0, once the number of valid tokens is known: each probability's two
// ranks.  One thread.
__device__ void set_ranks(XState& st, uint64_t nv, const XParamsDev& prm) {
    st.nvalid = nv;
    for (int t = 0; t < st.ntgt; t += 2) {
        const int i = t / 2;
        const double q = i < prm.nrq ? prm.rq[i] : prm.aq[i - prm.nrq];
        const QPos qp = nv > 0 ? quantile_pos(q, nv) : QPos{0, 0, 0.0};
        st.tgt[t].rank = qp.lo;
        st.tgt[t + 1].rank = qp.hi;
        if (nv == 0) st.tgt[t].resolved = st.tgt[t + 1].resolved = 1;
    }
    if (nv == 0 || st.ntgt == 0) st.all_done = 1;
}

// The slots of a pass, in registers (the same values in every lane).
struct Slots {
    uint64_t pre[kXMaxSlots];
    int kind[kXMaxSlots];
    int n;
};

__device__ __forceinline__ void load_slots(Slots& sl, const XState* st) {
    sl.n = st->nslots;
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) {
        sl.pre[s] = s < sl.n ? st->slot[s].prefix : 0;
        sl.kind[s] = s < sl.n ? st->slot[s].kind : 0;
    }
}

// Pass 0: delta's key into the one first-digit histogram, and its range.
__device__ __forceinline__ void visit_root(uint64_t k0, uint32_t* hist, uint64_t& a, uint64_t& b) {
    atomicAdd(&hist[(uint32_t)(k0 >> 50)], 1u);
    a = k0 < a ? k0 : a;
    b = k0 > b ? k0 : b;
}

// Passes 1-5: counts a token's keys in every slot whose prefix they share;
// returns whether any slot took it.  kHigh: prefix and digit lie in the top
// 32 bits (pass 1), and the tests use the keys' upper halves.
template <bool kHigh>
__device__ __forceinline__ bool visit(uint64_t k0, const Slots& sl, int before, int bits,
                                      uint32_t* hist, uint64_t (&lmn)[kXMaxSlots],
                                      uint64_t (&lmx)[kXMaxSlots]) {
    const uint64_t k1 = key_abs_of(k0);
    bool any = false;
    if (kHigh) {
        const uint32_t h0 = (uint32_t)(k0 >> 32), h1 = (uint32_t)(k1 >> 32);
        const int ps = 32 - before, ds = 32 - before - bits;
        const uint32_t p0 = h0 >> ps, p1 = h1 >> ps;
        const uint32_t dm = (1u << bits) - 1;
#pragma unroll
        for (int s = 0; s < kXMaxSlots; ++s) {
            if (s >= sl.n) break;
            const bool ka = sl.kind[s] != 0;
            if ((ka ? p1 : p0) == (uint32_t)sl.pre[s]) {
                atomicAdd(&hist[(s << bits) | (((ka ? h1 : h0) >> ds) & dm)], 1u);
                const uint64_t k = ka ? k1 : k0;
                lmn[s] = k < lmn[s] ? k : lmn[s];
                lmx[s] = k > lmx[s] ? k : lmx[s];
                any = true;
            }
        }
        return any;
    }
    const int shift = 64 - before - bits;
    const uint64_t dmask = (1ull << bits) - 1;
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) {
        if (s >= sl.n) break;
        const uint64_t k = sl.kind[s] ? k1 : k0;
        if ((k >> (64 - before)) == sl.pre[s]) {
            atomicAdd(&hist[(s << bits) | (uint32_t)((k >> shift) & dmask)], 1u);
            lmn[s] = k < lmn[s] ? k : lmn[s];
            lmx[s] = k > lmx[s] ? k : lmx[s];
            any = true;
        }
    }
    return any;
}

// Per-slot minimum and maximum into LDS: wave butterflies, then one LDS
// atomic per wave.  Every lane of the wave takes part.
__device__ __forceinline__ void flush_range(int nslots, uint64_t (&lmn)[kXMaxSlots],
                                            uint64_t (&lmx)[kXMaxSlots],
                                            unsigned long long* smn, unsigned long long* smx) {
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) {
        if (s >= nslots) break;
        uint64_t a = lmn[s], b = lmx[s];
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t a2 = __shfl_xor(a, o), b2 = __shfl_xor(b, o);
            a = a2 < a ? a2 : a;
            b = b2 > b ? b2 : b;
        }
        if ((threadIdx.x & 63) == 0) {
            atomicMin(&smn[s], (unsigned long long)a);
            atomicMax(&smx[s], (unsigned long long)b);
        }
    }
}

// One select step over this pass's histograms (slot s at h + (s << bits))
// and key ranges.  Every thread of a kXThreads block calls it; st is in LDS.
// Ends with a barrier, st then holds the next pass's slots.
__device__ void select_step(XState& st, int pass, const uint32_t* h,
                            const unsigned long long* mn, const unsigned long long* mx,
                            uint64_t* sh, uint64_t* fdig, uint64_t* frank) {
    const int tid = threadIdx.x;
    const int ntgt = st.ntgt, nslots = st.nslots;
    const int bits = digit_bits(pass), before = bits_before(pass);
    const int nb = 1 << bits;
    const int per = nb > kXThreads ? nb / kXThreads : 1;   // bins per thread
    // a bucket holding one key value resolves its targets at once
    if (tid == 0) {
        for (int t = 0; t < ntgt; ++t) {
            XTarget& g = st.tgt[t];
            // pass 0 knows the range of delta's keys only (range slot 0)
            const bool ranged = pass > 0 || st.slot[g.slot].kind == 0;
            if (!g.resolved && ranged && mn[g.slot] == mx[g.slot]) { g.resolved = 1; g.key = mn[g.slot]; }
        }
    }
    __syncthreads();
    // one scan per slot; every unresolved target of the slot finds its bin in
    // it (the thread holding that bin records digit and remaining rank)
    const int b0 = tid * per;
    for (int s = 0; s < nslots; ++s) {
        bool used = false;
        for (int t = 0; t < ntgt; ++t) used |= !st.tgt[t].resolved && st.tgt[t].slot == s;
        if (!used) continue;                                // uniform: same LDS state
        // pass 0 holds delta's histogram only: |delta|'s root is derived
        const bool derive = pass == 0 && st.slot[s].kind == 1;
        const uint32_t* hs = pass == 0 ? h : h + ((size_t)s << bits);
        // counts and ranks are below 2^31 (n is): 32-bit sums; the bins are
        // read again per target rather than held in registers
        auto bin = [&](int k) -> uint32_t {
            return derive ? abs_root_bin(h, b0 + k) : hs[b0 + k];
        };
        uint32_t mine = 0;
        if (b0 < nb)
            for (int k = 0; k < per; ++k) mine += bin(k);
        const uint32_t c0 = (uint32_t)block_excl_scan<kXThreads>(mine, sh);
        for (int t = 0; t < ntgt; ++t) {
            if (st.tgt[t].resolved || st.tgt[t].slot != s) continue;
            const uint32_t rank = (uint32_t)st.tgt[t].rank;
            if (b0 >= nb || rank - c0 >= mine) continue;    // not among this thread's bins
            uint32_t c = c0;
            for (int k = 0; k < per; ++k) {
                const uint32_t hk = bin(k);
                if (rank - c < hk) { fdig[t] = (uint64_t)(b0 + k); frank[t] = rank - c; }
                c += hk;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        for (int t = 0; t < ntgt; ++t) {
            XTarget& g = st.tgt[t];
            if (g.resolved) continue;
            g.prefix = before == 0 ? fdig[t] : ((g.prefix << bits) | fdig[t]);
            g.rank = frank[t];
            if (before + bits == 64) { g.resolved = 1; g.key = g.prefix; }
        }
        // slots of the next pass: one per distinct (kind, prefix) among the
        // unresolved targets, in target order
        int ns = 0;
        for (int t = 0; t < ntgt; ++t) {
            XTarget& g = st.tgt[t];
            if (g.resolved) continue;
            int k = 0;
            while (k < ns && !(st.slot[k].kind == g.kind && st.slot[k].prefix == g.prefix)) ++k;
            if (k == ns) {
                st.slot[ns].prefix = g.prefix;
                st.slot[ns].kind = g.kind;
                ++ns;
            }
            g.slot = k;
        }
        st.nslots = ns;
        if (ns == 0) st.all_done = 1;
    }
    __syncthreads();
}

// The output vector.  One thread.
__device__ void write_outputs(double* out, const XParamsDev& prm, const XState& st, double rel,
                              uint64_t next, uint64_t nv) {
    const double dnv = (double)nv;
    out[kXOutNValid] = dnv;
    out[kXOutNExtreme] = (double)next;
    out[kXOutExtremeFrac] = nv ? (double)next / dnv : 0.0;
    out[kXOutMeanRelDiff] = nv ? rel / dnv : 0.0;
    for (int i = 0; i < kXMaxQ; ++i) {
        out[kXOutRatioQ + i] = 0.0;
        out[kXOutAbsQ + i] = 0.0;
    }
    if (nv == 0) return;
    const int nq = prm.nrq + prm.naq;
    for (int i = 0; i < nq; ++i) {
        const bool ratio = i < prm.nrq;
        const double q = ratio ? prm.rq[i] : prm.aq[i - prm.nrq];
        const QPos qp = quantile_pos(q, nv);
        const int kind = ratio ? 0 : 1;
        double a = value_of(st.tgt[2 * i].key, kind);
        double b = value_of(st.tgt[2 * i + 1].key, kind);
        if (ratio) { a = exp(a); b = exp(b); }
        const double v = interpolate(a, b, qp.frac);
        if (ratio) out[kXOutRatioQ + i] = v;
        else out[kXOutAbsQ + i - prm.nrq] = v;
    }
}

// ---------------------------------------------------------------------------
// Up to kXFusedMax tokens: one block, keys and histograms in LDS.  Thread
// tid takes tokens tid + kXThreads j.
// ---------------------------------------------------------------------------

template <bool kMask>
__global__ void __launch_bounds__(kXThreads)
xsel_fused_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                  const uint8_t* __restrict__ mask, uint32_t n, XParamsDev prm,
                  double* __restrict__ out) {
    __shared__ uint32_t hist[kXLdsBins];
    // delta's key per token; 0 (the bit pattern of a NaN, which no finite
    // delta has) marks a token that does not count
    __shared__ uint64_t keys[kXFusedMax];
    __shared__ XState st;
    __shared__ uint64_t sh[kXThreads];
    __shared__ unsigned long long smn[kXMaxSlots], smx[kXMaxSlots];
    __shared__ uint64_t fdig[kXMaxTargets], frank[kXMaxTargets];
    const int tid = threadIdx.x;
    if (tid == 0) init_state(&st, prm);

    double rel = 0.0;
    uint32_t next = 0, nval = 0;
    if (n == 0)                                            // uniform; pointers may be null
        for (int j = 0; j < kXPerThreadFused; ++j) keys[tid + kXThreads * j] = 0;
    else
#pragma unroll
    for (int j = 0; j < kXPerThreadFused; ++j) {
        const uint32_t t = (uint32_t)(tid + kXThreads * j);
        const uint32_t tc = t < n ? t : 0;                 // n >= 1 here: in bounds
        const float x = lt[tc];
        const float y = lr[tc];
        const bool in = t < n && (!kMask || mask[tc] != 0);
        const double d = (double)x - (double)y;
        const bool valid = in && isfinite(d);
        uint64_t k = 0;
        if (valid) {
            k = key_delta(d);
            rel += fabs(d) / (fabs((double)x) + 1e-8);
            next += fabs(d) > prm.tok_tau ? 1u : 0u;
            ++nval;
        }
        keys[t] = k;
    }
    double* dsh = reinterpret_cast<double*>(sh);
    rel = block_sum<kXThreads>(rel, dsh);
    const uint64_t next_all = block_sum<kXThreads>((uint64_t)next, sh);
    const uint64_t nv = block_sum<kXThreads>((uint64_t)nval, sh);
    if (tid == 0) set_ranks(st, nv, prm);
    __syncthreads();

    for (int pass = 0; pass < kXPasses; ++pass) {
        if (st.all_done) break;                             // uniform: read after a barrier
        const int nslots = st.nslots;
        const int bits = digit_bits(pass), before = bits_before(pass);
        const int shift = 64 - before - bits;
        const uint64_t dmask = (1ull << bits) - 1;
        const int nbins = pass == 0 ? 1 << bits : nslots << bits;
        for (int i = tid; i < nbins; i += kXThreads) hist[i] = 0;
        if (tid < kXMaxSlots) { smn[tid] = ~0ull; smx[tid] = 0ull; }
        __syncthreads();
        if (pass == 0) {
            // delta's keys only, with their range in slot 0
            uint64_t a = ~0ull, b = 0;
            for (int j = 0; j < kXPerThreadFused; ++j) {
                const uint64_t k0 = keys[tid + kXThreads * j];
                if (k0 != 0) visit_root(k0, hist, a, b);
            }
            for (int o = 1; o < 64; o <<= 1) {
                const uint64_t a2 = __shfl_xor(a, o), b2 = __shfl_xor(b, o);
                a = a2 < a ? a2 : a;
                b = b2 > b ? b2 : b;
            }
            if ((tid & 63) == 0) {
                atomicMin(&smn[0], (unsigned long long)a);
                atomicMax(&smx[0], (unsigned long long)b);
            }
        }
        // passes 1-5 slot by slot, so that one slot's key range is live at a time
        for (int s = 0; s < (pass == 0 ? 0 : nslots); ++s) {
            const uint64_t pre = st.slot[s].prefix;
            const int kind = st.slot[s].kind;
            uint64_t a = ~0ull, b = 0;
            for (int j = 0; j < kXPerThreadFused; ++j) {
                const uint64_t k0 = keys[tid + kXThreads * j];
                const uint64_t k = kind ? key_abs_of(k0) : k0;
                if (k0 != 0 && (k >> (64 - before)) == pre) {
                    atomicAdd(&hist[(s << bits) | (uint32_t)((k >> shift) & dmask)], 1u);
                    a = k < a ? k : a;
                    b = k > b ? k : b;
                }
            }
            for (int o = 1; o < 64; o <<= 1) {
                const uint64_t a2 = __shfl_xor(a, o), b2 = __shfl_xor(b, o);
                a = a2 < a ? a2 : a;
                b = b2 > b ? b2 : b;
            }
            if ((tid & 63) == 0) {
                atomicMin(&smn[s], (unsigned long long)a);
                atomicMax(&smx[s], (unsigned long long)b);
            }
        }
        __syncthreads();
        select_step(st, pass, hist, smn, smx, sh, fdig, frank);
    }
    if (tid == 0) write_outputs(out, prm, st, rel, next_all, nv);
}

// ---------------------------------------------------------------------------
// Above kXFusedMax tokens: pass / reduce / select launches.
// ---------------------------------------------------------------------------

// cflag[0]: pass 0's regions overflowed; cflag[1]: pass 0's regions are
// not usable (overflow, or a target outside the predicted windows);
// cflag[2]: pass 1's regions overflowed (pass 1 copies only when cflag[1]);
// cflag[3]: valid tokens in the sample.
constexpr int kXSampleGroup = 16;        // consecutive tokens per sample group
constexpr int kXSampleEvery = 1024;      // one group per this many tokens
constexpr int kXSampleBlocks = 128;
// Below this many tokens the second read of the inputs costs less than the
// sample's two launches: no sample, no window, pass 1 reads the tokens.
constexpr uint32_t kXSampleMinN = 1u << 25;

__global__ void __launch_bounds__(256)
xsel_init_kernel(XParamsDev prm, XState* __restrict__ st, uint32_t* __restrict__ cflag,
                 uint32_t* __restrict__ shist, uint32_t* __restrict__ pmark) {
    for (int i = threadIdx.x; i < (1 << 14); i += 256) shist[i] = 0;
    for (int i = threadIdx.x; i < (1 << 14) / 32; i += 256) pmark[i] = 0;
    if (threadIdx.x < 4) cflag[threadIdx.x] = 0;
    if (threadIdx.x != 0) return;
    init_state(st, prm);
}

// First digits of the sample's delta keys into shist (integer atomics: the
// counts do not depend on their order), and the sample's valid count.
template <bool kMask>
__global__ void __launch_bounds__(kXThreads)
xsel_sample_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                   const uint8_t* __restrict__ mask, uint32_t n, uint32_t* __restrict__ shist,
                   uint32_t* __restrict__ cflag) {
    __shared__ uint32_t hist[1 << 14];
    __shared__ uint32_t cnt;
    for (int i = threadIdx.x; i < (1 << 14); i += kXThreads) hist[i] = 0;
    if (threadIdx.x == 0) cnt = 0;
    __syncthreads();
    const uint32_t groups = (n + kXSampleEvery - 1) / kXSampleEvery;
    const uint32_t total = groups * kXSampleGroup;
    uint32_t nv = 0;
    for (uint32_t i = blockIdx.x * kXThreads + threadIdx.x; i < total;
         i += gridDim.x * kXThreads) {
        const uint32_t t = (i / kXSampleGroup) * kXSampleEvery + (i % kXSampleGroup);
        if (t >= n) continue;
        const double d = (double)lt[t] - (double)lr[t];
        if ((kMask ? mask[t] != 0 : true) && isfinite(d)) {
            atomicAdd(&hist[(uint32_t)(key_delta(d) >> 50)], 1u);
            ++nv;
        }
    }
    atomicAdd(&cnt, nv);
    __syncthreads();
    for (int i = threadIdx.x; i < (1 << 14); i += kXThreads)
        if (hist[i]) atomicAdd(&shist[i], hist[i]);
    if (threadIdx.x == 0) atomicAdd(&cflag[3], cnt);
}

// The predicted windows as a bitmap over delta's first digits (pmark): for
// each probability, the bins (in the kind's key order) that hold the sample
// ranks within the margin of q (m - 1); a |delta| bin marks the two delta
// bins it counts.  One block.
__global__ void __launch_bounds__(kXThreads)
xsel_predict_kernel(XParamsDev prm, const uint32_t* __restrict__ shist,
                    const uint32_t* __restrict__ cflag, uint32_t* __restrict__ pmark) {
    constexpr int kPer = (1 << 14) / kXThreads;      // 16 bins per thread
    __shared__ uint32_t h[1 << 14];
    __shared__ uint32_t mk[(1 << 14) / 32];
    __shared__ uint64_t sh[kXThreads / 64];
    __shared__ uint32_t c0[1 << 14];                 // cumulative counts before each bin
    const int tid = threadIdx.x;
    for (int i = tid; i < (1 << 14); i += kXThreads) h[i] = shist[i];
    for (int i = tid; i < (1 << 14) / 32; i += kXThreads) mk[i] = 0;
    __syncthreads();
    const double m = (double)cflag[3];
    for (int kind = 0; kind < 2; ++kind) {
        const int nq = kind == 0 ? prm.nrq : prm.naq;
        if (nq == 0 || m == 0.0) continue;
        const int nb = kind == 0 ? 1 << 14 : 1 << 13;
        // bin b of this kind, in key order: delta's own, or |delta|'s root
        // bin counting two delta bins
        uint64_t local = 0;
        uint32_t v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int b = tid * kPer + j;
            v[j] = b < nb ? (kind == 0 ? h[b] : abs_root_bin(h, b)) : 0u;
            local += v[j];
        }
        uint64_t run = block_excl_scan<kXThreads>(local, sh);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            c0[tid * kPer + j] = (uint32_t)run;
            run += v[j];
        }
        __syncthreads();
        for (int i = 0; i < nq; ++i) {
            const double q = kind == 0 ? prm.rq[i] : prm.aq[i];
            const double r = q * (m - 1.0);
            const double delta = 8.0 * sqrt(m * q * (1.0 - q)) + 64.0;
            const double lo = r - delta, hi = r + delta;
            // bin b holds sample ranks [c0[b], c0[b] + count); mark it if
            // that range meets [lo, hi]
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int b = tid * kPer + j;
                if (b >= nb) continue;
                const double a = (double)c0[b], e = a + (double)v[j];
                // empty bins between the window's first and last are marked
                // too: c0 does not move across them
                if (e >= lo && a <= hi) {
                    if (kind == 0) {
                        atomicOr(&mk[b >> 5], 1u << (b & 31));
                    } else {
                        const int d0 = 0x2000 | b, d1 = 0x1FFF ^ b;
                        atomicOr(&mk[d0 >> 5], 1u << (d0 & 31));
                        atomicOr(&mk[d1 >> 5], 1u << (d1 & 31));
                    }
                }
            }
        }
        __syncthreads();
    }
    for (int i = tid; i < (1 << 14) / 32; i += kXThreads) pmark[i] = mk[i];
}

// One histogram pass; kMode 0: pass 0, 1: pass 1, 2: passes 2-5.  Reading
// the tokens, block b takes tokens b*1024 + tid + j*stride, stride = grid *
// 1024.  Pass 0 copies the keys whose first digit is marked in pmark into
// the block's region cand[b*cap ...]; passes 1-5 read the region when
// pass 0's copy is usable (cflag[1] == 0).  Otherwise pass 1 reads the
// tokens and copies the keys that any slot takes, and passes 2-5 read that
// copy unless it overflowed too.
template <bool kMask, int kMode>
__global__ void __launch_bounds__(kXThreads)
xsel_pass_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                 const uint8_t* __restrict__ mask, uint32_t n, int pass, XParamsDev prm,
                 const XState* __restrict__ st, uint32_t* __restrict__ bhist,
                 ulonglong2* __restrict__ bmm, XPart* __restrict__ part,
                 uint64_t* __restrict__ cand, uint32_t* __restrict__ ccnt, uint32_t cap,
                 uint32_t* __restrict__ cflag, const uint32_t* __restrict__ pmark) {
    __shared__ uint32_t hist[kXLdsBins];
    __shared__ unsigned long long smn[kXMaxSlots], smx[kXMaxSlots];
    __shared__ double rsh[kXThreads];
    __shared__ uint32_t lcount;
    __shared__ uint32_t mark[(1 << 14) / 32];   // root digits whose keys are copied
    constexpr bool first = kMode == 0;
    if (!first && st->all_done) return;
    // pass 1 reads pass 0's copy when it is usable; passes 2-5 read the
    // regions unless the last copy made overflowed
    const bool from_cand = kMode == 1 ? cflag[1] == 0
                         : kMode == 2 ? (cflag[1] == 0 || cflag[2] == 0) : false;
    Slots sl;
    load_slots(sl, st);
    const int bits = digit_bits(pass), before = bits_before(pass);
    const int tid = threadIdx.x;
    const int nbins = first ? 1 << bits : sl.n << bits;    // pass 0: delta's histogram only
    const int nranges = first ? 1 : sl.n;
    for (int i = tid; i < nbins; i += kXThreads) hist[i] = 0;
    if (tid < kXMaxSlots) { smn[tid] = ~0ull; smx[tid] = 0ull; }
    if (tid == 0) lcount = 0;
    const bool collect = kMode == 0 || (kMode == 1 && !from_cand);
    if (kMode == 0) {
        for (int i = tid; i < (1 << 14) / 32; i += kXThreads) mark[i] = pmark[i];
    } else if (collect) {
        for (int i = tid; i < (1 << 14) / 32; i += kXThreads) mark[i] = 0;
        __syncthreads();
        if (tid < sl.n) {
            // delta's root digit of the slot, or the two that |delta|'s covers
            const uint32_t d = (uint32_t)st->slot[tid].prefix;
            if (st->slot[tid].kind == 0) {
                atomicOr(&mark[d >> 5], 1u << (d & 31));
            } else {
                atomicOr(&mark[(0x2000 | d) >> 5], 1u << ((0x2000 | d) & 31));
                atomicOr(&mark[(0x1FFF ^ d) >> 5], 1u << ((0x1FFF ^ d) & 31));
            }
        }
    }
    __syncthreads();

    uint64_t lmn[kXMaxSlots], lmx[kXMaxSlots];
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) { lmn[s] = ~0ull; lmx[s] = 0; }
    double rel = 0.0;
    double dmin = INFINITY, dmax = -INFINITY;     // pass 0: the range of delta
    uint32_t next = 0, nval = 0;
    if (from_cand) {
        const uint32_t cnt = ccnt[blockIdx.x];
        const uint64_t* reg = cand + (size_t)blockIdx.x * cap;
        // kXUnroll keys per thread per trip, loaded before any is visited
        // (counts and ranges do not depend on the order of the visits)
        uint32_t i = tid;
        for (; i + (kXUnroll - 1) * kXThreads < cnt; i += kXUnroll * kXThreads) {
            uint64_t k[kXUnroll];
#pragma unroll
            for (int j = 0; j < kXUnroll; ++j) k[j] = reg[i + j * kXThreads];
#pragma unroll
            for (int j = 0; j < kXUnroll; ++j) visit<false>(k[j], sl, before, bits, hist, lmn, lmx);
        }
        for (; i < cnt; i += kXThreads) visit<false>(reg[i], sl, before, bits, hist, lmn, lmx);
    } else {
        const uint32_t stride = gridDim.x * kXThreads;
        uint64_t* reg = cand + (size_t)blockIdx.x * cap;
        for (uint32_t base = blockIdx.x * kXThreads + tid; base < n; base += kXUnroll * stride) {
            float x[kXUnroll], y[kXUnroll];
            uint32_t m[kXUnroll];
#pragma unroll
            for (int j = 0; j < kXUnroll; ++j) {
                const uint64_t t64 = (uint64_t)base + (uint64_t)j * stride;
                const uint32_t t = t64 < n ? (uint32_t)t64 : base;    // base < n: in bounds
                // every load is issued, in bounds, whatever the token's fate: a
                // short-circuit would put each mask load behind its own wait
                x[j] = lt[t];
                y[j] = lr[t];
                m[j] = (uint32_t)(t64 < n) & (kMask ? (uint32_t)(mask[t] != 0) : 1u);
            }
#pragma unroll
            for (int j = 0; j < kXUnroll; ++j) {
                const double d = (double)x[j] - (double)y[j];
                // not short-circuit: d, and so its loads, stay ahead of the
                // branch (else the compiler issues a load behind the mask's
                // wait and then waits for it)
                const bool valid = (m[j] != 0) & isfinite(d);
                bool take = false;
                uint64_t k0 = 0;
                if (valid) {
                    if (first) {
                        rel += div_in_range(fabs(d), fabs((double)x[j]) + 1e-8);
                        next += fabs(d) > prm.tok_tau ? 1u : 0u;
                        ++nval;
                    }
                    k0 = key_delta(d);
                    if (first) {
                        // the range as values (two instructions rather than
                        // six on 64-bit keys), made keys once at the end
                        atomicAdd(&hist[(uint32_t)(k0 >> 50)], 1u);
                        dmin = min_fin(dmin, d);
                        dmax = max_fin(dmax, d);
                        const uint32_t r = (uint32_t)(k0 >> 50);
                        take = (mark[r >> 5] >> (r & 31)) & 1u;
                    } else if (collect) {
                        const uint32_t r = (uint32_t)(k0 >> 50);
                        if ((mark[r >> 5] >> (r & 31)) & 1u)
                            take = visit<true>(k0, sl, before, bits, hist, lmn, lmx);
                    } else {
                        take = visit<false>(k0, sl, before, bits, hist, lmn, lmx);
                    }
                }
                if (collect) {
                    // append to this block's region: the compiler's atomic
                    // optimizer turns the takers' increments into one LDS
                    // atomic per wave and gives each taker the old count
                    // plus the number of takers in lower lanes
                    if (take) {
                        const uint32_t pos = atomicAdd(&lcount, 1u);
                        if (pos < cap) reg[pos] = k0;
                        else cflag[first ? 0 : 2] = 1;    // every writer stores the same value
                    }
                }
            }
        }
    }
    if (first && nval > 0) {
        // the key order is the value order, except that -0 and +0 (equal as
        // values) have two keys: a range whose ends are zeros of either sign
        // may then end on the same key though both occur, which resolves the
        // targets to a zero of one sign, and every output is the same for
        // either (ratio 1, |delta| 0)
        lmn[0] = key_delta(dmin);
        lmx[0] = key_delta(dmax);
    }
    flush_range(nranges, lmn, lmx, smn, smx);
    if (first) {
        const double r = block_sum<kXThreads>(rel, rsh);
        const double ne = block_sum<kXThreads>((double)next, rsh);   // exact: < 2^53
        const double nv = block_sum<kXThreads>((double)nval, rsh);
        if (tid == 0) part[blockIdx.x] = XPart{r, (uint64_t)ne, (uint64_t)nv, 0};
    }
    __syncthreads();
    uint32_t* outh = bhist + (size_t)blockIdx.x * kXLdsBins;
    for (int i = tid; i < nbins; i += kXThreads) outh[i] = hist[i];
    if (tid < nranges) bmm[(size_t)blockIdx.x * kXMaxSlots + tid] = make_ulonglong2(smn[tid], smx[tid]);
    if (collect && tid == 0) ccnt[blockIdx.x] = lcount;
}

// ghist[i] = sum over blocks of bhist[b][i], for the active bins.  A block
// takes kXReduceBins bins; its kXReduceGroups thread groups sum interleaved
// subsets of the pass blocks, then add their partial sums in LDS.
__global__ void __launch_bounds__(kXReduceThreads)
xsel_reduce_kernel(const uint32_t* __restrict__ bhist, int nblk, int pass,
                   const XState* __restrict__ st, uint32_t* __restrict__ ghist) {
    __shared__ uint32_t part[kXReduceGroups][kXReduceBins];
    if (pass > 0 && st->all_done) return;
    const int nbins = pass == 0 ? 1 << digit_bits(0) : st->nslots << digit_bits(pass);
    const int i0 = blockIdx.x * kXReduceBins;
    if (i0 >= nbins) return;                                  // uniform
    const int lane = threadIdx.x % kXReduceBins, g = threadIdx.x / kXReduceBins;
    const int i = i0 + lane;
    uint32_t acc = 0;
    if (i < nbins) {
        int b = g;
        for (; b + 3 * kXReduceGroups < nblk; b += 4 * kXReduceGroups) {
            const uint32_t a0 = bhist[(size_t)b * kXLdsBins + i];
            const uint32_t a1 = bhist[(size_t)(b + kXReduceGroups) * kXLdsBins + i];
            const uint32_t a2 = bhist[(size_t)(b + 2 * kXReduceGroups) * kXLdsBins + i];
            const uint32_t a3 = bhist[(size_t)(b + 3 * kXReduceGroups) * kXLdsBins + i];
            acc += (a0 + a1) + (a2 + a3);
        }
        for (; b < nblk; b += kXReduceGroups) acc += bhist[(size_t)b * kXLdsBins + i];
    }
    part[g][lane] = acc;
    __syncthreads();
    if (g == 0 && i < nbins) {
        uint32_t sum = 0;
        for (int k = 0; k < kXReduceGroups; ++k) sum += part[k][lane];
        ghist[i] = sum;
    }
}

__global__ void __launch_bounds__(kXThreads)
xsel_select_kernel(int pass, int nblk, XParamsDev prm, XState* __restrict__ gst,
                   const uint32_t* __restrict__ ghist, const ulonglong2* __restrict__ bmm,
                   const XPart* __restrict__ part, uint32_t* __restrict__ cflag,
                   const uint32_t* __restrict__ pmark) {
    __shared__ XState st;                    // working copy; thread 0 writes it back
    __shared__ uint64_t sh[kXThreads];
    __shared__ unsigned long long mn[kXMaxSlots], mx[kXMaxSlots];
    __shared__ uint64_t fdig[kXMaxTargets], frank[kXMaxTargets];
    const int tid = threadIdx.x;
    if (tid == 0) st = *gst;
    __syncthreads();
    if (pass > 0 && st.all_done) return;
    if (pass == 0) {
        uint64_t nv = 0;
        for (int b = tid; b < nblk; b += kXThreads) nv += part[b].nvalid;
        nv = block_sum<kXThreads>(nv, sh);
        if (tid == 0) set_ranks(st, nv, prm);
        __syncthreads();
        if (st.all_done) {
            if (tid == 0) *gst = st;
            return;
        }
    }
    const int nranges = pass == 0 ? 1 : st.nslots;
    if (tid < kXMaxSlots) { mn[tid] = ~0ull; mx[tid] = 0ull; }
    __syncthreads();
    // thread b takes pass block b (there are at most kXThreads of them);
    // wave butterflies, then one LDS atomic per wave and slot
    static_assert(kXMaxBlocks <= kXThreads, "one pass block per select thread");
    for (int s = 0; s < nranges; ++s) {
        uint64_t a = ~0ull, b = 0;
        if (tid < nblk) {
            const ulonglong2 v = bmm[(size_t)tid * kXMaxSlots + s];
            a = v.x;
            b = v.y;
        }
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t a2 = __shfl_xor(a, o), b2 = __shfl_xor(b, o);
            a = a2 < a ? a2 : a;
            b = b2 > b ? b2 : b;
        }
        if ((tid & 63) == 0) {
            atomicMin(&mn[s], (unsigned long long)a);
            atomicMax(&mx[s], (unsigned long long)b);
        }
    }
    __syncthreads();
    select_step(st, pass, ghist, mn, mx, sh, fdig, frank);
    if (tid == 0) {
        if (pass == 0) {
            // pass 0's copy serves the later passes iff it did not overflow
            // and every unresolved target's first digit was copied
            bool usable = cflag[0] == 0;
            for (int t = 0; t < st.ntgt; ++t) {
                if (st.tgt[t].resolved) continue;
                const uint32_t d = (uint32_t)st.tgt[t].prefix;
                auto marked = [&](uint32_t b) { return (pmark[b >> 5] >> (b & 31)) & 1u; };
                usable = usable && (st.tgt[t].kind == 0 ? marked(d) != 0
                                                        : (marked(0x2000 | d) && marked(0x1FFF ^ d)));
            }
            cflag[1] = usable ? 0u : 1u;
        }
        *gst = st;
    }
}

__global__ void __launch_bounds__(kXFinThreads)
xsel_final_kernel(int nblk, XParamsDev prm, const XState* __restrict__ st,
                  const XPart* __restrict__ part, double* __restrict__ out) {
    __shared__ double sh[kXFinThreads];
    __shared__ uint64_t shu[kXFinThreads];
    double rel = 0.0;
    uint64_t next = 0, nv = 0;
    for (int b = threadIdx.x; b < nblk; b += kXFinThreads) {
        rel += part[b].rel;
        next += part[b].next;
        nv += part[b].nvalid;
    }
    rel = block_sum<kXFinThreads>(rel, sh);
    next = block_sum<kXFinThreads>(next, shu);
    nv = block_sum<kXFinThreads>(nv, shu);
    if (threadIdx.x == 0) write_outputs(out, prm, *st, rel, next, nv);
}

}  // namespace

bool make_extras_plan(int64_t n, ExtrasPlan* p) {
    if (n < 0 || n > INT32_MAX) return false;
    p->n = n;
    p->fused = n <= kXFusedMax;
    int64_t g = (n + 16383) / 16384;
    if (g < 1) g = 1;
    if (g > kXMaxBlocks) g = kXMaxBlocks;
    p->nblk = p->fused ? 0 : g;
    // a block's region holds a quarter of its tokens, plus a margin
    const int64_t per_blk = p->fused ? 0 : (n + g - 1) / g;
    p->cap = p->fused ? 0 : (uint32_t)(per_blk / 4 + 4096);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    if (p->fused) {
        p->state_off = p->bhist_off = p->bmm_off = p->ghist_off = p->part_off = 0;
        p->cand_off = p->ccnt_off = p->cflag_off = p->shist_off = p->pmark_off = 0;
        p->total_bytes = 256;                      // unused: the fused kernel keeps all in LDS
        return true;
    }
    p->state_off = take(sizeof(XState));
    p->bhist_off = take((size_t)g * kXLdsBins * sizeof(uint32_t));
    p->bmm_off = take((size_t)g * kXMaxSlots * sizeof(ulonglong2));
    p->ghist_off = take((size_t)kXLdsBins * sizeof(uint32_t));
    p->part_off = take((size_t)g * sizeof(XPart));
    p->cand_off = take((size_t)g * p->cap * sizeof(uint64_t));
    p->ccnt_off = take((size_t)g * sizeof(uint32_t));
    p->cflag_off = take(4 * sizeof(uint32_t));
    p->shist_off = take((size_t)(1 << 14) * sizeof(uint32_t));
    p->pmark_off = take((size_t)(1 << 14) / 32 * sizeof(uint32_t));
    p->total_bytes = off;
    return true;
}

hipError_t launch_mismatch_extras(const ExtrasPlan& p, const float* lt, const float* lr,
                                  const uint8_t* mask, const XParamsDev& prm, double* out,
                                  void* workspace, hipStream_t st) {
    if (p.fused) {
        if (!out) return hipSuccess;           // nothing to write
        if (mask)
            hipLaunchKernelGGL((xsel_fused_kernel<true>), dim3(1), dim3(kXThreads), 0, st, lt, lr,
                               mask, (uint32_t)p.n, prm, out);
        else
            hipLaunchKernelGGL((xsel_fused_kernel<false>), dim3(1), dim3(kXThreads), 0, st, lt, lr,
                               mask, (uint32_t)p.n, prm, out);
        return hipGetLastError();
    }
    unsigned char* ws = (unsigned char*)workspace;
    XState* state = (XState*)(ws + p.state_off);
    uint32_t* bhist = (uint32_t*)(ws + p.bhist_off);
    ulonglong2* bmm = (ulonglong2*)(ws + p.bmm_off);
    uint32_t* ghist = (uint32_t*)(ws + p.ghist_off);
    XPart* part = (XPart*)(ws + p.part_off);
    uint64_t* cand = (uint64_t*)(ws + p.cand_off);
    uint32_t* ccnt = (uint32_t*)(ws + p.ccnt_off);
    uint32_t* cflag = (uint32_t*)(ws + p.cflag_off);
    uint32_t* shist = (uint32_t*)(ws + p.shist_off);
    uint32_t* pmark = (uint32_t*)(ws + p.pmark_off);
    const int nblk = (int)p.nblk;
    const uint32_t n = (uint32_t)p.n;
    hipLaunchKernelGGL(xsel_init_kernel, dim3(1), dim3(256), 0, st, prm, state, cflag, shist,
                       pmark);
    if (n >= kXSampleMinN) {
        if (mask)
            hipLaunchKernelGGL((xsel_sample_kernel<true>), dim3(kXSampleBlocks), dim3(kXThreads), 0,
                               st, lt, lr, mask, n, shist, cflag);
        else
            hipLaunchKernelGGL((xsel_sample_kernel<false>), dim3(kXSampleBlocks), dim3(kXThreads),
                               0, st, lt, lr, mask, n, shist, cflag);
        hipLaunchKernelGGL(xsel_predict_kernel, dim3(1), dim3(kXThreads), 0, st, prm,
                           (const uint32_t*)shist, (const uint32_t*)cflag, pmark);
    }
    static_assert(bits_before(1) + digit_bits(1) <= 32, "pass 1 tests upper halves");
    for (int pass = 0; pass < kXPasses; ++pass) {
        auto kern = pass == 0 ? (mask ? xsel_pass_kernel<true, 0> : xsel_pass_kernel<false, 0>)
                  : pass == 1 ? (mask ? xsel_pass_kernel<true, 1> : xsel_pass_kernel<false, 1>)
                              : (mask ? xsel_pass_kernel<true, 2> : xsel_pass_kernel<false, 2>);
        hipLaunchKernelGGL(kern, dim3(nblk), dim3(kXThreads), 0, st, lt, lr, mask, n, pass, prm,
                           (const XState*)state, bhist, bmm, part, cand, ccnt, p.cap, cflag,
                           (const uint32_t*)pmark);
        const int nbins_max = pass == 0 ? 1 << digit_bits(0) : kXMaxSlots << digit_bits(pass);
        hipLaunchKernelGGL(xsel_reduce_kernel,
                           dim3((nbins_max + kXReduceBins - 1) / kXReduceBins),
                           dim3(kXReduceThreads), 0, st, (const uint32_t*)bhist, nblk, pass,
                           (const XState*)state, ghist);
        hipLaunchKernelGGL(xsel_select_kernel, dim3(1), dim3(kXThreads), 0, st, pass, nblk, prm,
                           state, (const uint32_t*)ghist, (const ulonglong2*)bmm,
                           (const XPart*)part, cflag, (const uint32_t*)pmark);
    }
    if (out)
        hipLaunchKernelGGL(xsel_final_kernel, dim3(1), dim3(kXFinThreads), 0, st, nblk, prm,
                           (const XState*)state, (const XPart*)part, out);
    return hipGetLastError();
}

}  // namespace tim
