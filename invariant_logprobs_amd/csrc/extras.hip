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
// |delta|'s key is its bit pattern shifted left by one (the sign bit is 0).
// Each pass histograms one digit of the keys that share a target's prefix:
//
//   pass 0: top 13 bits; passes 1-4: 11 bits each; pass 5: the last 7.
//
//   1. xsel_init: targets (a lower and an upper order statistic per
//      probability) and the root slots, one per key kind.
//   2. per pass:
//      xsel_pass    every block histograms its share of the tokens in LDS,
//                   one histogram per slot (a distinct (kind, prefix)), and
//                   writes it with plain stores, with the minimum and
//                   maximum key it saw per slot.  Pass 0 also folds the
//                   extreme count and the relative difference of its
//                   tokens, in a fixed order, into a block partial.
//      xsel_reduce  sums the block histograms bin by bin (integers: the
//                   order does not matter).
//      xsel_select  one block: pass 0 turns probabilities into ranks; every
//                   pass moves each unresolved target into the bin that
//                   holds its rank.  A slot whose minimum equals its maximum
//                   resolves its targets at once (ties, zero mismatch).
//                   When every target is resolved the later passes return
//                   at their first instruction.
//   3. xsel_final: folds the block partials in a fixed tree and writes the
//      outputs.
//
// Every step is exact integer work except the per-token relative
// difference (one fp64 division, as the definition states) and its sum,
// whose order depends only on n.  The results are therefore deterministic,
// and the selected order statistics are bit-exact.

#include "tim_internal.h"

#include <math.h>

namespace tim {
namespace {

constexpr int kXThreads = 1024;          // threads per pass block
constexpr int kXUnroll = 8;              // tokens per thread per loop trip
constexpr int kXMaxTargets = 2 * kXMaxQ;
constexpr int kXMaxSlots = kXMaxTargets;
constexpr int kXLdsBins = 16384;         // 2 slots x 2^13 or 8 slots x 2^11
constexpr int kXReduceThreads = 256;
constexpr int kXFinThreads = 256;

__host__ __device__ constexpr int digit_bits(int pass) {
    return pass == 0 ? 13 : (pass < kXPasses - 1 ? 11 : 7);
}
__host__ __device__ constexpr int bits_before(int pass) {
    return pass == 0 ? 0 : 13 + 11 * (pass - 1);
}
static_assert(bits_before(kXPasses - 1) + digit_bits(kXPasses - 1) == 64, "64 key bits");
static_assert(2 * (1 << digit_bits(0)) <= kXLdsBins, "pass 0: one slot per key kind");
static_assert(kXMaxSlots * (1 << digit_bits(1)) <= kXLdsBins, "later passes: one slot per target");

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
__device__ __forceinline__ uint64_t key_abs(double d) {
    return (__builtin_bit_cast(uint64_t, d) & 0x7FFFFFFFFFFFFFFFull) << 1;
}
__device__ __forceinline__ double value_of(uint64_t k, int kind) {
    uint64_t u;
    if (kind == 0) u = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
    else u = k >> 1;
    return __builtin_bit_cast(double, u);
}

// Position q (m - 1) of probability q among m >= 1 sorted values: lower and
// upper index and the interpolation weight.
// Each operation is rounded on its own: no fused multiply-add may join the
// product and the subtraction.
__device__ __attribute__((noinline)) void quantile_pos(double q, uint64_t m, uint64_t* lo,
                                                        uint64_t* hi, double* frac) {
#pragma clang fp contract(off)
    const double pos = q * (double)(m - 1);
    const double fl = floor(pos);
    *lo = (uint64_t)fl;
    *hi = *lo + 1 < m ? *lo + 1 : *lo;
    *frac = pos - fl;
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

// Exclusive prefix sum over a block of kT threads.
template <int kT>
__device__ uint64_t block_excl_scan(uint64_t x, uint64_t* sh) {
    sh[threadIdx.x] = x;
    __syncthreads();
    for (int off = 1; off < kT; off <<= 1) {
        const uint64_t y = (int)threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
        __syncthreads();
        sh[threadIdx.x] += y;
        __syncthreads();
    }
    const uint64_t r = sh[threadIdx.x] - x;
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(64)
xsel_init_kernel(XParamsDev prm, XState* __restrict__ st) {
    if (threadIdx.x != 0) return;
    const int ntgt = 2 * (prm.nrq + prm.naq);
    // one root slot per key kind present: delta first, then |delta|
    const int root_abs = prm.nrq > 0 ? 1 : 0;
    st->ntgt = ntgt;
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

// One histogram pass.  Block b takes tokens b*1024 + tid + j*stride, j >= 0,
// stride = grid * 1024, kXUnroll of them per loop trip.
template <bool kMask>
__global__ void __launch_bounds__(kXThreads)
xsel_pass_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                 const uint8_t* __restrict__ mask, uint32_t n, int pass, XParamsDev prm,
                 const XState* __restrict__ st, uint32_t* __restrict__ bhist,
                 ulonglong2* __restrict__ bmm, XPart* __restrict__ part) {
    __shared__ uint32_t hist[kXLdsBins];
    __shared__ unsigned long long smn[kXMaxSlots], smx[kXMaxSlots];
    __shared__ double rsh[kXThreads];
    const bool first = pass == 0;
    if (!first && st->all_done) return;
    const int nslots = st->nslots;
    const int bits = digit_bits(pass), before = bits_before(pass);
    const int shift = 64 - before - bits;
    const uint64_t dmask = (1ull << bits) - 1;
    const int tid = threadIdx.x;
    const int nbins = nslots << bits;
    for (int i = tid; i < nbins; i += kXThreads) hist[i] = 0;
    if (tid < kXMaxSlots) { smn[tid] = ~0ull; smx[tid] = 0ull; }
    uint64_t spre[kXMaxSlots];
    int skind[kXMaxSlots];
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) {
        spre[s] = s < nslots ? st->slot[s].prefix : 0;
        skind[s] = s < nslots ? st->slot[s].kind : 0;
    }
    __syncthreads();

    uint64_t lmn[kXMaxSlots], lmx[kXMaxSlots];
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) { lmn[s] = ~0ull; lmx[s] = 0; }
    double rel = 0.0;
    uint32_t next = 0, nval = 0;
    const uint32_t stride = gridDim.x * kXThreads;
    for (uint32_t base = blockIdx.x * kXThreads + tid; base < n; base += kXUnroll * stride) {
        float x[kXUnroll], y[kXUnroll];
        uint32_t m[kXUnroll];
#pragma unroll
        for (int j = 0; j < kXUnroll; ++j) {
            const uint64_t t64 = (uint64_t)base + (uint64_t)j * stride;
            const uint32_t t = t64 < n ? (uint32_t)t64 : base;    // base < n: in bounds
            x[j] = lt[t];
            y[j] = lr[t];
            m[j] = (t64 < n) && (kMask ? mask[t] != 0 : true);
        }
#pragma unroll
        for (int j = 0; j < kXUnroll; ++j) {
            const double d = (double)x[j] - (double)y[j];
            const bool valid = m[j] && isfinite(d);
            if (!valid) continue;
            if (first) {
                rel += fabs(d) / (fabs((double)x[j]) + 1e-8);
                next += fabs(d) > prm.tok_tau ? 1u : 0u;
                ++nval;
            }
            const uint64_t k0 = key_delta(d), k1 = key_abs(d);
#pragma unroll
            for (int s = 0; s < kXMaxSlots; ++s) {
                if (s >= nslots) break;
                const uint64_t k = skind[s] ? k1 : k0;
                const bool match = before == 0 || (k >> (64 - before)) == spre[s];
                if (match) {
                    atomicAdd(&hist[(s << bits) | (uint32_t)((k >> shift) & dmask)], 1u);
                    lmn[s] = k < lmn[s] ? k : lmn[s];
                    lmx[s] = k > lmx[s] ? k : lmx[s];
                }
            }
        }
    }
    // per-slot minimum and maximum: wave butterflies, then one LDS atomic per wave
#pragma unroll
    for (int s = 0; s < kXMaxSlots; ++s) {
        if (s >= nslots) break;
        uint64_t a = lmn[s], b = lmx[s];
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
    if (first) {
        const double r = block_sum<kXThreads>(rel, rsh);
        const double ne = block_sum<kXThreads>((double)next, rsh);   // exact: < 2^53
        const double nv = block_sum<kXThreads>((double)nval, rsh);
        if (tid == 0) part[blockIdx.x] = XPart{r, (uint64_t)ne, (uint64_t)nv, 0};
    }
    __syncthreads();
    uint32_t* out = bhist + (size_t)blockIdx.x * kXLdsBins;
    for (int i = tid; i < nbins; i += kXThreads) out[i] = hist[i];
    if (tid < nslots) bmm[(size_t)blockIdx.x * kXMaxSlots + tid] = make_ulonglong2(smn[tid], smx[tid]);
}

// ghist[i] = sum over blocks of bhist[b][i], for the active bins.
__global__ void __launch_bounds__(kXReduceThreads)
xsel_reduce_kernel(const uint32_t* __restrict__ bhist, int nblk, int pass,
                   const XState* __restrict__ st, uint32_t* __restrict__ ghist) {
    if (pass > 0 && st->all_done) return;
    const int nbins = st->nslots << digit_bits(pass);
    const int i = blockIdx.x * kXReduceThreads + threadIdx.x;
    if (i >= nbins) return;
    uint32_t s = 0;
    for (int b = 0; b < nblk; ++b) s += bhist[(size_t)b * kXLdsBins + i];
    ghist[i] = s;
}

__global__ void __launch_bounds__(kXThreads)
xsel_select_kernel(int pass, int nblk, XParamsDev prm, XState* __restrict__ gst,
                   const uint32_t* __restrict__ ghist, const ulonglong2* __restrict__ bmm,
                   const XPart* __restrict__ part) {
    __shared__ XState st;                    // working copy; thread 0 writes it back
    __shared__ uint64_t sh[kXThreads];
    __shared__ unsigned long long mn[kXMaxSlots], mx[kXMaxSlots];
    __shared__ uint64_t found_digit, found_rank;
    const int tid = threadIdx.x;
    if (tid == 0) st = *gst;
    __syncthreads();
    if (pass > 0 && st.all_done) return;
    const int ntgt = st.ntgt;
    if (pass == 0) {
        // number of valid tokens, then each probability's two ranks
        uint64_t nv = 0;
        for (int b = tid; b < nblk; b += kXThreads) nv += part[b].nvalid;
        nv = block_sum<kXThreads>(nv, sh);
        if (tid == 0) {
            st.nvalid = nv;
            for (int t = 0; t < ntgt; t += 2) {
                const int i = t / 2;
                const double q = i < prm.nrq ? prm.rq[i] : prm.aq[i - prm.nrq];
                uint64_t lo = 0, hi = 0;
                double frac = 0.0;
                if (nv > 0) quantile_pos(q, nv, &lo, &hi, &frac);
                st.tgt[t].rank = lo;
                st.tgt[t + 1].rank = hi;
                if (nv == 0) st.tgt[t].resolved = st.tgt[t + 1].resolved = 1;
            }
            if (nv == 0 || ntgt == 0) st.all_done = 1;
        }
        __syncthreads();
        if (st.all_done) {
            if (tid == 0) *gst = st;
            return;
        }
    }
    const int nslots = st.nslots;
    if (tid < kXMaxSlots) { mn[tid] = ~0ull; mx[tid] = 0ull; }
    __syncthreads();
    for (int b = tid; b < nblk; b += kXThreads) {
        for (int s = 0; s < nslots; ++s) {
            const ulonglong2 v = bmm[(size_t)b * kXMaxSlots + s];
            atomicMin(&mn[s], v.x);
            atomicMax(&mx[s], v.y);
        }
    }
    __syncthreads();
    const int bits = digit_bits(pass), before = bits_before(pass);
    const int nb = 1 << bits;
    const int per = nb > kXThreads ? nb / kXThreads : 1;   // bins per thread
    for (int t = 0; t < ntgt; ++t) {
        // every thread reads target t before thread 0 may change it, so the
        // branches below are taken by the whole block (each wave then meets
        // the same barriers)
        const bool done_t = st.tgt[t].resolved;
        const int s = st.tgt[t].slot;
        const uint64_t rank = st.tgt[t].rank;
        __syncthreads();
        if (done_t) continue;
        if (mn[s] == mx[s]) {                               // one key value in the bucket
            if (tid == 0) { st.tgt[t].resolved = 1; st.tgt[t].key = mn[s]; }
            continue;
        }
        const uint32_t* h = ghist + ((size_t)s << bits);
        const int b0 = tid * per;
        uint64_t mine = 0;
        if (b0 < nb)
            for (int k = 0; k < per; ++k) mine += h[b0 + k];
        uint64_t c = block_excl_scan<kXThreads>(mine, sh);
        if (b0 < nb) {
            for (int k = 0; k < per; ++k) {
                const uint64_t hk = h[b0 + k];
                if (c <= rank && rank < c + hk) { found_digit = (uint64_t)(b0 + k); found_rank = rank - c; }
                c += hk;
            }
        }
        __syncthreads();
        if (tid == 0) {
            XTarget& g = st.tgt[t];
            g.prefix = before == 0 ? found_digit : ((g.prefix << bits) | found_digit);
            g.rank = found_rank;
            if (before + bits == 64) { g.resolved = 1; g.key = g.prefix; }
        }
        __syncthreads();
    }
    // slots of the next pass: one per distinct (kind, prefix) among the
    // unresolved targets, in target order
    if (tid == 0) {
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
    if (threadIdx.x != 0) return;
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
        uint64_t lo, hi;
        double frac;
        quantile_pos(q, nv, &lo, &hi, &frac);
        const int kind = ratio ? 0 : 1;
        double a = value_of(st->tgt[2 * i].key, kind);
        double b = value_of(st->tgt[2 * i + 1].key, kind);
        if (ratio) { a = exp(a); b = exp(b); }
        const double v = interpolate(a, b, frac);
        if (ratio) out[kXOutRatioQ + i] = v;
        else out[kXOutAbsQ + i - prm.nrq] = v;
    }
}

}  // namespace

bool make_extras_plan(int64_t n, ExtrasPlan* p) {
    if (n < 0 || n > INT32_MAX) return false;
    p->n = n;
    int64_t g = (n + 16383) / 16384;
    if (g < 1) g = 1;
    if (g > kXMaxBlocks) g = kXMaxBlocks;
    p->nblk = g;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    p->state_off = take(sizeof(XState));
    p->bhist_off = take((size_t)g * kXLdsBins * sizeof(uint32_t));
    p->bmm_off = take((size_t)g * kXMaxSlots * sizeof(ulonglong2));
    p->ghist_off = take((size_t)kXLdsBins * sizeof(uint32_t));
    p->part_off = take((size_t)g * sizeof(XPart));
    p->total_bytes = off;
    return true;
}

hipError_t launch_mismatch_extras(const ExtrasPlan& p, const float* lt, const float* lr,
                                  const uint8_t* mask, const XParamsDev& prm, double* out,
                                  void* workspace, hipStream_t st) {
    unsigned char* ws = (unsigned char*)workspace;
    XState* state = (XState*)(ws + p.state_off);
    uint32_t* bhist = (uint32_t*)(ws + p.bhist_off);
    ulonglong2* bmm = (ulonglong2*)(ws + p.bmm_off);
    uint32_t* ghist = (uint32_t*)(ws + p.ghist_off);
    XPart* part = (XPart*)(ws + p.part_off);
    const int nblk = (int)p.nblk;
    const uint32_t n = (uint32_t)p.n;
    hipLaunchKernelGGL(xsel_init_kernel, dim3(1), dim3(64), 0, st, prm, state);
    for (int pass = 0; pass < kXPasses; ++pass) {
        if (mask)
            hipLaunchKernelGGL((xsel_pass_kernel<true>), dim3(nblk), dim3(kXThreads), 0, st, lt,
                               lr, mask, n, pass, prm, (const XState*)state, bhist, bmm, part);
        else
            hipLaunchKernelGGL((xsel_pass_kernel<false>), dim3(nblk), dim3(kXThreads), 0, st, lt,
                               lr, mask, n, pass, prm, (const XState*)state, bhist, bmm, part);
        const int nbins_max = pass == 0 ? 2 << digit_bits(0) : kXMaxSlots << digit_bits(pass);
        hipLaunchKernelGGL(xsel_reduce_kernel,
                           dim3((nbins_max + kXReduceThreads - 1) / kXReduceThreads),
                           dim3(kXReduceThreads), 0, st, (const uint32_t*)bhist, nblk, pass,
                           (const XState*)state, ghist);
        hipLaunchKernelGGL(xsel_select_kernel, dim3(1), dim3(kXThreads), 0, st, pass, nblk, prm,
                           state, (const uint32_t*)ghist, (const ulonglong2*)bmm,
                           (const XPart*)part);
    }
    if (out)
        hipLaunchKernelGGL(xsel_final_kernel, dim3(1), dim3(kXFinThreads), 0, st, nblk, prm,
                           (const XState*)state, (const XPart*)part, out);
    return hipGetLastError();
}

}  // namespace tim
