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
// The pass is HBM-bound: 9 bytes per token are read once.  Every sequence is
// cut into sub-chunks of at most kSubChunk tokens that start at the
// sequence's first token and every kSubChunk tokens after it; a sub-chunk's
// sums are folded in an order that depends only on token offsets inside it,
// so a sequence's results never depend on the rest of the batch.
//
//   1. plan_count / plan_scan / plan_write: integer prefix sum of the
//      sub-chunk counts; writes one (start, length) descriptor per
//      sub-chunk, in token order, and each sequence's first descriptor.
//   2. stats_stream: each wave takes kSubPerWave consecutive descriptors and
//      streams their tokens through a kRing-slot LDS ring in kPiece-token
//      pieces.  Pieces are copied global -> LDS with global_load_lds_dword
//      (no registers held by loads in flight), kRing - 1 pieces ahead of the
//      fold, with exact vmcnt waits.  Sub-chunk partials are staged in LDS
//      and written once when the wave is done, so no store is ever counted
//      among the ring's loads.
//   3. seq_finalize: one thread per sequence folds its sub-chunks in
//      ascending order, writes means and flags; each block folds its
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
static_assert(sizeof(SubPartial) == 64, "four 16-byte quarters");

// Contribution of one sequence to the batch, and the running fold of many.
struct alignas(16) BatchAcc {
    double sd, sk2, sk3, sw, sabs, maxabs;           // token sums
    double md, mk1, mk2, mk3;                        // sums of sequence means
    int64_t nvalid, nclip, nnan, nonempty, rejected;
};

struct SubDesc {
    uint32_t start, len;
};

constexpr int kWave = 64;
constexpr int kFinBlock = 256;
constexpr int kScanBlock = 1024;
constexpr int kPiece = 256;                 // tokens per ring slot
constexpr int kRing = 4;                    // ring slots per wave
constexpr int kSubPerWave = 16;             // descriptors per wave
constexpr int kStreamWaves = 4;             // waves per block


__device__ __forceinline__ int64_t clamp_cu(const int32_t* cu, int64_t j, int64_t n) {
    // cu_seqlens is a documented precondition; clamping keeps a malformed one
    // from producing an out-of-range access (it can only give wrong numbers)
    const int64_t c = cu[j];
    return c < 0 ? 0 : (c > n ? n : c);
}

__device__ __forceinline__ uint32_t subchunks_of(const int32_t* cu, int64_t j, int64_t n) {
    const int64_t a = clamp_cu(cu, j, n), e = clamp_cu(cu, j + 1, n);
    return e > a ? (uint32_t)((e - a + kSubChunk - 1) / kSubChunk) : 0u;
}

// Inclusive scan of one value per thread over a kScanBlock-thread block.
__device__ uint32_t block_scan_incl(uint32_t x, uint32_t* sh) {
    const int tid = threadIdx.x;
    sh[tid] = x;
    __syncthreads();
    for (int off = 1; off < kScanBlock; off <<= 1) {
        const uint32_t y = tid >= off ? sh[tid - off] : 0u;
        __syncthreads();
        sh[tid] += y;
        __syncthreads();
    }
    const uint32_t r = sh[tid];
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(kScanBlock)
plan_count_kernel(const int32_t* __restrict__ cu, int64_t n, int64_t s, uint32_t* __restrict__ bsum) {
    __shared__ uint32_t sh[kScanBlock];
    const int64_t j = (int64_t)blockIdx.x * kScanBlock + threadIdx.x;
    const uint32_t c = j < s ? subchunks_of(cu, j, n) : 0u;
    const uint32_t incl = block_scan_incl(c, sh);
    if (threadIdx.x == kScanBlock - 1) bsum[blockIdx.x] = incl;
}

__global__ void __launch_bounds__(kScanBlock)
plan_scan_kernel(const uint32_t* __restrict__ bsum, int64_t nb, uint32_t* __restrict__ boff,
                 uint32_t* __restrict__ total) {
    __shared__ uint32_t sh[kScanBlock];
    __shared__ uint32_t last;
    uint32_t carry = 0;
    for (int64_t b0 = 0; b0 < nb; b0 += kScanBlock) {
        const int64_t b = b0 + threadIdx.x;
        const uint32_t x = b < nb ? bsum[b] : 0u;
        const uint32_t incl = block_scan_incl(x, sh);
        if (b < nb) boff[b] = carry + incl - x;
        if (threadIdx.x == kScanBlock - 1) last = incl;
        __syncthreads();
        carry += last;
        __syncthreads();
    }
    if (threadIdx.x == 0) *total = carry;
}

__global__ void __launch_bounds__(kScanBlock)
plan_write_kernel(const int32_t* __restrict__ cu, int64_t n, int64_t s, int64_t tmax,
                  const uint32_t* __restrict__ boff, uint32_t* __restrict__ seq_off,
                  SubDesc* __restrict__ desc) {
    __shared__ uint32_t sh[kScanBlock];
    const int64_t j = (int64_t)blockIdx.x * kScanBlock + threadIdx.x;
    const uint32_t c = j < s ? subchunks_of(cu, j, n) : 0u;
    const uint32_t incl = block_scan_incl(c, sh);
    if (j < s) {
        const uint32_t off = boff[blockIdx.x] + incl - c;
        seq_off[j] = off;
        const int64_t a = clamp_cu(cu, j, n), e = clamp_cu(cu, j + 1, n);
        // a well-formed cu_seqlens never reaches tmax; the bound keeps a
        // malformed one inside the descriptor array
        for (uint32_t k = 0; k < c && (int64_t)off + k < tmax; ++k) {
            const int64_t st = a + (int64_t)k * kSubChunk;
            const int64_t en = st + kSubChunk < e ? st + kSubChunk : e;
            desc[off + k] = SubDesc{(uint32_t)st, (uint32_t)(en - st)};
        }
    }
}

struct TokOut {
    float *delta, *ratio, *k1, *k2, *k3, *tis_w;
    uint8_t* clipped;
};

// One ring slot: a piece of lt and lr, and the 4-byte words holding its
// mask bytes (a piece's bytes span at most kPiece/4 + 1 words; 2 x 64 words
// are copied).
struct alignas(16) Slot {
    float lt[kPiece];
    float lr[kPiece];
    uint32_t mw[2 * kWave];
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma_dword(const void* g, void* l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)l, 4, 0, 0);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt low
// bits [3:0] and high bits [15:14]; expcnt [6:4] = 7 and lgkmcnt [11:8] = 15
// mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `ahead` pieces (kPer loads each) remain in flight.
template <int kPer>
__device__ __forceinline__ void wait_pieces_ahead(uint32_t ahead) {
    static_assert(kRing == 4, "cases cover up to three pieces ahead");
    switch (ahead) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<kPer>(); break;
        case 2: wait_vmcnt<2 * kPer>(); break;
        default: wait_vmcnt<3 * kPer>(); break;
    }
}

// e^d - 1 for finite |d| > 1/32 (the rare branch; |d| <= 1/32 uses a Taylor
// polynomial for e^d - 1 - d).  Range reduction d = k ln2 + r with
// |r| <= ln2 / 2 (ln2 split in a high part exact in 32 bits and a low part),
// e^r - 1 by a degree-12 Taylor polynomial (truncation < 1e-15 relative),
// then e^d - 1 = 2^k (e^r - 1) + (2^k - 1); both terms are exact-sign sums, so
// no cancellation beyond one rounding.  d > 709.78 overflows to +inf and
// d < -745 gives -1, as the exact value rounds.
__device__ __forceinline__ double expm1_large(double d) {
    if (d > 709.782712893384) return INFINITY;
    if (d < -745.0) return -1.0;
    const double kLn2Hi = 6.93147180369123816490e-01;   // 0x3FE62E42FEE00000
    const double kLn2Lo = 1.90821492927058770002e-10;
    const double k = rint(d * 1.4426950408889634);
    const double r = fma(-k, kLn2Lo, fma(-k, kLn2Hi, d));
    // e^r - 1 = r + r^2/2! + ... + r^12/12!
    double q = 1.0 / 479001600.0;
    q = fma(q, r, 1.0 / 39916800.0);
    q = fma(q, r, 1.0 / 3628800.0);
    q = fma(q, r, 1.0 / 362880.0);
    q = fma(q, r, 1.0 / 40320.0);
    q = fma(q, r, 1.0 / 5040.0);
    q = fma(q, r, 1.0 / 720.0);
    q = fma(q, r, 1.0 / 120.0);
    q = fma(q, r, 1.0 / 24.0);
    q = fma(q, r, 1.0 / 6.0);
    q = fma(q, r, 0.5);
    const double er1 = fma(q * r, r, r);                 // e^r - 1
    const int ki = (int)k;
    if (ki > 1023) {                                      // 2^k itself overflows
        return ldexp(er1 + 1.0, ki);
    }
    const double p2 = ldexp(1.0, ki);                     // 2^k, exact
    return fma(p2, er1, p2 - 1.0);
}

struct Acc {
    double sd, sd2, sk3, sem1, sabs, mx;   // sem1: sum of e^d - 1 over unclipped tokens
    uint32_t nvalid, nclip, nnan;
    __device__ void zero() { sd = sd2 = sk3 = sem1 = sabs = mx = 0; nvalid = nclip = nnan = 0; }
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The slot entries lane `lane` folds: lt and lr at offsets lane + 64 i and,
// with a mask, the mask bytes at mshift + lane + 64 i (i = 0..3), read in one
// asm block that ends with s_waitcnt lgkmcnt(0).  The ring is filled by LDS
// DMA; written as ordinary loads, the compiler cannot tell this slot from the
// ones still being filled and waits for every copy in flight (vmcnt(0))
// first, which would serialise the ring.  The explicit vmcnt waits of the
// main loop are what order these reads after the copies of their piece.
template <bool kMask>
__device__ __forceinline__ void read_slot(const Slot& sl, uint32_t mshift, int lane,
                                          float (&x)[4], float (&y)[4], uint32_t (&m)[4]) {
    const uint32_t a = lds_addr(&sl) + 4u * (uint32_t)lane;
    uint64_t p0, p1, p2, p3;
    if constexpr (kMask) {
        const uint32_t am = lds_addr(sl.mw) + mshift + (uint32_t)lane;
        asm volatile(
            "ds_read2st64_b32 %0, %8 offset1:4\n\t"
            "ds_read2st64_b32 %1, %8 offset0:1 offset1:5\n\t"
            "ds_read2st64_b32 %2, %8 offset0:2 offset1:6\n\t"
            "ds_read2st64_b32 %3, %8 offset0:3 offset1:7\n\t"
            "ds_read_u8 %4, %9\n\t"
            "ds_read_u8 %5, %9 offset:64\n\t"
            "ds_read_u8 %6, %9 offset:128\n\t"
            "ds_read_u8 %7, %9 offset:192\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(p0), "=&v"(p1), "=&v"(p2), "=&v"(p3), "=&v"(m[0]), "=&v"(m[1]), "=&v"(m[2]),
              "=&v"(m[3])
            : "v"(a), "v"(am)
            : "memory");
    } else {
        asm volatile(
            "ds_read2st64_b32 %0, %4 offset1:4\n\t"
            "ds_read2st64_b32 %1, %4 offset0:1 offset1:5\n\t"
            "ds_read2st64_b32 %2, %4 offset0:2 offset1:6\n\t"
            "ds_read2st64_b32 %3, %4 offset0:3 offset1:7\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(p0), "=&v"(p1), "=&v"(p2), "=&v"(p3)
            : "v"(a)
            : "memory");
        m[0] = m[1] = m[2] = m[3] = 1u;
    }
    const uint64_t p[4] = {p0, p1, p2, p3};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = __uint_as_float((uint32_t)p[i]);
        y[i] = __uint_as_float((uint32_t)(p[i] >> 32));
    }
}

// Fold the piece of a sub-chunk (start sub_start, length len) that begins at
// offset off0, read from slot `sl`: lane l takes offsets off0 + l + 64 i, i
// ascending, so across a sub-chunk's pieces each lane folds its offsets in
// ascending order.  Straight-line code: every slot entry is a valid copy, so
// the LDS reads are unconditional; a token that does not count (outside the
// sub-chunk, masked out or non-finite) gets delta = 0, which makes its d,
// d^2, k3 and |d| contributions exactly 0 with no further selects.  Counts
// come from ballots of single compares combined on the scalar unit.  k2 is
// accumulated as d^2 and halved once (a power-of-two scale: exact).  The
// truncated weight sum is assembled as n_unclipped + sum(e^d - 1 over
// unclipped) + C n_clipped, with e^d - 1 = d + k3.
template <bool kTok, bool kMask>
__device__ __forceinline__ void fold_piece(Acc& A, const Slot& sl, uint32_t mshift,
                                           uint32_t sub_start, uint32_t off0, uint32_t len,
                                           int lane, const StatsParamsDev& prm,
                                           const TokOut& tok) {
    static_assert(kPiece == 4 * kWave, "four slot entries per lane");
    float xs[4], ys[4];
    uint32_t ms[4];
    read_slot<kMask>(sl, mshift, lane, xs, ys, ms);
    const uint32_t lim = len - off0;                          // valid piece offsets < lim
#pragma unroll
    for (int i = 0; i < kPiece / kWave; ++i) {
        if ((uint32_t)(i * kWave) >= lim) break;              // uniform: rest of piece empty
        const uint32_t po = (uint32_t)(i * kWave + lane);      // offset in the piece
        const float x = xs[i];
        const float y = ys[i];
        const double draw = (double)x - (double)y;
        const uint64_t b_in = __builtin_amdgcn_ballot_w64(po < lim);
        const uint64_t b_m = kMask ? __builtin_amdgcn_ballot_w64(ms[i] != 0) : ~0ull;
        const uint64_t b_f = __builtin_amdgcn_ballot_w64(isfinite(draw));
        const uint64_t b_scored = b_in & b_m;
        const uint64_t b_fin = b_scored & b_f;
        const uint64_t bit = 1ull << lane;
        const bool fin = (b_fin & bit) != 0;
        const double d = fin ? draw : 0.0;
        // e^d - 1 - d without cancellation for |d| <= 1/32 (degree-6 Taylor,
        // truncation below 2e-11 relative)
        const double d2 = d * d;
        double p = 1.0 / 720.0;
        p = fma(p, d, 1.0 / 120.0);
        p = fma(p, d, 1.0 / 24.0);
        p = fma(p, d, 1.0 / 6.0);
        p = fma(p, d, 0.5);
        double k3 = d2 * p;
        if (!(fabs(d) <= 0.03125)) k3 = expm1_large(d) - d;            // rare
        const double em1 = d + k3;
        const uint64_t b_clip = __builtin_amdgcn_ballot_w64(draw > prm.log_c) & b_fin;
        const bool clipped = (b_clip & bit) != 0;
        A.sd += d;
        A.sd2 += d2;
        A.sk3 += k3;
        A.sem1 += clipped ? 0.0 : em1;
        A.sabs += fabs(d);
        A.mx = fmax(A.mx, fabs(d));
        A.nvalid += (uint32_t)__popcll(b_fin);
        A.nclip += (uint32_t)__popcll(b_clip);
        A.nnan += (uint32_t)__popcll(b_scored & ~b_f);
        if (kTok && po < lim) {
            // per-token outputs; a non-finite delta reports exp/expm1 as computed
            const bool scored = (b_scored & bit) != 0;
            const uint32_t t = sub_start + off0 + po;
            const double dd = scored ? draw : 0.0;
            const double r = 1.0 + em1;
            const double wgt = clipped ? prm.clip_c : (fin ? r : 0.0);
            const double rr = fin ? r : (scored ? exp(dd) : 1.0);
            const double kk3 = fin ? k3 : (scored ? expm1(dd) - dd : 0.0);
            if (tok.delta) tok.delta[t] = (float)dd;
            if (tok.ratio) tok.ratio[t] = (float)rr;
            if (tok.k1) tok.k1[t] = (float)(-dd);
            if (tok.k2) tok.k2[t] = (float)(0.5 * (dd * dd));
            if (tok.k3) tok.k3[t] = (float)kk3;
            if (tok.tis_w) tok.tis_w[t] = (float)wgt;
            if (tok.clipped) tok.clipped[t] = clipped ? 1 : 0;
        }
    }
}

// Cross-lane fold of a sub-chunk's fp64 sums: a fixed xor butterfly over the
// 64 lanes (partner distance 1, 2, 4, ..., 32).  Each step adds two values
// whose order does not matter (a + b == b + a bit for bit), so every lane ends
// with the same bits and the tree depends on lane positions only.  Lane
// shuffles touch no LDS memory, so nothing here has to wait for the ring's
// copies still in flight.
__device__ __forceinline__ double bfly_sum(double x) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ double bfly_max(double x) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x = fmax(x, __shfl_xor(x, m));
    return x;
}

// The sub-chunk's partial (valid in every lane).  Counts come from ballots
// already and are wave-uniform.
__device__ __forceinline__ SubPartial finish(const Acc& A, double clip_c) {
    SubPartial q;
    q.sd = bfly_sum(A.sd);
    q.sk2 = 0.5 * bfly_sum(A.sd2);
    q.sk3 = bfly_sum(A.sk3);
    const double sem1 = bfly_sum(A.sem1);
    q.sw = ((double)(A.nvalid - A.nclip) + sem1) + clip_c * (double)A.nclip;
    q.sabs = bfly_sum(A.sabs);
    q.maxabs = bfly_max(A.mx);
    q.nvalid = (int32_t)A.nvalid; q.nclip = (int32_t)A.nclip;
    q.nnan = (int32_t)A.nnan; q.pad = 0;
    return q;
}

template <bool kTok, bool kMask>
__global__ void __launch_bounds__(kWave * kStreamWaves)
stats_stream_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                    const uint8_t* __restrict__ mask, const SubDesc* __restrict__ desc,
                    const uint32_t* __restrict__ total, uint32_t tmax, StatsParamsDev prm,
                    TokOut tok, SubPartial* __restrict__ partial) {
    __shared__ Slot ring[kStreamWaves][kRing];
    __shared__ SubPartial stage[kStreamWaves][kSubPerWave];
    constexpr int kPer = 2 * (kPiece / kWave) + (kMask ? 2 : 0);   // DMA loads per piece
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    uint32_t T = __builtin_amdgcn_readfirstlane(*total);
    T = T < tmax ? T : tmax;
    const uint64_t k0 = ((uint64_t)blockIdx.x * kStreamWaves + wv) * kSubPerWave;
    if (k0 >= T) return;
    const uint32_t nsub = (uint32_t)(T - k0 < kSubPerWave ? T - k0 : kSubPerWave);
    Slot* R = ring[wv];

    // this wave's descriptors, one per lane; read by any lane with shfl
    const SubDesc my = lane < (int)nsub ? desc[k0 + lane] : SubDesc{0u, 0u};
    auto d_start = [&](uint32_t k) {
        return (uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)my.start, (int)k));
    };
    auto d_len = [&](uint32_t k) {
        return (uint32_t)__builtin_amdgcn_readfirstlane(__shfl((int)my.len, (int)k));
    };

    uint32_t npieces = 0;
    for (uint32_t k = 0; k < nsub; ++k) npieces += (d_len(k) + kPiece - 1) / kPiece;

    // issue iterator: (sub-chunk ik, piece ip)
    uint32_t ik = 0, ip = 0, is0 = d_start(0), il = d_len(0);
    auto issue = [&](uint32_t slot) {
        Slot& S = R[slot];
        const uint32_t st = is0 + ip * kPiece;
        const uint32_t en = st + kPiece < is0 + il ? st + kPiece : is0 + il;
        const uint32_t cnt = en - st;
        const float* blt = lt + st;              // uniform bases, small per-lane offsets
        const float* blr = lr + st;
#pragma unroll
        for (int j = 0; j < kPiece / kWave; ++j) {
            uint32_t o = (uint32_t)(j * kWave + lane);
            o = o < cnt ? o : cnt - 1;
            dma_dword(blt + o, S.lt + j * kWave);
            dma_dword(blr + o, S.lr + j * kWave);
        }
        if (kMask) {
            const uintptr_t m0 = (uintptr_t)(mask + st) & ~(uintptr_t)3;
            const uintptr_t m1 = ((uintptr_t)(mask + en) + 3) & ~(uintptr_t)3;
            const uint32_t nw = (uint32_t)((m1 - m0) >> 2);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t wd = (uint32_t)(j * kWave + lane);
                wd = wd < nw ? wd : nw - 1;
                dma_dword((const void*)(m0 + 4 * (uintptr_t)wd), S.mw + j * kWave);
            }
        }
        if (++ip * kPiece >= il) {
            ip = 0;
            if (++ik < nsub) { is0 = d_start(ik); il = d_len(ik); }
        }
    };

    uint32_t issued = 0;
    for (; issued < kRing - 1 && issued < npieces; ++issued) issue(issued);

    Acc A;
    A.zero();
    uint32_t fk = 0, fp = 0, fs = d_start(0), fl = d_len(0);
    for (uint32_t c = 0; c < npieces; ++c) {
        // the slot refilled here held piece c - 1, folded in the last iteration
        if (issued < npieces) { issue(issued % kRing); ++issued; }
        if (kTok) wait_vmcnt<0>();          // token stores share the counter
        else wait_pieces_ahead<kPer>(issued - c - 1);
        const Slot& S = R[c % kRing];
        const uint32_t mshift = kMask ? (uint32_t)((uintptr_t)(mask + fs + fp * kPiece) & 3) : 0u;
        fold_piece<kTok, kMask>(A, S, mshift, fs, fp * kPiece, fl, lane, prm, tok);
        if (++fp * kPiece >= fl) {
            const SubPartial q = finish(A, prm.clip_c);
            if (lane == 0) stage[wv][fk] = q;
            A.zero();
            fp = 0;
            if (++fk < nsub) { fs = d_start(fk); fl = d_len(fk); }
        }
    }
    // every ring load has completed (the last fold waited for vmcnt(0));
    // lane l writes 16 bytes of staged partial l / 4
    __builtin_amdgcn_s_waitcnt(0);
    const int e = lane >> 2, q4 = lane & 3;
    if (e < (int)nsub) ((uint4*)&partial[k0 + e])[q4] = ((const uint4*)&stage[wv][e])[q4];
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
seq_finalize_kernel(const int32_t* __restrict__ cu, int64_t n, int64_t s, int64_t tmax,
                    StatsParamsDev prm,
                    const uint32_t* __restrict__ seq_off, const SubPartial* __restrict__ partial,
                    SeqOut so, BatchAcc* __restrict__ blk) {
    __shared__ BatchAcc buf[kFinBlock];
    const int64_t j = (int64_t)blockIdx.x * kFinBlock + threadIdx.x;
    BatchAcc c = acc_zero();
    if (j < s) {
        const uint32_t nsub = subchunks_of(cu, j, n);
        double sd = 0, sk2 = 0, sk3 = 0, sw = 0, sabs = 0, mx = 0;
        int64_t nvalid = 0, nclip = 0, nnan = 0;
        if (nsub > 0) {
            const uint32_t off = seq_off[j];
            for (uint32_t k = 0; k < nsub && (int64_t)off + k < tmax; ++k) {
                const SubPartial p = partial[off + k];
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
    // sum over sequences of ceil(len / SC) <= n / SC + s
    p->tmax = (n + kSubChunk - 1) / kSubChunk + s;
    p->nblk_scan = (s + kScanBlock - 1) / kScanBlock;
    p->nblk_seq = (s + kFinBlock - 1) / kFinBlock;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    p->bsum_off = take((size_t)p->nblk_scan * 4);
    p->boff_off = take((size_t)p->nblk_scan * 4);
    p->total_off = take(4);
    p->seqoff_off = take((size_t)s * 4);
    p->desc_off = take((size_t)p->tmax * sizeof(SubDesc));
    p->part_off = take((size_t)p->tmax * sizeof(SubPartial));
    p->blk_off = take((size_t)(p->nblk_seq > 0 ? p->nblk_seq : 1) * sizeof(BatchAcc));
    p->total_bytes = off;
    return true;
}

hipError_t launch_mismatch_stats(const StatsPlan& p, const float* lt, const float* lr,
                                 const uint8_t* mask, const int32_t* cu,
                                 const StatsParamsDev& prm, const TokenOutPtrs& tok,
                                 const SeqOutPtrs& seq, double* batch, void* workspace,
                                 hipStream_t st) {
    unsigned char* ws = (unsigned char*)workspace;
    uint32_t* bsum = (uint32_t*)(ws + p.bsum_off);
    uint32_t* boff = (uint32_t*)(ws + p.boff_off);
    uint32_t* total = (uint32_t*)(ws + p.total_off);
    uint32_t* seq_off = (uint32_t*)(ws + p.seqoff_off);
    SubDesc* desc = (SubDesc*)(ws + p.desc_off);
    SubPartial* partial = (SubPartial*)(ws + p.part_off);
    BatchAcc* blk = (BatchAcc*)(ws + p.blk_off);
    TokOut to{tok.delta, tok.ratio, tok.k1, tok.k2, tok.k3, tok.tis_w, tok.clipped};
    SeqOut so{seq.n_valid, seq.n_clipped, seq.n_nan, seq.mean_delta, seq.mean_k1,
              seq.mean_k2, seq.mean_k3, seq.mean_tis_w, seq.reject};
    if (p.s > 0) {
        hipLaunchKernelGGL(plan_count_kernel, dim3((unsigned)p.nblk_scan), dim3(kScanBlock), 0, st,
                           cu, p.n, p.s, bsum);
        hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kScanBlock), 0, st, bsum, p.nblk_scan,
                           boff, total);
        hipLaunchKernelGGL(plan_write_kernel, dim3((unsigned)p.nblk_scan), dim3(kScanBlock), 0, st,
                           cu, p.n, p.s, p.tmax, boff, seq_off, desc);
        if (p.n > 0) {
            const int64_t waves = (p.tmax + kSubPerWave - 1) / kSubPerWave;
            const dim3 grid((unsigned)((waves + kStreamWaves - 1) / kStreamWaves));
            const dim3 bdim(kWave * kStreamWaves);
            const bool want_tok = to.delta || to.ratio || to.k1 || to.k2 || to.k3 || to.tis_w ||
                                  to.clipped;
            if (want_tok && mask)
                hipLaunchKernelGGL((stats_stream_kernel<true, true>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial);
            else if (want_tok)
                hipLaunchKernelGGL((stats_stream_kernel<true, false>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial);
            else if (mask)
                hipLaunchKernelGGL((stats_stream_kernel<false, true>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial);
            else
                hipLaunchKernelGGL((stats_stream_kernel<false, false>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial);
        }
        hipLaunchKernelGGL(seq_finalize_kernel, dim3((unsigned)p.nblk_seq), dim3(kFinBlock), 0, st,
                           cu, p.n, p.s, p.tmax, prm, seq_off, partial, so, blk);
    }
    if (batch)
        hipLaunchKernelGGL(batch_finalize_kernel, dim3(1), dim3(kFinBlock), 0, st, blk,
                           p.nblk_seq, batch);
    return hipGetLastError();
}

}  // namespace tim
