// stats.hip — training/rollout mismatch statistics for gfx950.
//
// Per token (mask != 0): delta = lt - lr in fp64 ("Diagnosing Training
// Inference Mismatch ... (VeXact)", eq. (1), token-level TIM), r = e^delta
// ("训推一致性与 determinism", section 2), k1 = -delta, k2 = delta^2/2,
// k3 = (r - 1) - delta ("RL: Training Inference Mismatch", KL-estimator
// table; VeXact K1/K3), truncated IS weight w = min(r, C) with a clip flag
// ("Train-Inference Consistency", section 4).  Per sequence: means over the
// valid tokens, the geometric-mean-ratio rejection flag (VeXact
// compensation table, r_corr-based sequence rejection; exp(mean delta) is
// the geometric mean of r, tested in the log domain) and its K3 form (mean
// k3 above a bound, the srs-k3 rows of the same table).  Per batch: token
// means and the mean of per-sequence means ("RL: Training Inference
// Mismatch", monitoring flow), and the is_* ratios named in
// "Train-Inference Consistency", section 5.
//
// The pass is HBM-bound: 9 bytes per token are read once.  Every sequence is
// cut into sub-chunks of at most kSubChunk tokens that start at the
// sequence's first token and every kSubChunk tokens after it.  A sub-chunk's
// sums are folded in an order that depends only on token offsets inside it,
// and a sequence's sums are its sub-chunks' sums added in ascending order,
// so a sequence's results never depend on the rest of the batch.
//
//   1. stats_stream: a fixed number of waves (at most kMaxStreamWaves), each
//      owning a contiguous token range.  A wave finds its first sequence in
//      cu_seqlens with a 64-way search, then walks sequences and sub-chunks
//      in token order and folds every sub-chunk that starts in its range: the
//      tokens stream in 256-token pieces through a ring of kBufs LDS slots
//      filled by LDS DMA (lane l folds piece offsets l + 64 i), and a
//      finished sub-chunk is folded across the wave with a fixed LDS
//      transpose + DPP tree.  A sequence whose sub-chunks all start in the range is finished
//      by the wave (per-sequence outputs, and its share of the batch sums in
//      the wave's partial).  Any other sub-chunk's sums go to slot
//      floor(c_j / kSubChunk) + j + k (strictly increasing in (j, k), so no
//      prefix sum is needed to place them), and the wave in whose range such
//      a sequence starts names it for step 2.
//   2. stats_final: one thread per streaming wave finishes the sequence that
//      wave named (its slots added in ascending order, exactly as a wave adds
//      them), adds the wave's partial; each block folds its threads with a
//      fixed tree, and the last block to finish folds the block partials with
//      a fixed tree into the batch aggregates.

#include "tim_internal.h"

#include <atomic>
#include <math.h>

namespace tim {
namespace {

// Sums of one sub-chunk (48 bytes).
struct alignas(16) SubPartial {
    double sd, sk2, sk3, sw;
    int32_t nvalid, nclip, nnan, pad;
};
static_assert(sizeof(SubPartial) == 48, "three 16-byte quarters");

// Contribution of one sequence to the batch, and the running fold of many.
struct alignas(16) BatchAcc {
    double sd, sk2, sk3, sw, sabs, maxabs;           // token sums
    double md, mk1, mk2, mk3;                        // sums of sequence means
    int64_t nvalid, nclip, nnan, nonempty, rejected, rejected_k3;
};

constexpr int kWave = 64;
constexpr int kFinBlock = 256;
constexpr int kPiece = 256;                 // tokens per piece (4 per lane)
constexpr int kStreamWaves = 4;             // waves per block (each works on its own)
constexpr uint32_t kBufs = 3;               // pieces in flight per wave (LDS ring slots)
constexpr int kFoldVals = 4;                // fp64 sums folded across lanes per sub-chunk
constexpr int64_t kMaxStreamWaves = 4096;   // streaming waves, at most (16 per CU)
constexpr int64_t kMinRange = 512;          // tokens per streaming wave, at least
constexpr uint32_t kSC = (uint32_t)kSubChunk;

// piece record flags
constexpr uint32_t kLastPiece = 1u;         // the piece ends its sub-chunk
constexpr uint32_t kLastSub = 2u;           // ... and that sub-chunk ends its sequence
constexpr uint32_t kComplete = 4u;          // the sequence is finished by this wave

// cu_seqlens is a documented precondition; clamping keeps a malformed one
// from producing an out-of-range access (it can only give wrong numbers)
__device__ __forceinline__ uint32_t clamp_c(int32_t c, uint32_t n) {
    return c < 0 ? 0u : ((uint32_t)c > n ? n : (uint32_t)c);
}

// clamp(cu[j]) for a wave-uniform j, through the scalar data cache: its
// wait (lgkmcnt) leaves the vector-memory copies in flight alone.
__device__ __forceinline__ uint32_t cu_scalar(const int32_t* __restrict__ cu, uint32_t j,
                                              uint32_t n) {
    int32_t c;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(c)
                 : "s"(cu + j)
                 : "memory");
    return clamp_c(c, n);
}

struct TokOut {
    float *delta, *ratio, *k1, *k2, *k3, *tis_w;
    uint8_t* clipped;
};

// e^d - 1 for finite |d| > 1/32 (the rare branch; |d| <= 1/32 uses a Taylor
// polynomial for e^d - 1 - d).  Cody and Waite's additive range reduction
// (W. J. Cody, W. Waite, "Software Manual for the Elementary Functions",
// 1980): d = k ln2 + r with |r| <= ln2 / 2, ln2 split in a high part whose
// product with k is exact and a low part (the usual published pair),
// e^r - 1 by a degree-12 Taylor polynomial (truncation < 1e-15 relative),
// then e^d - 1 = 2^k (e^r - 1) + (2^k - 1); both terms are exact-sign sums, so
// no cancellation beyond one rounding.  d > 709.78 overflows to +inf and
// d < -745 gives -1, as the exact value rounds.
__device__ __attribute__((noinline)) double expm1_large(double d) {
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
    // Per sub-chunk.  sclip: sum of e^d - 1 over clipped tokens; the
    // unclipped sum the truncated weight needs is (sd + sk3) - sclip.
    double sd, sd2, sk3, sclip;
    uint32_t nvalid, nclip, nnan;
    // Per wave, over all its sub-chunks: sum and maximum of |d|, which only
    // the batch aggregates use (no per-sequence output depends on them).
    double sabs, mx;
    __device__ void zero() { sd = sd2 = sk3 = sclip = 0; nvalid = nclip = nnan = 0; }
};

// A piece in registers for the fold: the lane's tokens 4 l .. 4 l + 3.
struct Regs {
    float x[4], y[4];
    uint32_t m[4];
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
constexpr int kRsrcWord3 = 0x00020000;   // buffer descriptor word 3: 32-bit data, no swizzle

// One ring slot in LDS: a piece's lt and lr (one dword per token, in token
// order), then its mask: four bytes per lane-quad of tokens (kMaskDw), or
// one zero-extended dword per token.
template <bool kMaskDw>
struct Slot {
    static constexpr int kMaskBytes = kMaskDw ? kPiece : 4 * kPiece;
    static constexpr int kBytes = 2 * 4 * kPiece + kMaskBytes;
};
// LDS DMA copies per piece: lt and lr as one 16-byte load per lane, the
// mask as one 4-byte load per lane (kMaskDw) or four 1-byte loads.
template <bool kMask, bool kMaskDw>
struct PieceLoads { static constexpr int value = !kMask ? 2 : (kMaskDw ? 3 : 6); };

// Copy the piece of tokens [st, st + 256) into a ring slot with LDS DMA.
// Lane l moves tokens st + 4 l .. st + 4 l + 3 of lt and lr (offsets
// relative to the descriptors' bases; the descriptors' extents end at the
// arrays' ends, and a dword out of range reads as 0, so no address leaves
// the arrays).  The mask: with kMaskDw lane l moves the four bytes from
// moff + 4 l, where moff places the last lane-quad that reaches the array's
// end on the array's last four bytes (a dword only partly in range would
// read as 0); the fold shifts such a lane's bytes back.  Otherwise four
// one-byte loads per lane (token 64 i + l of the piece, clamped to the
// array's end).
template <bool kMask, bool kMaskDw>
__device__ __forceinline__ void dma_piece(__amdgpu_buffer_rsrc_t rlt, __amdgpu_buffer_rsrc_t rlr,
                                          __amdgpu_buffer_rsrc_t rm, unsigned char* slot,
                                          uint32_t st, uint32_t mst, uint32_t mlast, int lane) {
    const uint32_t o = (st + 4u * (uint32_t)lane) * 4u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rlt, (lds_void*)slot, 16, o, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rlr, (lds_void*)(slot + 4 * kPiece), 16, o, 0, 0, 0);
    if constexpr (kMask) {
        if constexpr (kMaskDw) {
            uint32_t mo = mst + 4u * (uint32_t)lane;
            mo = mo < mlast ? mo : mlast;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (lds_void*)(slot + 8 * kPiece), 4, mo, 0,
                                                     0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t mo = mst + (uint32_t)(i * kWave + lane);
                mo = mo < mlast ? mo : mlast;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rm, (lds_void*)(slot + 8 * kPiece + i * 256),
                                                         1, mo, 0, 0, 0);
            }
        }
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Rows 0 .. 2 kHalf - 1 of a ring slot for lane l (row i: the piece's token
// 64 i + l), read in asm: the slot is filled by LDS DMA, which the
// compiler's own waits would otherwise guard with a wait for every copy in
// flight.  The caller has waited for the slot's copies.  kMaskDw: the mask
// byte of token t sits at byte t of the slot's mask, except in the array's
// last piece (tail), where a lane-quad that reaches past the array's end
// was read from the array's last four bytes: token t of such a quad q sits
// at byte 4 q + (mst + t - mlast) (tokens beyond the array read bytes of
// their own quad and are never counted).
template <int kRows, bool kMask, bool kMaskDw>
__device__ __forceinline__ void read_slot(Regs& r, const unsigned char* slot, int lane, bool tail,
                                          uint32_t mst, uint32_t mlast) {
    static_assert(kRows == 2 || kRows == 4, "two or four rows");
    const uint32_t base = lds_addr(slot);
    const uint32_t a = base + 4u * (uint32_t)lane;
    if constexpr (kRows == 4)
        asm volatile(
            "ds_read_b32 %0, %8\n\tds_read_b32 %1, %8 offset:256\n\t"
            "ds_read_b32 %2, %8 offset:512\n\tds_read_b32 %3, %8 offset:768\n\t"
            "ds_read_b32 %4, %8 offset:1024\n\tds_read_b32 %5, %8 offset:1280\n\t"
            "ds_read_b32 %6, %8 offset:1536\n\tds_read_b32 %7, %8 offset:1792"
            : "=&v"(r.x[0]), "=&v"(r.x[1]), "=&v"(r.x[2]), "=&v"(r.x[3]), "=&v"(r.y[0]),
              "=&v"(r.y[1]), "=&v"(r.y[2]), "=&v"(r.y[3])
            : "v"(a)
            : "memory");
    else
        asm volatile(
            "ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:256\n\t"
            "ds_read_b32 %2, %4 offset:1024\n\tds_read_b32 %3, %4 offset:1280"
            : "=&v"(r.x[0]), "=&v"(r.x[1]), "=&v"(r.y[0]), "=&v"(r.y[1])
            : "v"(a)
            : "memory");
    if constexpr (kMask && kMaskDw) {
        if (!tail) {
            const uint32_t b = base + (uint32_t)lane;
            if constexpr (kRows == 4)
                asm volatile(
                    "ds_read_u8 %0, %4 offset:2048\n\tds_read_u8 %1, %4 offset:2112\n\t"
                    "ds_read_u8 %2, %4 offset:2176\n\tds_read_u8 %3, %4 offset:2240\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(r.m[0]), "=&v"(r.m[1]), "=&v"(r.m[2]), "=&v"(r.m[3])
                    : "v"(b)
                    : "memory");
            else
                asm volatile(
                    "ds_read_u8 %0, %2 offset:2048\n\tds_read_u8 %1, %2 offset:2112\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(r.m[0]), "=&v"(r.m[1])
                    : "v"(b)
                    : "memory");
        } else {
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                const uint32_t t = 64u * i + (uint32_t)lane;
                const uint32_t q = t >> 2;
                const uint32_t mo = mst + 4u * q;
                uint32_t pos = t;
                if (mo > mlast) {
                    const uint32_t k = mst + t - mlast;
                    pos = 4u * q + (k < 3u ? k : 3u);
                }
                asm volatile("ds_read_u8 %0, %1 offset:2048\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(r.m[i])
                             : "v"(base + pos)
                             : "memory");
            }
        }
    } else if constexpr (kMask) {
        if constexpr (kRows == 4)
            asm volatile(
                "ds_read_b32 %0, %4 offset:2048\n\tds_read_b32 %1, %4 offset:2304\n\t"
                "ds_read_b32 %2, %4 offset:2560\n\tds_read_b32 %3, %4 offset:2816\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r.m[0]), "=&v"(r.m[1]), "=&v"(r.m[2]), "=&v"(r.m[3])
                : "v"(a)
                : "memory");
        else
            asm volatile(
                "ds_read_b32 %0, %2 offset:2048\n\tds_read_b32 %1, %2 offset:2304\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r.m[0]), "=&v"(r.m[1])
                : "v"(a)
                : "memory");
    } else {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < kRows; ++i) r.m[i] = 1u;
    }
}

// Wave mask of the lanes whose x is finite (v_cmp_class with the six finite
// classes: -normal, -denormal, -0, +0, +denormal, +normal), straight into
// scalar registers.  Every lane of the wave is active where this is used.
__device__ __forceinline__ uint64_t finite_mask(double x) {
    uint64_t m;
    asm("v_cmp_class_f64_e64 %0, %1, %2" : "=s"(m) : "v"(x), "s"(0x1F8));
    return m;
}

// max(m, |d|) as one v_max_f64 (both operands are finite, so no
// canonicalisation is needed)
__device__ __forceinline__ double max_abs(double m, double d) {
    double r;
    asm("v_max_f64 %0, %1, |%2|" : "=v"(r) : "v"(m), "v"(d));
    return r;
}

// fma(a, b, c) as one v_fma_f64 with c in vector registers, held across
// the loop (the compiler otherwise copies loop-invariant constants before a
// two-address fmac, and scalar registers are the scarcer kind here)
__device__ __forceinline__ double fma_s(double a, double b, double c) {
    double r;
    asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Fold rows i0 and i0 + 1 of a piece of a sub-chunk: lane l of row i holds
// piece offset 64 i + l; lim of the piece's tokens lie inside the sub-chunk
// (64 i0 < lim <= 256), tok0 is the piece's first token.  A piece is folded
// pair by pair, the second pair only when lim > 128, so lane l adds its
// offsets in ascending order; the two rows of a pair are independent until
// then, so their arithmetic interleaves.  A token that does not count (outside the
// sub-chunk, masked out or non-finite) gets d = 0, which makes its d, d^2,
// k3 and |d| contributions exactly 0 with no further selects.  Counts are
// popcounts of the wave masks; the rare ones (non-finite, clipped) are
// counted in the rare branch, which any such token sends the wave into.  k2
// is accumulated as d^2 and halved once (a power-of-two scale: exact).  For
// the truncated weight only the clipped tokens' e^d - 1 is summed (rare
// path); the unclipped sum is recovered as (sum d + sum k3) - that.
// The series' coefficients 1/120, 1/24, 1/6 in vector registers for the
// whole kernel: formed once and made opaque, so that the compiler keeps them
// rather than moving each into registers again before every use (v_fma_f64
// reads at most one scalar operand).
// log C, the clip threshold, rides along the same way: a vector operand of
// its compares instead of two scalar registers the kernel runs short of.
struct SeriesC {
    double c5, c4, c3, log_c;
};
__device__ __forceinline__ SeriesC series_c(double log_c) {
    SeriesC c{1.0 / 120.0, 1.0 / 24.0, 1.0 / 6.0, log_c};
    asm volatile("" : "+v"(c.c5), "+v"(c.c4), "+v"(c.c3), "+v"(c.log_c));
    return c;
}

template <int kI0, bool kTok, bool kMask, bool kFull, bool kClipRare>
__device__ __forceinline__ void fold_pair(Acc& A, const Regs& rg, uint32_t tok0, uint32_t lim,
                                          int lane, const StatsParamsDev& prm,
                                          const TokOut& tok, const SeriesC& sc3) {
    // kClipRare: log C >= 1/32, so a clipped token (d > log C) is among the
    // |d| > 1/32 tokens of the rare branch and needs no test of its own
    static_assert(!(kTok && kClipRare), "per-token outputs test the clip on every row");
    double draw[2], d[2], dp[2];
    uint64_t m_fin[2];
    uint64_t m_clip[kClipRare ? 1 : 2], m_sc[kTok ? 2 : 1];
    double k3x[kTok ? 2 : 1];                      // per-token k3, for the outputs
    uint64_t rare = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        draw[i] = (double)rg.x[kI0 + i] - (double)rg.y[kI0 + i];
        // lane predicates as wave masks: each ballot is one compare, the
        // combinations are scalar, and inverse_ballot reads a lane's bit back
        uint64_t sc = kMask ? __builtin_amdgcn_ballot_w64((uint8_t)rg.m[kI0 + i] != 0) : ~0ull;
        if constexpr (!kFull) sc &= __builtin_amdgcn_ballot_w64((uint32_t)(64 * (kI0 + i) + lane) < lim);
        m_fin[i] = sc & finite_mask(draw[i]);
        A.nvalid += (uint32_t)__popcll(m_fin[i]);
        rare |= sc & ~m_fin[i];                        // non-finite: counted in the branch
        if constexpr (kTok) m_sc[i] = sc;
        if constexpr (!kClipRare) {
            m_clip[i] = m_fin[i] & __builtin_amdgcn_ballot_w64(draw[i] > sc3.log_c);
            rare |= m_clip[i];
        }
        d[i] = __builtin_amdgcn_inverse_ballot_w64(m_fin[i]) ? draw[i] : 0.0;
        // e^d - 1 - d = d dp for |d| <= 1/32, dp = d (1/2 + d/6 + d^2/24 +
        // d^3/120), truncation below 4e-9 relative
        double p = fma_s(d[i], sc3.c5, sc3.c4);
        p = fma_s(p, d[i], sc3.c3);
        p = fma_s(p, d[i], 0.5);
        dp[i] = d[i] * p;
        rare |= __builtin_amdgcn_ballot_w64(!(fabs(d[i]) <= 0.03125));
        if constexpr (kTok) k3x[i] = d[i] * dp[i];
    }
    if (rare != 0) {                                   // uniform test, rarely taken
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint64_t sc = kTok ? m_sc[i]
                                     : (kMask ? __builtin_amdgcn_ballot_w64((uint8_t)rg.m[kI0 + i] != 0)
                                              : ~0ull) &
                                           (kFull ? ~0ull
                                                  : __builtin_amdgcn_ballot_w64(
                                                        (uint32_t)(64 * (kI0 + i) + lane) < lim));
            A.nnan += (uint32_t)__popcll(sc & ~m_fin[i]);
            const uint64_t clip = kClipRare
                                      ? m_fin[i] & __builtin_amdgcn_ballot_w64(draw[i] > sc3.log_c)
                                      : m_clip[i];
            A.nclip += (uint32_t)__popcll(clip);
            const bool big = !(fabs(d[i]) <= 0.03125);
            double k3 = d[i] * dp[i];
            if (big) {
                // the exact e^d - 1 - d, added here; the row's fused add
                // below then adds d * 0
                k3 = expm1_large(d[i]) - d[i];
                double e = k3;
                asm volatile("" : "+v"(e));            // keeps this work inside the branch
                A.sk3 += e;
                dp[i] = 0.0;
            }
            if (__builtin_amdgcn_inverse_ballot_w64(clip)) {
                double e = d[i] + k3;
                asm volatile("" : "+v"(e));
                A.sclip += e;
            }
            if constexpr (kTok) {
                m_clip[i] = clip;
                k3x[i] = k3;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        A.sd += d[i];
        A.sd2 = fma(d[i], d[i], A.sd2);
        A.sk3 = fma(d[i], dp[i], A.sk3);
        A.sabs += fabs(d[i]);
        A.mx = max_abs(A.mx, d[i]);
    }
    if constexpr (kTok) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t po = (uint32_t)(64 * (kI0 + i) + lane);  // offset in the piece
            if (po < lim) {
                // per-token outputs; a non-finite delta reports exp/expm1 as computed
                const bool scored = __builtin_amdgcn_inverse_ballot_w64(m_sc[i]);
                const bool fin = __builtin_amdgcn_inverse_ballot_w64(m_fin[i]);
                const bool clipped = __builtin_amdgcn_inverse_ballot_w64(m_clip[i]);
                const uint32_t t = tok0 + po;
                const double dd = scored ? draw[i] : 0.0;
                const double k3 = k3x[i];
                const double em1 = d[i] + k3;
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
}


// 64-bit value of the lane selected by a DPP control (both 32-bit halves
// moved with v_mov_b32_dpp).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, 0xf,
                                                              0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Cross-lane fold of a sub-chunk's four fp64 sums, in a fixed order that
// depends on lane positions only:
//   1. every lane stores its four values to the wave's scratch: v[value][lane];
//   2. lane j < 32 sums v[j / 8][8 (j % 8) .. 8 (j % 8) + 7] left to right;
//   3. the eight partials of a value (lanes 8 v .. 8 v + 7) are combined by
//      three DPP steps: neighbours (quad_perm 1,0,3,2), pairs (quad_perm
//      2,3,0,1), half-rows (row_half_mirror);
//   4. lane 8 v holds value v and is read into scalar registers.
// A wave's LDS operations complete in issue order, so the reads see the
// writes without a wait between them; the read block ends in lgkmcnt(0).
__device__ __forceinline__ SubPartial finish(const Acc& A, double clip_c, int lane, const double* scratch) {
    const uint32_t base = lds_addr(scratch);
    const uint32_t aw = base + 8u * (uint32_t)lane;               // v[0][lane]
    asm volatile(
        "ds_write2st64_b64 %0, %1, %2 offset1:1\n\t"
        "ds_write2st64_b64 %0, %3, %4 offset0:2 offset1:3"
        :
        : "v"(aw), "v"(A.sd), "v"(A.sd2), "v"(A.sk3), "v"(A.sclip)
        : "memory");
    // lanes 32..63 repeat lanes 0..31 (in range; their results are unused)
    const int j = lane & 31;
    const uint32_t ar = base + 8u * (uint32_t)((j >> 3) * kWave + (j & 7) * 8);
    typedef __attribute__((__vector_size__(2 * sizeof(double)))) double f64x2;
    f64x2 r0, r1, r2, r3;
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:16\n\t"
        "ds_read_b128 %2, %4 offset:32\n\t"
        "ds_read_b128 %3, %4 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(ar)
        : "memory");
    double t = r0[0];
    t += r0[1];
    t += r1[0];
    t += r1[1];
    t += r2[0];
    t += r2[1];
    t += r3[0];
    t += r3[1];
    t += dpp_f64<0xB1>(t);                                         // quad_perm 1,0,3,2
    t += dpp_f64<0x4E>(t);                                         // quad_perm 2,3,0,1
    t += dpp_f64<0x141>(t);                                        // row_half_mirror
    SubPartial q;
    q.sd = readlane_f64(t, 0);
    q.sk2 = 0.5 * readlane_f64(t, 8);
    q.sk3 = readlane_f64(t, 16);
    const double sem1 = (q.sd + q.sk3) - readlane_f64(t, 24);     // unclipped e^d - 1
    q.sw = ((double)(A.nvalid - A.nclip) + sem1) + clip_c * (double)A.nclip;
    q.nvalid = (int32_t)A.nvalid; q.nclip = (int32_t)A.nclip;
    q.nnan = (int32_t)A.nnan; q.pad = 0;
    return q;
}

// Fixed xor butterfly over the 64 lanes (partner distance 1, 2, ..., 32);
// a + b == b + a bit for bit, so every lane ends with the same bits.
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

__device__ __forceinline__ void acc_add(BatchAcc& x, const BatchAcc& y) {
    x.sd += y.sd; x.sk2 += y.sk2; x.sk3 += y.sk3; x.sw += y.sw; x.sabs += y.sabs;
    x.maxabs = fmax(x.maxabs, y.maxabs);
    x.md += y.md; x.mk1 += y.mk1; x.mk2 += y.mk2; x.mk3 += y.mk3;
    x.nvalid += y.nvalid; x.nclip += y.nclip; x.nnan += y.nnan;
    x.nonempty += y.nonempty; x.rejected += y.rejected; x.rejected_k3 += y.rejected_k3;
}

__device__ __forceinline__ BatchAcc acc_zero() {
    BatchAcc a;
    a.sd = a.sk2 = a.sk3 = a.sw = a.sabs = a.maxabs = 0;
    a.md = a.mk1 = a.mk2 = a.mk3 = 0;
    a.nvalid = a.nclip = a.nnan = a.nonempty = a.rejected = a.rejected_k3 = 0;
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
    uint8_t *reject, *reject_k3;
};

// A sequence's sums: its sub-chunks' sums added in ascending order, by the
// streaming wave or by the finalize kernel with this same code.
struct SeqSums {
    double sd, sk2, sk3, sw;
    int64_t nvalid, nclip, nnan;
};

__device__ __forceinline__ SeqSums seq_zero() {
    SeqSums a;
    a.sd = a.sk2 = a.sk3 = a.sw = 0.0;
    a.nvalid = a.nclip = a.nnan = 0;
    return a;
}

__device__ __forceinline__ void seq_add(SeqSums& a, const SubPartial& p) {
    a.sd += p.sd; a.sk2 += p.sk2; a.sk3 += p.sk3; a.sw += p.sw;
    a.nvalid += p.nvalid; a.nclip += p.nclip; a.nnan += p.nnan;
}

// Means and rejection flags of sequence j, written to the per-sequence
// outputs when `writer`, and the sequence's contribution added to c.
__device__ __forceinline__ void seq_finish(uint32_t j, const SeqSums& a, const StatsParamsDev& prm,
                                           const SeqOut& so, bool writer, BatchAcc& c) {
    const int64_t nvalid = a.nvalid;
    const double nv = (double)nvalid;
    const double md = nvalid ? a.sd / nv : 0.0;
    const double mk1 = nvalid ? (-a.sd) / nv : 0.0;
    const double mk2 = nvalid ? a.sk2 / nv : 0.0;
    const double mk3 = nvalid ? a.sk3 / nv : 0.0;
    const double mw = nvalid ? a.sw / nv : 0.0;
    const bool rej = nvalid > 0 && (md < prm.seq_lo || md > prm.seq_hi);
    const bool rej_k3 = nvalid > 0 && mk3 > prm.seq_k3_hi;   // K3 form
    if (writer) {
        if (so.n_valid) so.n_valid[j] = (int32_t)nvalid;
        if (so.n_clipped) so.n_clipped[j] = (int32_t)a.nclip;
        if (so.n_nan) so.n_nan[j] = (int32_t)a.nnan;
        if (so.mean_delta) so.mean_delta[j] = md;
        if (so.mean_k1) so.mean_k1[j] = mk1;
        if (so.mean_k2) so.mean_k2[j] = mk2;
        if (so.mean_k3) so.mean_k3[j] = mk3;
        if (so.mean_tis_w) so.mean_tis_w[j] = mw;
        if (so.reject) so.reject[j] = rej ? 1 : 0;
        if (so.reject_k3) so.reject_k3[j] = rej_k3 ? 1 : 0;
    }
    c.sd += a.sd; c.sk2 += a.sk2; c.sk3 += a.sk3; c.sw += a.sw;
    c.nvalid += nvalid; c.nclip += a.nclip; c.nnan += a.nnan;
    if (nvalid > 0) {
        c.md += md; c.mk1 += mk1; c.mk2 += mk2; c.mk3 += mk3;
        c.nonempty += 1;
        c.rejected += rej ? 1 : 0;
        c.rejected_k3 += rej_k3 ? 1 : 0;
    }
}

// First j in [0, s) with clamp(cu[j]) >= x (s if none), for a monotone
// cu_seqlens; 64 entries are probed per step.  For any input the result
// lies in [0, s] and every probe inside cu[0 .. s - 1].
__device__ uint32_t lower_bound_cu(const int32_t* __restrict__ cu, uint32_t s, uint32_t n,
                                   uint32_t x, int lane) {
    uint32_t lo = 0, hi = s;                        // the answer is in [lo, hi]
    while (hi - lo > (uint32_t)kWave) {
        const uint32_t step = (hi - lo + kWave - 1) / kWave;
        const uint64_t idx = (uint64_t)lo + (uint64_t)lane * step;
        const bool below = idx < hi && clamp_c(cu[idx], n) < x;
        const uint32_t t = (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(below));
        // probes 0 .. t - 1 are below x: the answer is in
        // (lo + (t - 1) step, min(hi, lo + t step)]
        const uint32_t nlo = t == 0 ? lo : lo + (t - 1) * step + 1;
        const uint64_t up = (uint64_t)lo + (uint64_t)t * step;
        hi = up < hi ? (uint32_t)up : hi;
        lo = nlo < hi ? nlo : hi;
    }
    const uint32_t idx = lo + (uint32_t)lane;
    const bool below = idx < hi && clamp_c(cu[idx], n) < x;
    return lo + (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(below));
}

// One piece to fold: tokens [start, start + lim) of a sub-chunk; lim == 0:
// none.  id: the sequence's index if the wave finishes it (kComplete), else
// the sub-chunk's slot.
struct PieceRec {
    uint32_t start, lim_flags, id;     // lim_flags = lim | flags << 16
};

// A result waiting in LDS for the wave's next flush: a finished sequence's
// sums (id = its index) or a sub-chunk's sums (id = its slot), the id kept
// in the sums' spare word with the kind in its top bit.
typedef SubPartial StageEnt;
constexpr uint32_t kSlotKind = 0x80000000u;     // set for a sub-chunk's sums
constexpr int kStage = 21;                      // entries per wave (one per lane at a flush)

// Contribution of a lane's staged entry to the wave's batch sums, folded
// over the wave's lanes with a fixed butterfly.
__device__ __forceinline__ void wave_fold_acc(BatchAcc& c) {
    c.sd = bfly_sum(c.sd); c.sk2 = bfly_sum(c.sk2); c.sk3 = bfly_sum(c.sk3);
    c.sw = bfly_sum(c.sw);
    c.md = bfly_sum(c.md); c.mk1 = bfly_sum(c.mk1); c.mk2 = bfly_sum(c.mk2);
    c.mk3 = bfly_sum(c.mk3);
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        c.nvalid += __shfl_xor(c.nvalid, m);
        c.nclip += __shfl_xor(c.nclip, m);
        c.nnan += __shfl_xor(c.nnan, m);
        c.nonempty += __shfl_xor(c.nonempty, m);
        c.rejected += __shfl_xor(c.rejected, m);
        c.rejected_k3 += __shfl_xor(c.rejected_k3, m);
    }
}

template <bool kTok, bool kMask, bool kMaskDw>
__global__ void __launch_bounds__(kWave * kStreamWaves)
stats_stream_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                    const uint8_t* __restrict__ mask, const int32_t* __restrict__ cu,
                    uint32_t n, uint32_t s, uint32_t range, uint32_t nwaves, StatsParamsDev prm,
                    TokOut tok, SeqOut so, SubPartial* __restrict__ slots,
                    BatchAcc* __restrict__ wpart, int32_t* __restrict__ cross,
                    uint32_t* __restrict__ ticket) {
    __shared__ __attribute__((aligned(16)))
    unsigned char ring[kStreamWaves][kBufs][Slot<kMaskDw>::kBytes];
    __shared__ __attribute__((aligned(16))) double scratch[kStreamWaves][kFoldVals * kWave];
    __shared__ StageEnt stage[kStreamWaves][kStage];
    // per wave, touched by its lane 0 only: the wave's share of the batch sums
    __shared__ BatchAcc acc_lds[kStreamWaves];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const uint32_t w = blockIdx.x * kStreamWaves + (uint32_t)wv;
    if (w >= nwaves) return;
    if (w == 0 && lane == 0) *ticket = 0u;         // the finalize kernel's counter
    if (lane == 0) acc_lds[wv] = acc_zero();
    const bool last = w == nwaves - 1;
    const uint32_t b0 = w * range;
    const uint32_t b1 = last ? n : b0 + range;     // the last wave also owns c_j == n
    const uint32_t ja = lower_bound_cu(cu, s, n, b0, lane);

    // Owned empty sequences (c_j in this wave's range, c_{j+1} == c_j): zero
    // outputs, nothing for the batch; 64 sequences per round.
    for (uint32_t jb = ja;; jb += kWave) {
        const uint32_t jj = jb + (uint32_t)lane;
        bool more = false;
        if (jj < s) {
            const uint32_t c = clamp_c(cu[jj], n);
            if (last || c < b1) {
                more = true;
                if (clamp_c(cu[jj + 1], n) <= c) {
                    BatchAcc dummy = acc_zero();
                    seq_finish(jj, seq_zero(), prm, so, true, dummy);
                }
            }
        }
        if (__builtin_amdgcn_ballot_w64(more) != ~0ull) break;
    }

    // ---- the walk over sequences and sub-chunks (wave-uniform state): the
    // next piece starts at pos, inside the sub-chunk ending at se, of
    // sequence j ending at ej; id is j if this wave finishes the sequence
    // (complete), else the current sub-chunk's slot.
    uint32_t pos = 0, se = 0, ej = 0, j = 0, id = 0;
    bool complete = false, done = false;
    int32_t crossj = -1;                           // owned sequence left to step 2

    // Enter the first sequence at or after jj that this wave owns and that
    // has a token (owned empty sequences are written by the pass above).
    auto enter = [&](uint32_t jj) {
        for (;;) {
            if (jj >= s) { done = true; return; }
            const uint32_t c = cu_scalar(cu, jj, n);
            if (!last && c >= b1) { done = true; return; }
            const uint32_t e = cu_scalar(cu, jj + 1, n);
            if (e > c) {
                j = jj; ej = e; pos = c;
                se = c + kSC < e ? c + kSC : e;
                const uint32_t K = (e - c + kSC - 1) / kSC;
                complete = last || c + (K - 1) * kSC < b1;
                // slot of sub-chunk 0: floor(c / SC) + j (below floor(n / SC) +
                // s + 1 for any clamped c_j <= n and j < s)
                id = complete ? jj : c / kSC + jj;
                if (!complete) crossj = (int32_t)jj;
                return;
            }
            ++jj;
        }
    };
    {
        bool cont = false;
        if (ja > 0) {
            // the sequence that contains token b0, started before it: its
            // sub-chunks that start in [b0, b1)
            const uint32_t c = cu_scalar(cu, ja - 1, n), e = cu_scalar(cu, ja, n);
            if (c < b0 && e > b0) {
                const uint32_t k = (b0 - c + kSC - 1) / kSC;
                const uint32_t st = c + k * kSC;
                if (st < e && st < b1) {
                    j = ja - 1; ej = e; pos = st;
                    se = st + kSC < e ? st + kSC : e;
                    complete = false;
                    id = c / kSC + (ja - 1) + k;
                    cont = true;
                }
            }
        }
        if (!cont) enter(ja);
    }
    // The next piece of the walk, then advance.
    auto next_rec = [&](PieceRec& r) {
        r.start = pos;
        const uint32_t left = se - pos;
        const bool lastp = left <= (uint32_t)kPiece;
        const uint32_t flags = (lastp ? kLastPiece : 0u) | (complete ? kComplete : 0u) |
                               (lastp && se == ej ? kLastSub : 0u);
        r.lim_flags = (lastp ? left : (uint32_t)kPiece) | (flags << 16);
        r.id = id;
        if (!lastp) { pos += kPiece; return; }
        pos = se;
        if (pos < ej) {
            // later sub-chunks of this sequence start in later waves' ranges
            if (pos >= b1) { done = true; return; }
            se = pos + kSC < ej ? pos + kSC : ej;
            if (!complete) ++id;
            return;
        }
        enter(j + 1);
    };

    Acc A;
    A.zero();
    A.sabs = 0.0;
    A.mx = 0.0;
    const SeriesC sc3 = series_c(prm.log_c);
    uint32_t nstage = 0;                           // staged entries (uniform)
    SeqSums S = seq_zero();                        // the sequence being finished
    // Buffer descriptors based at the wave's first token: every copy's
    // offset is 32-bit (the wave's tokens span less than a range plus a
    // sub-chunk past it), and the extents end at the arrays' ends.
    const uint32_t s0 = done ? 0u : pos;
    const uint64_t span = (uint64_t)(n - s0);
    const int ext4 = (int)(uint32_t)(span * 4 < 0xffffffffull ? span * 4 : 0xffffffffull);
    const __amdgpu_buffer_rsrc_t rlt =
        __builtin_amdgcn_make_buffer_rsrc((void*)(lt + s0), (short)0, ext4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rlr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(lr + s0), (short)0, ext4, kRsrcWord3);
    // mask: kMaskDw (n >= 4) reads lane-quads, the last of which sits on the
    // array's last four bytes, so its base is at most n - 4
    const uint32_t mbase = kMaskDw ? (s0 < n - 4 ? s0 : n - 4) : s0;
    const uint32_t mlast = kMaskDw ? n - 4 - mbase : (n > s0 ? n - 1 - s0 : 0u);
    const __amdgpu_buffer_rsrc_t rm =
        kMask ? __builtin_amdgcn_make_buffer_rsrc((void*)(mask + mbase), (short)0,
                                                  (int)(n - mbase), kRsrcWord3)
              : rlt;
    constexpr int kLoads = PieceLoads<kMask, kMaskDw>::value;
    const bool clip_rare = prm.log_c >= 0.03125;
    // No global store happens between a round's first copy and its last
    // fold, and every issue makes the same kLoads copies: a slot's copies
    // are complete once at most (kBufs - 1) kLoads copies are in flight, and
    // each fold waits for exactly that.  Results wait in LDS; a round stops
    // issuing when the stage could overflow, and the stage is written out
    // between rounds.
    for (;;) {
        if (!done) {
            bool paused = false;
            PieceRec r0, r1, r2;
            next_rec(r0);
            // Past the round's end every issue copies the round's first piece
            // again (never folded): the same copies on every path.
            const uint32_t d_start = r0.start;
            dma_piece<kMask, kMaskDw>(rlt, rlr, rm, ring[wv][0], d_start - s0, d_start - mbase,
                                      mlast, lane);
            auto issue = [&](unsigned char* slot, PieceRec& r) {
                const bool go = !done && !paused;
                if (go) next_rec(r);
                else r.lim_flags = 0u;
                const uint32_t st = go ? r.start : d_start;
                dma_piece<kMask, kMaskDw>(rlt, rlr, rm, slot, st - s0, st - mbase, mlast, lane);
            };
            issue(ring[wv][1], r1);
            issue(ring[wv][2], r2);
            // Fold the piece in slot (if any).  The slot is refilled as soon as
            // its tokens are in registers, before the fold, so the copy runs
            // under the fold's arithmetic.
            auto step = [&](unsigned char* slot, PieceRec& r) -> bool {
                const PieceRec cur = r;
                const uint32_t lim = cur.lim_flags & 0xffffu, flags = cur.lim_flags >> 16;
                if (lim == 0) return false;
                // the array's last piece, whose last lane-quads of the mask
                // were read from the array's last four bytes
                const bool tail = kMask && kMaskDw && cur.start - mbase + 4u * (kWave - 1) > mlast;
                wait_vmcnt<(kBufs - 1) * kLoads>();
                Regs g;
                if (lim > 2u * kWave)
                    read_slot<4, kMask, kMaskDw>(g, slot, lane, tail, cur.start - mbase, mlast);
                else
                    read_slot<2, kMask, kMaskDw>(g, slot, lane, tail, cur.start - mbase, mlast);
                issue(slot, r);
#define TIM_FOLD2(I0, F, C) \
    fold_pair<I0, kTok, kMask, F, C>(A, g, cur.start, lim, lane, prm, tok, sc3)
                if (lim == (uint32_t)kPiece) {
                    if (!kTok && clip_rare) { TIM_FOLD2(0, true, !kTok); TIM_FOLD2(2, true, !kTok); }
                    else { TIM_FOLD2(0, true, false); TIM_FOLD2(2, true, false); }
                } else {
                    if (!kTok && clip_rare) {
                        TIM_FOLD2(0, false, !kTok);
                        if (lim > 2u * kWave) TIM_FOLD2(2, false, !kTok);
                    } else {
                        TIM_FOLD2(0, false, false);
                        if (lim > 2u * kWave) TIM_FOLD2(2, false, false);
                    }
                }
#undef TIM_FOLD2
                if (flags & kLastPiece) {
                    const SubPartial q = finish(A, prm.clip_c, lane, scratch[wv]);
                    A.zero();
                    if (flags & kComplete) {
                        seq_add(S, q);
                        if (flags & kLastSub) {
                            if (lane == 0) {
                                StageEnt& e = stage[wv][nstage];
                                e.sd = S.sd; e.sk2 = S.sk2; e.sk3 = S.sk3; e.sw = S.sw;
                                e.nvalid = (int32_t)S.nvalid; e.nclip = (int32_t)S.nclip;
                                e.nnan = (int32_t)S.nnan; e.pad = (int32_t)cur.id;
                            }
                            S = seq_zero();
                            ++nstage;
                        }
                    } else {
                        if (lane == 0) {
                            StageEnt& e = stage[wv][nstage];
                            e = q;
                            e.pad = (int32_t)(cur.id | kSlotKind);
                        }
                        ++nstage;
                    }
                    // room for what the pieces in flight (issued ones included)
                    // can still finish
                    if (nstage + kBufs >= (uint32_t)kStage) paused = true;
                }
                return true;
            };
            for (;;) {
                if (!step(ring[wv][0], r0)) break;
                if (!step(ring[wv][1], r1)) break;
                if (!step(ring[wv][2], r2)) break;
            }
        }
        // write the staged results out, one per lane
        {
            BatchAcc c = acc_zero();
            if ((uint32_t)lane < nstage) {
                StageEnt e = stage[wv][lane];
                const uint32_t id = (uint32_t)e.pad;
                if (!(id & kSlotKind)) {
                    SeqSums a;
                    a.sd = e.sd; a.sk2 = e.sk2; a.sk3 = e.sk3; a.sw = e.sw;
                    a.nvalid = e.nvalid; a.nclip = e.nclip; a.nnan = e.nnan;
                    seq_finish(id, a, prm, so, true, c);
                } else {
                    e.pad = 0;
                    slots[id & ~kSlotKind] = e;
                }
            }
            if (nstage > 0) {
                wave_fold_acc(c);
                if (lane == 0) acc_add(acc_lds[wv], c);
            }
            nstage = 0;
        }
        if (done) break;
    }
    wait_vmcnt<0>();                               // no copy in flight into LDS at the end
    const double wsabs = bfly_sum(A.sabs), wmx = bfly_max(A.mx);
    if (lane == 0) {
        BatchAcc c = acc_lds[wv];
        c.sabs += wsabs;
        c.maxabs = fmax(c.maxabs, wmx);
        wpart[w] = c;
        cross[w] = crossj;
    }
}

__global__ void __launch_bounds__(kFinBlock)
stats_final_kernel(const int32_t* __restrict__ cu, uint32_t n, uint32_t s, StatsParamsDev prm,
                   const SubPartial* __restrict__ slots, uint64_t nslots,
                   const BatchAcc* __restrict__ wpart, const int32_t* __restrict__ cross,
                   uint32_t nwaves, SeqOut so, BatchAcc* __restrict__ blk,
                   uint32_t* __restrict__ ticket, double* __restrict__ out) {
    __shared__ BatchAcc buf[kFinBlock];
    __shared__ uint32_t is_last;
    const uint32_t w = blockIdx.x * kFinBlock + threadIdx.x;
    BatchAcc c = acc_zero();
    if (w < nwaves) {
        c = wpart[w];
        const int32_t jj = cross[w];
        if (jj >= 0 && (uint32_t)jj < s) {
            // the sequence that starts in wave w's range and ends past it
            const uint32_t c0 = clamp_c(cu[jj], n), e0 = clamp_c(cu[jj + 1], n);
            SeqSums a = seq_zero();
            if (e0 > c0) {
                const uint32_t K = (e0 - c0 + kSC - 1) / kSC;
                const uint64_t base = (uint64_t)(c0 / kSC) + (uint32_t)jj;
                for (uint32_t k = 0; k < K && base + k < nslots; ++k) seq_add(a, slots[base + k]);
            }
            seq_finish((uint32_t)jj, a, prm, so, true, c);
        }
    }
    buf[threadIdx.x] = c;
    __syncthreads();
    block_tree(buf);
    if (!out) return;
    // the last block to get here folds every block's partial
    if (threadIdx.x == 0) {
        blk[blockIdx.x] = buf[0];
        __threadfence();
        is_last = atomicAdd(ticket, 1u) == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    c = acc_zero();
    for (uint32_t i = threadIdx.x; i < gridDim.x; i += kFinBlock) acc_add(c, blk[i]);
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
        out[19] = dv((double)a.rejected_k3, ns);  // TIM_B_REJECT_K3_FRAC
        out[20] = (double)a.rejected_k3;
    }
}

// Streaming waves the current device holds at once (the kernel's blocks
// per CU from the occupancy query, times its CUs, times kStreamWaves),
// looked up once per device.
hipError_t stream_waves_per_device(bool with_mask, int64_t* out) {
    constexpr int kDevs = 64;
    static std::atomic<int64_t> cached[2][kDevs];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevs) return hipErrorInvalidDevice;
    int64_t v = cached[with_mask][dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, blocks = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        // the mask variant has the larger LDS footprint of the two that
        // stream large batches (with or without per-token outputs alike)
        e = with_mask ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &blocks, stats_stream_kernel<false, true, true>, kWave * kStreamWaves, 0)
                      : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &blocks, stats_stream_kernel<false, false, true>, kWave * kStreamWaves, 0);
        if (e != hipSuccess) return e;
        v = (int64_t)cus * (blocks > 0 ? blocks : 1) * kStreamWaves;
        cached[with_mask][dev].store(v, std::memory_order_relaxed);
    }
    *out = v;
    return hipSuccess;
}

}  // namespace

// Tokens per streaming wave (a multiple of kPiece, at least kMinRange) and
// the number of waves, for n tokens and at most `waves` waves.
void split_tokens(int64_t n, int64_t waves, int64_t* range, int64_t* nwaves) {
    if (waves < 1) waves = 1;
    int64_t r = (n + waves - 1) / waves;
    r = (r + kPiece - 1) / kPiece * kPiece;
    *range = r < kMinRange ? kMinRange : r;
    *nwaves = n > 0 ? (n + *range - 1) / *range : 1;
}

bool make_stats_plan(int64_t n, int64_t s, StatsPlan* p) {
    if (n < 0 || s < 0 || s > INT32_MAX - 1 || n > INT32_MAX) return false;
    p->n = n;
    p->s = s;
    // the workspace holds the most waves any device gets
    split_tokens(n, kMaxStreamWaves, &p->range, &p->nwaves);
    // slot floor(c_j / SC) + j + k <= floor((n - 1) / SC) + s - 1; a slot
    // index keeps its top bit free (the stage marks the kind there)
    p->nslots = n / kSubChunk + s + 1;
    if (p->nslots >= ((int64_t)1 << 31)) return false;
    p->nblk_fin = (p->nwaves + kFinBlock - 1) / kFinBlock;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    p->slot_off = take((size_t)p->nslots * sizeof(SubPartial));
    p->wpart_off = take((size_t)p->nwaves * sizeof(BatchAcc));
    p->cross_off = take((size_t)p->nwaves * sizeof(int32_t));
    p->blk_off = take((size_t)p->nblk_fin * sizeof(BatchAcc));
    p->ticket_off = take(sizeof(uint32_t));
    p->total_bytes = off;
    return true;
}

hipError_t launch_mismatch_stats(const StatsPlan& p, const float* lt, const float* lr,
                                 const uint8_t* mask, const int32_t* cu,
                                 const StatsParamsDev& prm, const TokenOutPtrs& tok,
                                 const SeqOutPtrs& seq, double* batch, void* workspace,
                                 hipStream_t st) {
    if (p.s <= 0) return hipSuccess;               // no sequence: nothing to write
    unsigned char* ws = (unsigned char*)workspace;
    SubPartial* slots = (SubPartial*)(ws + p.slot_off);
    BatchAcc* wpart = (BatchAcc*)(ws + p.wpart_off);
    int32_t* cross = (int32_t*)(ws + p.cross_off);
    BatchAcc* blk = (BatchAcc*)(ws + p.blk_off);
    uint32_t* ticket = (uint32_t*)(ws + p.ticket_off);
    TokOut to{tok.delta, tok.ratio, tok.k1, tok.k2, tok.k3, tok.tis_w, tok.clipped};
    SeqOut so{seq.n_valid, seq.n_clipped, seq.n_nan, seq.mean_delta, seq.mean_k1,
              seq.mean_k2, seq.mean_k3, seq.mean_tis_w, seq.reject, seq.reject_k3};
    const uint32_t n = (uint32_t)p.n, s = (uint32_t)p.s;
    // every streaming wave resident at once: as many waves as the device
    // holds, at most the plan's (which sized the workspace)
    int64_t waves_dev = 0;
    {
        const hipError_t e = stream_waves_per_device(mask != nullptr, &waves_dev);
        if (e != hipSuccess) return e;
    }
    int64_t range64 = 0, nw64 = 0;
    split_tokens(p.n, waves_dev < kMaxStreamWaves ? waves_dev : kMaxStreamWaves, &range64, &nw64);
    const uint32_t range = (uint32_t)range64, nw = (uint32_t)nw64;
    const uint64_t nslots = (uint64_t)p.nslots;
    const dim3 grid((nw + kStreamWaves - 1) / kStreamWaves);
    const dim3 bdim(kWave * kStreamWaves);
    const bool want_tok = to.delta || to.ratio || to.k1 || to.k2 || to.k3 || to.tis_w ||
                          to.clipped;
#define TIM_STATS_STREAM(KT, KM, KD)                                                            \
    hipLaunchKernelGGL((stats_stream_kernel<KT, KM, KD>), grid, bdim, 0, st, lt, lr, mask, cu, n,  \
                       s, range, nw, prm, to, so, slots, wpart, cross, ticket)
    // the mask is read four bytes per lane once the array has four
    const bool mdw = n >= 4;
    if (want_tok && mask && mdw) TIM_STATS_STREAM(true, true, true);
    else if (want_tok && mask) TIM_STATS_STREAM(true, true, false);
    else if (want_tok) TIM_STATS_STREAM(true, false, true);
    else if (mask && mdw) TIM_STATS_STREAM(false, true, true);
    else if (mask) TIM_STATS_STREAM(false, true, false);
    else TIM_STATS_STREAM(false, false, true);
#undef TIM_STATS_STREAM
    hipLaunchKernelGGL(stats_final_kernel, dim3((unsigned)((nw + kFinBlock - 1) / kFinBlock)),
                       dim3(kFinBlock), 0, st, cu,
                       n, s, prm, (const SubPartial*)slots, nslots, (const BatchAcc*)wpart,
                       (const int32_t*)cross, nw, so, blk, ticket, batch);
    return hipGetLastError();
}

}  // namespace tim
