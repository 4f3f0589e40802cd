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
//      in token order and folds every sub-chunk that starts in its range.
//      Tokens stream as 64-token rows (lane l: token 64 R + l) through a
//      ring of kRing rows held in registers, loaded with non-temporal
//      buffer loads kRing rows ahead; a row inside one sub-chunk is folded
//      as is, a row that holds sub-chunk boundaries is folded lane range by
//      lane range.  Because every boundary of a sequence's sub-chunks sits
//      at the same lane, each lane adds the same tokens in the same order
//      as it would with rows taken from the sub-chunk's start; a finished
//      sub-chunk is folded across the wave with a fixed LDS transpose + DPP
//      tree that undoes that rotation.  Every sub-chunk's sums go to slot
//      floor(c_j / kSubChunk) + j + k (strictly increasing in (j, k), so no
//      prefix sum is needed to place them).
//   2. stats_final: one thread per sequence adds the sequence's slots in
//      ascending order and writes its outputs; the sums and maxima of |d|
//      the streaming waves carried are added in too.  Each block folds its
//      threads with a fixed tree, and the last block to finish folds the
//      block partials with a fixed tree into the batch aggregates.

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
constexpr int64_t kMaxFinBlocks = 512;      // finalize blocks, at most
constexpr int kRangeQuantum = 256;          // a streaming wave's range is a multiple of this
constexpr int kStreamWaves = 4;             // waves per block (each works on its own)
constexpr int kRing = 8;                    // rows in flight per wave (register ring)
constexpr int kFoldVals = 4;                // fp64 sums folded across lanes per sub-chunk
constexpr int64_t kMaxStreamWaves = 8192;   // streaming waves, at most (32 per CU)
constexpr int64_t kMinRange = 512;          // tokens per streaming wave, at least
constexpr uint32_t kSC = (uint32_t)kSubChunk;

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
// A double formed in scalar registers where it is used: two s_mov_b32 of
// its bit pattern in a volatile asm, which the compiler cannot hoist out of
// the rare branch.  As immediates, the compiler kept all of expm1_large's
// constants in vector registers across the whole row loop, which cost the
// kernel a wave per SIMD.
template <uint32_t kLo, uint32_t kHi>
__device__ __forceinline__ double sconst() {
    uint32_t lo, hi;
    asm volatile("s_mov_b32 %0, %2\n\ts_mov_b32 %1, %3" : "=s"(lo), "=s"(hi) : "i"(kLo), "i"(kHi));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double expm1_large(double d) {
    if (d > sconst<0xFEFA39EFu, 0x40862E42u>()) return INFINITY;     // 709.782712893384
    if (d < sconst<0x00000000u, 0xC0874800u>()) return -1.0;         // -745
    // log2(e), and ln2 split into a high part whose product with k is exact
    // (0x3FE62E42FEE00000) and a low part
    const double k = rint(d * sconst<0x652B82FEu, 0x3FF71547u>());
    const double r = fma(-k, sconst<0x35793C76u, 0x3DEA39EFu>(),
                         fma(-k, sconst<0xFEE00000u, 0x3FE62E42u>(), d));
    // e^r - 1 = r + r^2/2! + ... + r^12/12!; the coefficients 1/12! .. 1/3!
    // are the doubles nearest to them (the bit patterns of 1.0 / k!)
    double q = sconst<0xEFF8D898u, 0x3E21EED8u>();                    // 1/12!
    q = fma(q, r, sconst<0x67F544E4u, 0x3E5AE645u>());                // 1/11!
    q = fma(q, r, sconst<0xB7789F5Cu, 0x3E927E4Fu>());                // 1/10!
    q = fma(q, r, sconst<0xA556C734u, 0x3EC71DE3u>());                // 1/9!
    q = fma(q, r, sconst<0x1A01A01Au, 0x3EFA01A0u>());                // 1/8!
    q = fma(q, r, sconst<0x1A01A01Au, 0x3F2A01A0u>());                // 1/7!
    q = fma(q, r, sconst<0x16C16C17u, 0x3F56C16Cu>());                // 1/6!
    q = fma(q, r, sconst<0x11111111u, 0x3F811111u>());                // 1/5!
    q = fma(q, r, sconst<0x55555555u, 0x3FA55555u>());                // 1/4!
    q = fma(q, r, sconst<0x55555555u, 0x3FC55555u>());                // 1/3!
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
    // Zeroed in place (tied asm), so that the sums keep their registers
    // across every path of the row loop (see acc_row).
    __device__ void zero() {
        asm volatile("v_mov_b64 %0, 0\n\tv_mov_b64 %1, 0\n\tv_mov_b64 %2, 0\n\tv_mov_b64 %3, 0"
                     : "+v"(sd), "+v"(sd2), "+v"(sk3), "+v"(sclip));
        nvalid = nclip = nnan = 0;
    }
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
constexpr int kRsrcWord3 = 0x00020000;   // buffer descriptor word 3: 32-bit data, no swizzle

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wave mask of the lanes whose x is finite (v_cmp_class with the six finite
// classes: -normal, -denormal, -0, +0, +denormal, +normal), straight into
// scalar registers.  Every lane of the wave is active where this is used.
__device__ __forceinline__ uint64_t finite_mask(double x) {
    uint64_t m;
    asm("v_cmp_class_f64_e64 %0, %1, %2" : "=s"(m) : "v"(x), "s"(0x1F8));
    return m;
}

// fma(a, b, c) as one v_fma_f64 with c in vector registers, held across
// the loop (the compiler otherwise copies loop-invariant constants before a
// two-address fmac, and scalar registers are the scarcer kind here)
__device__ __forceinline__ double fma_s(double a, double b, double c) {
    double r;
    asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

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

// The row's additions to the sums, each accumulator updated in place: sd +=
// d, sd2 = fma(d, d, sd2), sk3 = fma(d, dp, sk3), sabs += |d|, mx = max(mx,
// |d|) (both finite: no canonicalisation needed).  Written as one asm block
// with the accumulators tied, so that every path through a row leaves them
// in the same registers (with separate destinations the register allocator
// moved all six between two register sets at every join of the row paths).
// The trailing wait states separate a v_max_f64 from the next read of its
// result, as the compiler's hazard recognizer does for that instruction.
__device__ __forceinline__ void acc_row(Acc& A, double d, double dp) {
    asm volatile(
        "v_add_f64 %0, %0, %5\n\t"
        "v_fma_f64 %1, %5, %5, %1\n\t"
        "v_fma_f64 %2, %5, %6, %2\n\t"
        "v_add_f64 %3, %3, |%5|\n\t"
        "v_max_f64 %4, %4, |%5|\n\t"
        "s_nop 1"
        : "+v"(A.sd), "+v"(A.sd2), "+v"(A.sk3), "+v"(A.sabs), "+v"(A.mx)
        : "v"(d), "v"(dp));
}
// acc += x in place (the rare branch's additions)
__device__ __forceinline__ void acc_inc(double& acc, double x) {
    asm volatile("v_add_f64 %0, %0, %1" : "+v"(acc) : "v"(x));
}

// One row of the stream in a lane's registers: token 64 R + lane of the
// wave's rows (lt, lr and the mask byte, zero-extended).
struct Row {
    float x, y;
    uint32_t m;
};

// Cache policy of the stream's loads: non-temporal (every token is read
// once, so its lines need not stay in the caches).
constexpr int kStreamCpol = 2;

// Row loads: one dword of lt and lr and one byte of the mask per lane, at
// token offset `off` from the descriptors' bases.  The offset is in the
// vector operand, which the descriptor's range check covers: a token past
// the extent reads as 0 and no memory is touched for it.
template <bool kMask>
__device__ __forceinline__ void load_row(Row& r, __amdgpu_buffer_rsrc_t rlt,
                                         __amdgpu_buffer_rsrc_t rlr, __amdgpu_buffer_rsrc_t rm,
                                         uint32_t off) {
    r.x = __builtin_bit_cast(float,
                             __builtin_amdgcn_raw_buffer_load_b32(rlt, off * 4u, 0, kStreamCpol));
    r.y = __builtin_bit_cast(float,
                             __builtin_amdgcn_raw_buffer_load_b32(rlr, off * 4u, 0, kStreamCpol));
    if constexpr (kMask) r.m = __builtin_amdgcn_raw_buffer_load_b8(rm, off, 0, kStreamCpol);
    else r.m = 1u;
}

// Wave mask of lanes a .. b - 1 (0 <= a < b <= 64).
__device__ __forceinline__ uint64_t lane_range(uint32_t a, uint32_t b) {
    const uint64_t hi = b >= 64u ? ~0ull : ((1ull << b) - 1ull);
    return hi & (~0ull << a);
}

// Fold one row into a sub-chunk's sums: the lanes of `sel` hold tokens of
// the sub-chunk, lane l adds its token after every
// earlier token of the sub-chunk it holds.  A token that does not count
// (outside sel, masked out or non-finite) gets d = 0, which makes its d,
// d^2, k3 and |d| contributions exactly 0 with no further selects.  Counts
// are popcounts of wave masks; the rare ones (non-finite, clipped) are
// counted in the rare branch, which any such token sends the wave into.  k2
// is accumulated as d^2 and halved once (a power-of-two scale: exact).  For
// the truncated weight only the clipped tokens' e^d - 1 is summed (rare
// path); the unclipped sum is recovered as (sum d + sum k3) - that.
// kClipRare: log C >= 1/32, so a clipped token (d > log C) is among the
// |d| > 1/32 tokens of the rare branch and needs no test of its own.
template <bool kTok, bool kMask, bool kClipRare>
__device__ __forceinline__ void fold_row(Acc& A, const Row& rw, uint64_t sel, uint32_t t0, int lane,
                                         const StatsParamsDev& prm, const TokOut& tok,
                                         const SeriesC& sc3) {
    static_assert(!(kTok && kClipRare), "per-token outputs test the clip on every token");
    const double draw = (double)rw.x - (double)rw.y;
    // lane predicates as wave masks: each ballot is one compare, the
    // combinations are scalar, and inverse_ballot reads a lane's bit back
    uint64_t sc = kMask ? __builtin_amdgcn_ballot_w64((uint8_t)rw.m != 0) : ~0ull;
    sc &= sel;
    const uint64_t m_fin = sc & finite_mask(draw);
    A.nvalid += (uint32_t)__popcll(m_fin);
    uint64_t rare = sc & ~m_fin;                       // non-finite: counted in the branch
    uint64_t m_clip = 0;
    if constexpr (!kClipRare) {
        m_clip = m_fin & __builtin_amdgcn_ballot_w64(draw > sc3.log_c);
        rare |= m_clip;
    }
    const double d = __builtin_amdgcn_inverse_ballot_w64(m_fin) ? draw : 0.0;
    // e^d - 1 - d = d dp for |d| <= 1/32, dp = d (1/2 + d/6 + d^2/24 +
    // d^3/120), truncation below 4e-9 relative
    double p = fma_s(d, sc3.c5, sc3.c4);
    p = fma_s(p, d, sc3.c3);
    p = fma_s(p, d, 0.5);
    double dp = d * p;
    rare |= __builtin_amdgcn_ballot_w64(!(fabs(d) <= 0.03125));
    double k3x = 0.0;                                  // the token's k3, for the outputs
    if constexpr (kTok) k3x = d * dp;
    if (rare != 0) {                                   // uniform test, rarely taken
        A.nnan += (uint32_t)__popcll(sc & ~m_fin);
        const uint64_t clip =
            kClipRare ? m_fin & __builtin_amdgcn_ballot_w64(draw > sc3.log_c) : m_clip;
        A.nclip += (uint32_t)__popcll(clip);
        double k3 = d * dp;
        if (!(fabs(d) <= 0.03125)) {
            // the exact e^d - 1 - d, added here; the fused add below then
            // adds d * 0
            k3 = expm1_large(d) - d;
            acc_inc(A.sk3, k3);
            dp = 0.0;
        }
        if (__builtin_amdgcn_inverse_ballot_w64(clip)) acc_inc(A.sclip, d + k3);
        if constexpr (kTok) {
            m_clip = clip;
            k3x = k3;
        }
    }
    acc_row(A, d, dp);
    if constexpr (kTok) {
        if (__builtin_amdgcn_inverse_ballot_w64(sel)) {
            // per-token outputs; a non-finite delta reports exp/expm1 as computed
            const bool scored = __builtin_amdgcn_inverse_ballot_w64(sc);
            const bool fin = __builtin_amdgcn_inverse_ballot_w64(m_fin);
            const bool clipped = __builtin_amdgcn_inverse_ballot_w64(m_clip);
            const uint32_t t = t0 + (uint32_t)lane;
            const double dd = scored ? draw : 0.0;
            const double em1 = d + k3x;
            const double r = 1.0 + em1;
            const double wgt = clipped ? prm.clip_c : (fin ? r : 0.0);
            const double rr = fin ? r : (scored ? exp(dd) : 1.0);
            const double kk3 = fin ? k3x : (scored ? expm1(dd) - dd : 0.0);
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
// depends on offsets inside the sub-chunk only.  Lane l holds the sums of
// the sub-chunk's offsets congruent to l - rot (mod 64), rot being the lane
// of its first token:
//   1. every lane stores its four values to the wave's scratch at that
//      offset class: v[value][(l - rot) mod 64];
//   2. lane j < 32 sums v[j / 8][8 (j % 8) .. 8 (j % 8) + 7] left to right;
//   3. the eight partials of a value (lanes 8 v .. 8 v + 7) are combined by
//      three DPP steps: neighbours (quad_perm 1,0,3,2), pairs (quad_perm
//      2,3,0,1), half-rows (row_half_mirror);
//   4. lane 8 v holds value v and is read into scalar registers.
// A wave's LDS operations complete in issue order, so the reads see the
// writes without a wait between them; the read block ends in lgkmcnt(0).
__device__ __forceinline__ SubPartial finish(const Acc& A, double clip_c, int lane, const double* scratch,
                                             uint32_t rot) {
    const uint32_t base = lds_addr(scratch);
    const uint32_t aw = base + 8u * (((uint32_t)lane - rot) & 63u);   // v[0][(lane - rot) mod 64]
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

// The 64 lanes' partials combined by a fixed xor butterfly (partner
// distance 1, 2, ..., 32), field by field; every lane ends with the same
// bits.
__device__ __forceinline__ void wave_reduce(BatchAcc& c) {
    c.sd = bfly_sum(c.sd); c.sk2 = bfly_sum(c.sk2); c.sk3 = bfly_sum(c.sk3);
    c.sw = bfly_sum(c.sw); c.sabs = bfly_sum(c.sabs); c.maxabs = bfly_max(c.maxabs);
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

// A block's partials in a fixed order: each wave's by the butterfly, then
// the waves' in ascending order.  The result is returned to every thread.
__device__ BatchAcc block_fold(BatchAcc c, BatchAcc* wbuf) {
    wave_reduce(c);
    if ((threadIdx.x & (kWave - 1)) == 0) wbuf[threadIdx.x / kWave] = c;
    __syncthreads();
    BatchAcc r = wbuf[0];
#pragma unroll
    for (int i = 1; i < kFinBlock / kWave; ++i) acc_add(r, wbuf[i]);
    __syncthreads();                                   // wbuf may be written again
    return r;
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

// A streaming wave's share of the batch sums that no sequence carries: the
// sum and maximum of |d| over the tokens it folded.
struct alignas(16) WavePart {
    double sabs, maxabs;
};

template <bool kTok, bool kMask, bool kClipRare>
__global__ void __launch_bounds__(kWave * kStreamWaves)
stats_stream_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                    const uint8_t* __restrict__ mask, const int32_t* __restrict__ cu,
                    uint32_t n, uint32_t s, uint32_t range, uint32_t nwaves, StatsParamsDev prm,
                    TokOut tok, SubPartial* __restrict__ slots, WavePart* __restrict__ wpart,
                    uint32_t* __restrict__ ticket) {
    __shared__ __attribute__((aligned(16))) double scratch[kStreamWaves][kFoldVals * kWave];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const uint32_t w = blockIdx.x * kStreamWaves + (uint32_t)wv;
    if (w >= nwaves) return;
    if (w == 0 && lane == 0) *ticket = 0u;         // the finalize kernel's counter
    const bool last = w == nwaves - 1;
    const uint32_t b0 = w * range;
    const uint32_t b1 = last ? n : b0 + range;     // the last wave also owns c_j == n
    const uint32_t ja = lower_bound_cu(cu, s, n, b0, lane);

    // ---- the walk over sequences and sub-chunks (wave-uniform state): the
    // current sub-chunk is tokens [ss, se) of sequence j, which ends at ej,
    // and its sums go to slot id.  A wave folds the sub-chunks that start in
    // its range [b0, b1).
    uint32_t ss = 0, se = 0, ej = 0, j = 0, id = 0;
    bool done = false;
    // Enter the first sequence at or after jj that starts in this wave's
    // range and has a token (the finalize kernel writes empty ones); c is
    // where sequence jj starts, the end of the one before (already read).
    // One entry of cu_seqlens is read per sequence.  The walk never goes
    // back: a sequence whose end lies before its start (a malformed
    // cu_seqlens) is taken as empty and the next one starts at c again.
    auto enter = [&](uint32_t jj, uint32_t c) __attribute__((always_inline)) {
        for (;;) {
            if (jj >= s) { done = true; return; }
            if (!last && c >= b1) { done = true; return; }
            const uint32_t e = cu_scalar(cu, jj + 1, n);
            if (e > c) {
                j = jj; ej = e; ss = c;
                se = c + kSC < e ? c + kSC : e;
                // slot of sub-chunk 0: floor(c / SC) + j (below floor(n / SC) +
                // s + 1 for any clamped c_j <= n and j < s)
                id = c / kSC + jj;
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
                    j = ja - 1; ej = e; ss = st;
                    se = st + kSC < e ? st + kSC : e;
                    id = c / kSC + (ja - 1) + k;
                    cont = true;
                }
            }
        }
        if (!cont) {
            const uint32_t c = ja < s ? cu_scalar(cu, ja, n) : n;
            enter(ja, c > b0 ? c : b0);
        }
    }

    // Rows: row R is tokens tb + 64 R .. tb + 64 R + 63, lane l holds token
    // tb + 64 R + l.  Every boundary of a sequence's sub-chunks (its start,
    // and the later sub-chunk starts, kSubChunk = 16 rows apart) sits at lane
    // c_j mod 64, so lane l holds the sub-chunk offsets o = l - ss (mod 64)
    // + 64 i in ascending order: the same tokens, in the same order, as lane
    // (l - ss) mod 64 of rows taken from ss.  The cross-lane fold (finish)
    // undoes the rotation, so a sub-chunk's sums depend on its tokens only.
    const uint32_t tb = done ? 0u : (ss & ~63u);
    // Descriptors based at tb: offsets are 32-bit (a wave's rows span less
    // than its range plus a sub-chunk and the ring past it); the extents end
    // at the arrays' ends.
    const uint64_t span = (uint64_t)(n - tb);
    const int ext4 = (int)(uint32_t)(span * 4 < 0xffffffffull ? span * 4 : 0xffffffffull);
    const __amdgpu_buffer_rsrc_t rlt =
        __builtin_amdgcn_make_buffer_rsrc((void*)(lt + tb), (short)0, ext4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rlr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(lr + tb), (short)0, ext4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rm =
        kMask ? __builtin_amdgcn_make_buffer_rsrc((void*)(mask + tb), (short)0, (int)(uint32_t)span,
                                                  kRsrcWord3)
              : rlt;

    Acc A;
    A.zero();
    A.sabs = 0.0;
    A.mx = 0.0;
    const SeriesC sc3 = series_c(prm.log_c);

    // The current sub-chunk is complete: fold it across the wave, write its
    // sums to its slot, go on to the next sub-chunk (the sequence's next
    // one, or the next sequence's first).
    auto end_sub = [&]() __attribute__((always_inline)) {
        SubPartial q = finish(A, prm.clip_c, lane, scratch[wv], ss & 63u);
        A.zero();
        if (lane == 0) slots[id] = q;
        if (se < ej) {
            // later sub-chunks of this sequence may start in later waves' ranges
            if (se >= b1) {
                done = true;
            } else {
                ss = se;
                se = ss + kSC < ej ? ss + kSC : ej;
                ++id;
            }
        } else {
            enter(j + 1, ej);
        }
    };

    // Fold a row: the lanes of each sub-chunk in it, in token order (one
    // pass for a row inside a sub-chunk).  Every row takes this one path:
    // with a separate path for rows inside a sub-chunk, the register
    // allocator moved all six sums between two register sets at every row.
    auto fold_rows_of = [&](const Row& rw, uint32_t R) __attribute__((always_inline)) {
        const uint32_t t0 = tb + 64u * R, t1 = t0 + 64u;
        while (!done && ss < t1) {
            const uint64_t sel = ss <= t0 && se >= t1
                                     ? ~0ull
                                     : lane_range(ss > t0 ? ss - t0 : 0u, se < t1 ? se - t0 : 64u);
            fold_row<kTok, kMask, kClipRare>(A, rw, sel, t0, lane, prm, tok, sc3);
            if (se > t1) break;                        // the sub-chunk goes on
            end_sub();
        }
    };

    if (!done) {
        Row ring[kRing];
#pragma unroll
        for (int i = 0; i < kRing; ++i)
            load_row<kMask>(ring[i], rlt, rlr, rm, (uint32_t)(64 * i + lane));
        uint32_t R = 0;                                // the next row to fold
        // Fold row R from its ring slot, then refill the slot with the row
        // kRing ahead.  Once the walk has ended the rows left in the block
        // fold nothing.
        auto step = [&](Row& slot) __attribute__((always_inline)) {
            fold_rows_of(slot, R);
            load_row<kMask>(slot, rlt, rlr, rm, 64u * (R + kRing) + (uint32_t)lane);
            ++R;
        };
        do {
#pragma unroll
            for (int i = 0; i < kRing; ++i) step(ring[i]);
        } while (!done);
    }
    const double wsabs = bfly_sum(A.sabs), wmx = bfly_max(A.mx);
    if (lane == 0) {
        WavePart p;
        p.sabs = wsabs;
        p.maxabs = wmx;
        wpart[w] = p;
    }
}

// Step 2: thread t finishes sequence t (its sub-chunks' sums, from their
// slots, added in ascending order; per-sequence outputs; its contribution
// to the batch) and adds streaming wave t's partial.  Each block folds its
// threads with a fixed tree; the last block to finish (a ticket counter,
// then a device-scope fence) folds the block partials with a fixed tree
// into the batch vector and resets the ticket for the next call.
__global__ void __launch_bounds__(kFinBlock)
stats_final_kernel(const int32_t* __restrict__ cu, uint32_t n, uint32_t s, StatsParamsDev prm,
                   const SubPartial* __restrict__ slots, uint64_t nslots,
                   const WavePart* __restrict__ wpart, uint32_t nwaves, SeqOut so,
                   BatchAcc* __restrict__ blk, uint32_t* __restrict__ ticket,
                   double* __restrict__ out) {
    __shared__ BatchAcc wbuf[kFinBlock / kWave];
    __shared__ uint32_t is_last;
    // thread t takes sequences t, t + T, t + 2T, ... (T threads in the
    // grid, a function of the call's sizes only) and the streaming waves
    // with the same indices
    const uint32_t T = gridDim.x * kFinBlock;
    BatchAcc c = acc_zero();
    for (uint32_t t = blockIdx.x * kFinBlock + threadIdx.x; t < s; t += T) {
        const uint32_t c0 = clamp_c(cu[t], n), e0 = clamp_c(cu[t + 1], n);
        SeqSums a = seq_zero();
        if (e0 > c0) {
            const uint32_t K = (e0 - c0 + kSC - 1) / kSC;
            const uint64_t base = (uint64_t)(c0 / kSC) + t;
            // the first four sub-chunks' loads issued together, added in order
            SubPartial q[4];
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k)
                if (k < K && base + k < nslots) q[k] = slots[base + k];
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k)
                if (k < K && base + k < nslots) seq_add(a, q[k]);
            for (uint32_t k = 4; k < K && base + k < nslots; ++k) seq_add(a, slots[base + k]);
        }
        seq_finish(t, a, prm, so, true, c);
    }
    for (uint32_t t = blockIdx.x * kFinBlock + threadIdx.x; t < nwaves; t += T) {
        const WavePart p = wpart[t];
        c.sabs += p.sabs;
        c.maxabs = fmax(c.maxabs, p.maxabs);
    }
    const BatchAcc bsum = block_fold(c, wbuf);
    if (!out) return;
    // the last block to get here folds every block's partial
    if (threadIdx.x == 0) {
        blk[blockIdx.x] = bsum;
        __threadfence();
        is_last = atomicAdd(ticket, 1u) == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    c = acc_zero();
    for (uint32_t i = threadIdx.x; i < gridDim.x; i += kFinBlock) acc_add(c, blk[i]);
    const BatchAcc a = block_fold(c, wbuf);
    if (threadIdx.x == 0) {
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

// Finalize blocks for s sequences and nw streaming waves: one thread each,
// at most kMaxFinBlocks blocks (their threads then take several; fewer
// blocks, fewer completion tickets on the one counter).
static int64_t fin_blocks(int64_t s, int64_t nw) {
    const int64_t nfin = s > nw ? s : nw;
    const int64_t b = (nfin + kFinBlock - 1) / kFinBlock;
    return b < 1 ? 1 : (b > kMaxFinBlocks ? kMaxFinBlocks : b);
}

// Tokens per streaming wave (a multiple of kRangeQuantum, at least kMinRange) and
// the number of waves, for n tokens and at most `waves` waves.
void split_tokens(int64_t n, int64_t waves, int64_t* range, int64_t* nwaves) {
    if (waves < 1) waves = 1;
    int64_t r = (n + waves - 1) / waves;
    r = (r + kRangeQuantum - 1) / kRangeQuantum * kRangeQuantum;
    *range = r < kMinRange ? kMinRange : r;
    *nwaves = n > 0 ? (n + *range - 1) / *range : 1;
}

bool make_stats_plan(int64_t n, int64_t s, StatsPlan* p) {
    if (n < 0 || s < 0 || s > INT32_MAX - 1 || n > INT32_MAX) return false;
    p->n = n;
    p->s = s;
    // the workspace holds the most waves any device gets
    split_tokens(n, kMaxStreamWaves, &p->range, &p->nwaves);
    // slot floor(c_j / SC) + j + k <= floor((n - 1) / SC) + s - 1
    p->nslots = n / kSubChunk + s + 1;
    if (p->nslots >= ((int64_t)1 << 31)) return false;
    // finalize threads: one per sequence and one per streaming wave
    p->nblk_fin = fin_blocks(s, p->nwaves);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    p->slot_off = take((size_t)p->nslots * sizeof(SubPartial));
    p->wpart_off = take((size_t)p->nwaves * sizeof(WavePart));
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
    WavePart* wpart = (WavePart*)(ws + p.wpart_off);
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
#define TIM_STATS_STREAM(KT, KM, KC)                                                            \
    hipLaunchKernelGGL((stats_stream_kernel<KT, KM, KC>), grid, bdim, 0, st, lt, lr, mask, cu, n,  \
                       s, range, nw, prm, to, slots, wpart, ticket)
    // log C >= 1/32: a clipped token is also a rare-branch token (|d| > 1/32)
    const bool clip_rare = prm.log_c >= 0.03125;
    if (want_tok && mask) TIM_STATS_STREAM(true, true, false);
    else if (want_tok) TIM_STATS_STREAM(true, false, false);
    else if (mask && clip_rare) TIM_STATS_STREAM(false, true, true);
    else if (mask) TIM_STATS_STREAM(false, true, false);
    else if (clip_rare) TIM_STATS_STREAM(false, false, true);
    else TIM_STATS_STREAM(false, false, false);
#undef TIM_STATS_STREAM
    hipLaunchKernelGGL(stats_final_kernel, dim3((unsigned)fin_blocks(s, nw)),
                       dim3(kFinBlock), 0, st, cu, n, s, prm, (const SubPartial*)slots, nslots,
                       (const WavePart*)wpart, nw, so, blk, ticket, batch);
    return hipGetLastError();
}

}  // namespace tim
