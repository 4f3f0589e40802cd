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
// sequence's first token and every kSubChunk tokens after it; a sub-chunk's
// sums are folded in an order that depends only on token offsets inside it,
// so a sequence's results never depend on the rest of the batch.
//
//   1. plan_count / plan_scan / plan_write: integer prefix sum of the
//      sub-chunk counts; writes one (start, length) descriptor per
//      sub-chunk, in token order, and each sequence's first descriptor.
//   2. stats_stream: each wave takes a few (at most 16) consecutive
//      descriptors and streams their tokens in kPiece-token pieces: lane l
//      holds piece offsets l + 64 i (i = 0..3) of lt, lr and the mask in
//      registers, with kBufs pieces in flight, and folds one piece while the
//      next ones load.  A sub-chunk's lanes are folded across the wave with a
//      fixed LDS transpose + DPP tree.  Sub-chunk partials are staged in LDS
//      and written once when the wave is done.
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
    int64_t nvalid, nclip, nnan, nonempty, rejected, rejected_k3;
};

struct SubDesc {
    uint32_t start, len;
};

constexpr int kWave = 64;
constexpr int kFinBlock = 256;
constexpr int kScanBlock = 1024;
constexpr int kPiece = 256;                 // tokens per piece (4 per lane)
constexpr int kMaxSubPerWave = 16;          // descriptors per wave, at most
constexpr int kStreamWaves = 4;             // waves per block
constexpr uint32_t kBufs = 3;               // pieces in flight per wave (registers)
constexpr int kFoldVals = 4;                // fp64 sums folded across lanes per sub-chunk
constexpr int kWavesPerFinBlock = 4 * 256;  // streaming-wave partials per finalize block

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

// e^d - 1 for finite |d| > 1/32 (the rare branch; |d| <= 1/32 uses a Taylor
// polynomial for e^d - 1 - d).  Range reduction d = k ln2 + r with
// |r| <= ln2 / 2 (ln2 split in a high part exact in 32 bits and a low part),
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

// A piece held in registers: the lane's tokens at piece offsets lane + 64 i.
struct Regs {
    float x[4], y[4];
    uint32_t m[4];
};

template <bool kMask>
__device__ __forceinline__ void load_piece(Regs& r, const float* __restrict__ lt,
                                           const float* __restrict__ lr,
                                           const uint8_t* __restrict__ mask, uint32_t st,
                                           uint32_t cnt, int lane) {
    // uniform bases (scalar registers) and 32-bit lane offsets: one address
    // computation per entry, shared by the three streams
    const float* blt = lt + st;
    const float* blr = lr + st;
    const uint8_t* bm = kMask ? mask + st : mask;
    if (cnt == (uint32_t)kPiece) {                 // full piece: fixed lane offsets
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = (uint32_t)(i * kWave + lane);
            r.x[i] = *(const float*)((const char*)blt + (o << 2));
            r.y[i] = *(const float*)((const char*)blr + (o << 2));
            r.m[i] = kMask ? (uint32_t)bm[o] : 1u;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t o = (uint32_t)(i * kWave + lane);
            o = o < cnt ? o : cnt - 1;             // clamped: a valid copy, ignored later
            const uint32_t ob = o << 2;            // byte offset, 32-bit
            r.x[i] = *(const float*)((const char*)blt + ob);
            r.y[i] = *(const float*)((const char*)blr + ob);
            r.m[i] = kMask ? (uint32_t)bm[o] : 1u;
        }
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

// fma(a, b, c) as one v_fma_f64 with c in scalar registers (the compiler
// otherwise copies loop-invariant constants before a two-address fmac)
__device__ __forceinline__ double fma_s(double a, double b, double c) {
    double r;
    asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

// Fold the piece of a sub-chunk (start sub_start, length len) that begins at
// offset off0: lane l takes offsets off0 + l + 64 i, i ascending, so across a
// sub-chunk's pieces each lane folds its offsets in ascending order.  A token
// that does not count (outside the sub-chunk, masked out or non-finite) gets
// d = 0, which makes its d, d^2, k3 and |d| contributions exactly 0 with no
// further selects.  Counts are popcounts of the wave masks.  k2 is
// accumulated as d^2 and halved once (a power-of-two scale: exact).  For the
// truncated weight only the clipped tokens' e^d - 1 is summed (rare path);
// the unclipped sum is recovered as (sum d + sum k3) - that.
template <bool kTok, bool kMask>
__device__ __forceinline__ void fold_piece(Acc& A, const Regs& rg,
                                           uint32_t sub_start, uint32_t off0, uint32_t len,
                                           int lane, const StatsParamsDev& prm,
                                           const TokOut& tok) {
    static_assert(kPiece == 4 * kWave, "four piece entries per lane");
    const uint32_t lim = len - off0;                          // valid piece offsets < lim
#pragma unroll
    for (int i = 0; i < kPiece / kWave; ++i) {
        if ((uint32_t)(i * kWave) >= lim) break;              // uniform: rest of piece empty
        const uint32_t po = (uint32_t)(i * kWave + lane);      // offset in the piece
        const double draw = (double)rg.x[i] - (double)rg.y[i];
        // lane predicates as wave masks: each ballot is one compare, the
        // combinations are scalar, and inverse_ballot reads a lane's bit back
        uint64_t m_in = ~0ull;                                    // full row: all lanes in
        if ((uint32_t)((i + 1) * kWave) > lim) m_in = __builtin_amdgcn_ballot_w64(po < lim);
        const uint64_t m_scored = m_in & (kMask ? __builtin_amdgcn_ballot_w64(rg.m[i] != 0) : ~0ull);
        const uint64_t m_fin = m_scored & finite_mask(draw);
        const uint64_t m_clip = m_fin & __builtin_amdgcn_ballot_w64(draw > prm.log_c);
        A.nvalid += (uint32_t)__popcll(m_fin);
        A.nnan += (uint32_t)__popcll(m_scored & ~m_fin);
        A.nclip += (uint32_t)__popcll(m_clip);
        const double d = __builtin_amdgcn_inverse_ballot_w64(m_fin) ? draw : 0.0;
        // e^d - 1 - d for |d| <= 1/32: d^2 (1/2 + d/6 + d^2/24 + d^3/120),
        // truncation below 4e-9 relative
        double p = fma_s(d, 1.0 / 120.0, 1.0 / 24.0);
        p = fma_s(p, d, 1.0 / 6.0);
        p = fma_s(p, d, 0.5);
        double k3 = d * (d * p);
        const uint64_t m_big = __builtin_amdgcn_ballot_w64(!(fabs(d) <= 0.03125));
        if ((m_big | m_clip) != 0) {                                    // rare, uniform test
            if (__builtin_amdgcn_inverse_ballot_w64(m_big)) k3 = expm1_large(d) - d;
            if (__builtin_amdgcn_inverse_ballot_w64(m_clip)) A.sclip += d + k3;
        }
        A.sd += d;
        A.sd2 = fma(d, d, A.sd2);
        A.sk3 += k3;
        A.sabs += fabs(d);
        A.mx = max_abs(A.mx, d);
        if (kTok && po < lim) {
            // per-token outputs; a non-finite delta reports exp/expm1 as computed
            const bool scored = __builtin_amdgcn_inverse_ballot_w64(m_scored);
            const bool fin = __builtin_amdgcn_inverse_ballot_w64(m_fin);
            const bool clipped = __builtin_amdgcn_inverse_ballot_w64(m_clip);
            const uint32_t t = sub_start + off0 + po;
            const double dd = scored ? draw : 0.0;
            const double em1 = d + k3;
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
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
    q.sabs = 0.0;                                                  // per wave instead
    q.maxabs = 0.0;
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

// Descriptors per wave: enough waves to cover the chip several times over at
// any size (a wave's descriptors are folded one after another, its pieces
// streamed through one pipeline), at most kMaxSubPerWave: with many short
// sequences the longer per-wave stream hides the pipeline's start (at 2^28
// tokens in log-normal sequences, 16 per wave instead of 4 is ~7 % faster).
// Which wave folds a sub-chunk never changes its result.
inline uint32_t subs_per_wave(int64_t tmax) {
    constexpr int64_t kTargetWaves = 16384;
    int64_t k = (tmax + kTargetWaves - 1) / kTargetWaves;
    if (k < 1) k = 1;
    if (k > kMaxSubPerWave) k = kMaxSubPerWave;
    return (uint32_t)k;
}

template <bool kTok, bool kMask>
__global__ void __launch_bounds__(kWave * kStreamWaves)
stats_stream_kernel(const float* __restrict__ lt, const float* __restrict__ lr,
                    const uint8_t* __restrict__ mask, const SubDesc* __restrict__ desc,
                    const uint32_t* __restrict__ total, uint32_t tmax, StatsParamsDev prm,
                    TokOut tok, SubPartial* __restrict__ partial, uint32_t spw,
                    double2* __restrict__ wpart) {
    __shared__ __attribute__((aligned(16))) double scratch[kStreamWaves][kFoldVals * kWave];
    __shared__ SubPartial stage[kStreamWaves][kMaxSubPerWave];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    uint32_t T = __builtin_amdgcn_readfirstlane(*total);
    T = T < tmax ? T : tmax;
    const uint64_t wid = (uint64_t)blockIdx.x * kStreamWaves + wv;
    const uint64_t k0 = wid * spw;
    if (k0 >= T) {                                 // no sub-chunk for this wave
        if (lane == 0) wpart[wid] = make_double2(0.0, 0.0);
        return;
    }
    const uint32_t nsub = (uint32_t)(T - k0 < spw ? T - k0 : spw);

    // this wave's descriptors, one per lane, read into scalar registers
    const SubDesc my = lane < (int)nsub ? desc[k0 + lane] : SubDesc{0u, 0u};
    auto d_start = [&](uint32_t k) { return (uint32_t)__builtin_amdgcn_readlane((int)my.start, (int)k); };
    auto d_len = [&](uint32_t k) { return (uint32_t)__builtin_amdgcn_readlane((int)my.len, (int)k); };

    uint32_t npieces = 0;
    for (uint32_t k = 0; k < nsub; ++k) npieces += (d_len(k) + kPiece - 1) / kPiece;

    // issue iterator: (sub-chunk ik, piece ip)
    uint32_t ik = 0, ip = 0, is0 = d_start(0), il = d_len(0);
    // Every call issues the same loads, on every path: past the last piece it
    // reloads the first piece of the wave (never folded again).  The
    // compiler's load counting then sees a fixed number of loads between a
    // buffer's refill and its use, and waits for exactly that piece.
    const uint32_t s_first = d_start(0);
    const uint32_t c_first = d_len(0) < (uint32_t)kPiece ? d_len(0) : (uint32_t)kPiece;
    auto issue = [&](Regs& r) {
        if (ik < nsub) {
            const uint32_t st = is0 + ip * kPiece;
            const uint32_t en = st + kPiece < is0 + il ? st + kPiece : is0 + il;
            load_piece<kMask>(r, lt, lr, mask, st, en - st, lane);
            if (++ip * kPiece >= il) {
                ip = 0;
                if (++ik < nsub) { is0 = d_start(ik); il = d_len(ik); }
            }
        } else {
            load_piece<kMask>(r, lt, lr, mask, s_first, c_first, lane);
        }
    };

    Acc A;
    A.zero();
    A.sabs = 0.0;
    A.mx = 0.0;
    uint32_t fk = 0, fp = 0, fs = d_start(0), fl = d_len(0);
    // fold piece c from r (if it exists), then refill r with piece c + kBufs
    auto step = [&](Regs& r, uint32_t c) {
        if (c < npieces) {
            fold_piece<kTok, kMask>(A, r, fs, fp * kPiece, fl, lane, prm, tok);
            if (++fp * kPiece >= fl) {
                const SubPartial q = finish(A, prm.clip_c, lane, scratch[wv]);
                if (lane == 0) stage[wv][fk] = q;
                A.zero();
                fp = 0;
                if (++fk < nsub) { fs = d_start(fk); fl = d_len(fk); }
            }
        }
        issue(r);
    };
    Regs b0, b1, b2;
    issue(b0);
    issue(b1);
    issue(b2);
    for (uint32_t c = 0; c < npieces; c += kBufs) {
        step(b0, c);
        step(b1, c + 1);
        step(b2, c + 2);
    }
    // stage[wv] is this wave's own: lane 0's LDS writes precede these reads in order
    const int e = lane >> 2, q4 = lane & 3;
    if (e < (int)nsub) ((uint4*)&partial[k0 + e])[q4] = ((const uint4*)&stage[wv][e])[q4];
    const double wsabs = bfly_sum(A.sabs), wmx = bfly_max(A.mx);
    if (lane == 0) wpart[wid] = make_double2(wsabs, wmx);
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

__global__ void __launch_bounds__(kFinBlock)
seq_finalize_kernel(const int32_t* __restrict__ cu, int64_t n, int64_t s, int64_t tmax,
                    StatsParamsDev prm,
                    const uint32_t* __restrict__ seq_off, const SubPartial* __restrict__ partial,
                    const double2* __restrict__ wpart, int64_t nw,
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
        const bool rej_k3 = nvalid > 0 && mk3 > prm.seq_k3_hi;   // K3 form
        if (so.n_valid) so.n_valid[j] = (int32_t)nvalid;
        if (so.n_clipped) so.n_clipped[j] = (int32_t)nclip;
        if (so.n_nan) so.n_nan[j] = (int32_t)nnan;
        if (so.mean_delta) so.mean_delta[j] = md;
        if (so.mean_k1) so.mean_k1[j] = mk1;
        if (so.mean_k2) so.mean_k2[j] = mk2;
        if (so.mean_k3) so.mean_k3[j] = mk3;
        if (so.mean_tis_w) so.mean_tis_w[j] = mw;
        if (so.reject) so.reject[j] = rej ? 1 : 0;
        if (so.reject_k3) so.reject_k3[j] = rej_k3 ? 1 : 0;
        c.sd = sd; c.sk2 = sk2; c.sk3 = sk3; c.sw = sw; c.sabs = sabs; c.maxabs = mx;
        c.nvalid = nvalid; c.nclip = nclip; c.nnan = nnan;
        if (nvalid > 0) {
            c.md = md; c.mk1 = mk1; c.mk2 = mk2; c.mk3 = mk3;
            c.nonempty = 1;
            c.rejected = rej ? 1 : 0;
            c.rejected_k3 = rej_k3 ? 1 : 0;
        }
    }
    // this block's slice of the streaming waves' sum and maximum of |delta|
#pragma unroll
    for (int r = 0; r < kWavesPerFinBlock / kFinBlock; ++r) {
        const int64_t i = (int64_t)blockIdx.x * kWavesPerFinBlock + r * kFinBlock + threadIdx.x;
        if (i < nw) {
            const double2 q = wpart[i];
            c.sabs += q.x;
            c.maxabs = fmax(c.maxabs, q.y);
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
        out[19] = dv((double)a.rejected_k3, ns);  // TIM_B_REJECT_K3_FRAC
        out[20] = (double)a.rejected_k3;
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
    p->spw = subs_per_wave(p->tmax);
    p->nwaves = ((p->tmax + p->spw - 1) / p->spw + kStreamWaves - 1) / kStreamWaves * kStreamWaves;
    {
        const int64_t nbw = (p->nwaves + kWavesPerFinBlock - 1) / kWavesPerFinBlock;
        p->nblk_fin = p->nblk_seq > nbw ? p->nblk_seq : nbw;
    }
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
    p->blk_off = take((size_t)(p->nblk_fin > 0 ? p->nblk_fin : 1) * sizeof(BatchAcc));
    p->wpart_off = take((size_t)p->nwaves * sizeof(double2));
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
    double2* wpart = (double2*)(ws + p.wpart_off);
    const bool streamed = p.s > 0 && p.n > 0;
    TokOut to{tok.delta, tok.ratio, tok.k1, tok.k2, tok.k3, tok.tis_w, tok.clipped};
    SeqOut so{seq.n_valid, seq.n_clipped, seq.n_nan, seq.mean_delta, seq.mean_k1,
              seq.mean_k2, seq.mean_k3, seq.mean_tis_w, seq.reject, seq.reject_k3};
    if (p.s > 0) {
        hipLaunchKernelGGL(plan_count_kernel, dim3((unsigned)p.nblk_scan), dim3(kScanBlock), 0, st,
                           cu, p.n, p.s, bsum);
        hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kScanBlock), 0, st, bsum, p.nblk_scan,
                           boff, total);
        hipLaunchKernelGGL(plan_write_kernel, dim3((unsigned)p.nblk_scan), dim3(kScanBlock), 0, st,
                           cu, p.n, p.s, p.tmax, boff, seq_off, desc);
        if (p.n > 0) {
            const uint32_t spw = p.spw;
            const dim3 grid((unsigned)(p.nwaves / kStreamWaves));
            const dim3 bdim(kWave * kStreamWaves);
            const bool want_tok = to.delta || to.ratio || to.k1 || to.k2 || to.k3 || to.tis_w ||
                                  to.clipped;
            if (want_tok && mask)
                hipLaunchKernelGGL((stats_stream_kernel<true, true>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial, spw, wpart);
            else if (want_tok)
                hipLaunchKernelGGL((stats_stream_kernel<true, false>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial, spw, wpart);
            else if (mask)
                hipLaunchKernelGGL((stats_stream_kernel<false, true>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial, spw, wpart);
            else
                hipLaunchKernelGGL((stats_stream_kernel<false, false>), grid, bdim, 0, st, lt, lr,
                                   mask, desc, total, (uint32_t)p.tmax, prm, to, partial, spw, wpart);
        }
        hipLaunchKernelGGL(seq_finalize_kernel, dim3((unsigned)p.nblk_fin), dim3(kFinBlock), 0, st,
                           cu, p.n, p.s, p.tmax, prm, seq_off, partial, (const double2*)wpart,
                           streamed ? p.nwaves : (int64_t)0, so, blk);
    }
    if (batch)
        hipLaunchKernelGGL(batch_finalize_kernel, dim3(1), dim3(kFinBlock), 0, st, blk,
                           p.s > 0 ? p.nblk_fin : (int64_t)0, batch);
    return hipGetLastError();
}

}  // namespace tim
