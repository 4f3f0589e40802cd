// lmhead.hip — fused LM-head contraction, online log-sum-exp and token
// gather for gfx950, plus the fixed-order merge of vocabulary-chunk partials.
//
// What is computed ("RL: Training Inference Mismatch", section "log p": the
// chain hidden -> LM head -> logits -> log-softmax -> gather):
//     z[t,v]  = sum_k h[t,k] W[v,k]
//     logp[t] = z[t,a_t] - log sum_v exp z[t,v]
// The logits live only in MFMA accumulators; they are never written.
// bf16 inputs run lmhead8w_kernel (16x16x32 MFMAs, eight waves), fp32
// inputs lmhead_partials_kernel (32x32x2 MFMAs, four waves); both follow
// the same tiles, chunks and merge order, described first for the latter.
//
// Batch invariance ("训推一致性与 determinism", section 1.2: a request's
// result must not depend on which other requests share its batch): every
// reduction order here is a function of (V, D, dtype) alone.
//   * K order: ascending D in 128-byte stages, one MFMA accumulator chain per
//     logit, no split-K.  A logit's bits do not depend on which MFMA column
//     (token slot) it occupies: every column runs the same instruction
//     sequence on its own data.
//   * Vocabulary: fixed chunks of kInvariantChunkTiles tiles of 256 rows.
//     Inside a chunk each lane folds its 64 rows of a tile into a running
//     (max, sum-exp) in a fixed order, tile after tile; at the end of the
//     chunk the two half-waves and then the two vocabulary waves are merged
//     in a fixed order.  The merge kernel folds the chunks in a fixed order
//     that depends on the number of chunks only.
//   * N only sets how many token tiles are launched; rows past N are clamped
//     loads whose results are discarded.
// This is the single-GPU form of the batch-invariant matmul/reduction the
// pages list ("训推一致性与 determinism", section 6 table; VeXact
// methodology), written for CDNA4 MFMA rather than copied from any design.

#include "mfma_pipe.h"

#include <math.h>

namespace tim {
namespace {

using namespace mfma;


// Online softmax state of a set of logits at the scale c2 = log2(e) / tau
// (tau the temperature): m = max z, s = sum 2^((z - m) c2), and, for the
// entropy, u = sum 2^a a with a = (z - m) c2 (a <= 0, so u <= 0).  Then
// ln sum exp(z / tau) = m / tau + ln s and the entropy of softmax(z / tau)
// is ln 2 (log2 s - u / s).

// (m, s): merge b into a.
__device__ __forceinline__ void lse_combine(float& m, float& s, float mb, float sb, float c2) {
    float mm = fmaxf(m, mb);
    if (mm == -INFINITY) { m = mm; s = 0.f; return; }
    float fa = (m == mm) ? 1.f : fast_exp2((m - mm) * c2);
    float fb = (mb == mm) ? 1.f : fast_exp2((mb - mm) * c2);
    s = fmaf(s, fa, sb * fb);      // written out: both helpers round alike
    m = mm;
}

// (m, s, u): merge b into a.  A state's exponent arguments all shift by
// d = (m_old - m_new) c2 when its reference moves up: s' = 2^d s and
// u' = 2^d (u + d s).  An empty state (s = 0) stays (0, 0).
__device__ __forceinline__ void lse_combine3(float& m, float& s, float& u, float mb, float sb,
                                             float ub, float c2) {
    const float mm = fmaxf(m, mb);
    if (mm == -INFINITY) { m = mm; s = 0.f; u = 0.f; return; }
    float fa = 1.f, fb = 1.f, ua = u, uo = ub;
    if (m != mm) {
        const float d = (m - mm) * c2;
        fa = fast_exp2(d);
        ua = s > 0.f ? fa * fmaf(d, s, u) : 0.f;
    }
    if (mb != mm) {
        const float d = (mb - mm) * c2;
        fb = fast_exp2(d);
        uo = sb > 0.f ? fb * fmaf(d, sb, ub) : 0.f;
    }
    s = fmaf(s, fa, sb * fb);
    u = ua + uo;
    m = mm;
}

// Exponent arguments are clamped here before 2^a a is formed, so that a
// masked logit (-inf) contributes 0 rather than 0 * inf.
constexpr float kArgFloor = -3.0e38f;

// XCD-aware order of workgroups.  The dispatcher hands workgroup b to XCD
// b % 8; renumber so that each XCD receives one contiguous range of logical
// tiles, and inside the range walk groups of kGroupChunks vocabulary chunks
// by all token tiles.  Workgroups resident on one XCD at a time then share
// W and h stages in that XCD's L2.  Changes only who computes a tile, never
// how: results are unaffected.
constexpr int kGroupChunks = 4;
__device__ __forceinline__ void tile_of_block(int64_t b, int64_t G, int64_t nchunks,
                                              int64_t nttiles, int64_t& chunk, int64_t& ttile) {
    const int64_t per = G >> 3, rem = G & 7, x = b & 7, i = b >> 3;
    const int64_t L = x * per + (x < rem ? x : rem) + i;
    const int64_t span = (int64_t)kGroupChunks * nttiles;
    const int64_t group = L / span;
    const int64_t first = group * kGroupChunks;
    const int64_t gm = nchunks - first < kGroupChunks ? nchunks - first : kGroupChunks;
    const int64_t within = L - group * span;
    chunk = first + within % gm;
    ttile = within / gm;
}

// fp32 inputs.  kEnt: also carry u (entropy).  c2 = log2(e) / tau.
//
// kMode selects what becomes of a tile of fp32 products (F32Gemm in
// tim_internal.h): the forward's fold (kF32Fold), or, for the backward of
// the fp32 head, with W as the A rows (v) and h as the B rows (n):
//   kF32Dz        the logits, formed by the very MFMA sequence of the
//                 forward, turned into dz[t][v] = g_t ([v == a_t] - p_t[v])
//                 (fp32, zero outside V x N up to the padded sizes), written
//                 as dz [Np][Vp] and/or dz^T [Vp][Np];
//   kF32Store     C[m][n] = sum_k A[m][k] B[n][k] stored (fp32);
//   kF32StoreAcc  the same, the chain continuing from the stored C.
// A lane holds rows 8 q + 4 lhalf + i (i = 0..3) of column lrow of each
// 32 x 32 block (acc register 4 q + i).
template <bool kEnt, int kMode = kF32Fold>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
lmhead_partials_kernel(const unsigned char* __restrict__ h, int64_t ldh_b,
                       const unsigned char* __restrict__ w, int64_t ldw_b,
                       const int32_t* __restrict__ ids, int64_t n, int64_t v,
                       int nk, int chunk_tiles, int64_t nvtiles, int64_t nchunks,
                       int64_t nttiles, float c2, float2* __restrict__ part,
                       float* __restrict__ upart, float* __restrict__ zsel,
                       int32_t* __restrict__ n_bad_ids, F32Epi ep) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wv = wave & 1;        // vocabulary half of the tile (128 rows)
    const int wt = wave >> 1;       // token half of the tile (128 tokens)
    const int lrow = lane & 31;
    const int lhalf = lane >> 5;

    if (blockIdx.x == 0 && tid == 0 && n_bad_ids) *n_bad_ids = 0;

    int64_t chunk, ttile;
    tile_of_block(blockIdx.x, gridDim.x, nchunks, nttiles, chunk, ttile);
    const int64_t t0 = ttile * kTileT;
    // one vocabulary tile per chunk (chunk_tiles == 1, checked on the host):
    // with several, the compiler copied the look-ahead fragments at the end
    // of a tile's K loop before their reads had been waited for, and the
    // next tile started from those copies
    const int64_t vt_first = chunk * chunk_tiles;
    constexpr int ntiles_here = 1;
    (void)nvtiles;

    // the 4 tokens of this lane (one per 32-column block), their target ids
    int32_t my_id[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        int64_t t = t0 + wt * 128 + bj * 32 + lrow;
        if constexpr (kMode == kF32Fold || kMode == kF32Dz) my_id[bj] = t < n ? ids[t] : -1;
        else my_id[bj] = -1;
    }

    f32x16 acc[4][4];
    float m_run[4], s_run[4], u_run[4];
    float zsel_reg[4] = {0.f, 0.f, 0.f, 0.f};   // selected logit, if owned
    bool have_zsel = false;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) { m_run[bj] = -INFINITY; s_run[bj] = 0.f; u_run[bj] = 0.f; }

    // Copy assignment: wave `wave` fills 8-row blocks 8 wave .. 8 wave + 7 of
    // both operands; lane i writes physical chunk i % 8 of row 8 blk + i / 8,
    // i.e. logical chunk (i % 8) ^ ((row >> 1) & 7).  Addresses are a buffer
    // descriptor per operand tile (base, byte extent), a fixed 32-bit per-lane
    // row offset and the stage's K offset.  Rows past N or V are redirected to
    // the last valid row; their results are discarded or masked.  Every
    // access then lies inside the tensors, and inside the descriptor's extent.
    uint32_t hoff[8], wrow_off[8], wtail_off[8];
    int drow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        drow[j] = (wave * 8 + j) * 8 + (lane >> 3);
        const uint32_t cb = (uint32_t)(((lane & 7) ^ ((drow[j] >> 1) & 7)) * 16);
        int64_t t = t0 + drow[j];
        if (t > n - 1) t = n - 1;
        hoff[j] = (uint32_t)((t - t0) * ldh_b) + cb;
        wrow_off[j] = (uint32_t)(drow[j] * ldw_b) + cb;
        wtail_off[j] = cb;             // + (v - 1 - vbase) * ldw_b, set per tile
    }
    const unsigned char* hbase = h + t0 * ldh_b;
    const int64_t hrows = (n - t0) < kTileT ? (n - t0) : kTileT;
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)hbase, (short)0, (int)((hrows - 1) * ldh_b + (int64_t)nk * kStageBytes), kRsrcWord3);
    uint32_t woff[8];
    const unsigned char* wbase = w;
    __amdgpu_buffer_rsrc_t wrs = hrs;
    auto set_wtile = [&](int vt_l) {
        const int64_t vbase = (vt_first + vt_l) * kTileV;
        wbase = w + vbase * ldw_b;
        const int64_t wrows = (v - vbase) < kTileV ? (v - vbase) : kTileV;
        wrs = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0,
                                                (int)((wrows - 1) * ldw_b + (int64_t)nk * kStageBytes), kRsrcWord3);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            woff[j] = vbase + drow[j] < v ? wrow_off[j]
                                          : (uint32_t)((v - 1 - vbase) * ldw_b) + wtail_off[j];
    };

    // per-lane LDS byte offset of k-step ks inside an operand tile: row lrow
    // of each 32-row block (the swizzle does not depend on the block), logical
    // chunk lhalf*4 + ks
    const uint32_t lds_base = lds_addr(lds);
    uint32_t kofs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kofs[ks] = (uint32_t)swz(lrow, lhalf * 4 + ks);
    }

    // Copy iterators: W of stage st + 1 and h of stage st + 2 are copied
    // while stage st computes.  Past the last stage both wrap to K offset 0
    // (of the last W tile): the extra copies read valid rows into positions
    // that are never read again, and every stage issues the same copies.
    int w_kb = 0, h_kb = 0;
    set_wtile(0);
    auto copy_w = [&](int part, int pos) {
        unsigned char* base = lds + pos * kOperandBytes;
        const uint32_t koff = (uint32_t)(w_kb * kStageBytes);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = part * 4 + jj;
            dma16_buf(wrs, base + (wave * 8 + j) * 1024, woff[j], koff);
        }
    };
    auto copy_h = [&](int part, int pos) {
        unsigned char* base = lds + pos * kOperandBytes;
        const uint32_t koff = (uint32_t)(h_kb * kStageBytes);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = part * 4 + jj;
            dma16_buf(hrs, base + (wave * 8 + j) * 1024, hoff[j], koff);
        }
    };
    auto advance_w = [&]() {
        if (++w_kb == nk) w_kb = 0;
    };
    auto advance_h = [&]() {
        if (++h_kb == nk) h_kb = 0;
    };
    auto next_pos = [](int p) { return p + 2 >= kPos ? p + 2 - kPos : p + 2; };
    // fragment k-step ks: A rows wv*128 + bi*32 + lrow from the W tile at
    // ring position pw, B rows wt*128 + bj*32 + lrow from the h tile at ph
    // (block bi / bj is an immediate 4 KiB step)
    auto issue_frags = [&](u32x4 (&f)[8], int pw, int ph, int ks) {
        lds_issue_8x16(f, lds_base + (uint32_t)(pw * kOperandBytes) + kofs[ks] + (uint32_t)(wv * 128 * kStageBytes),
                       lds_base + (uint32_t)(ph * kOperandBytes) + kofs[ks] + (uint32_t)(wt * 128 * kStageBytes));
    };
    auto mfma_step = [&](const u32x4 (&f)[8]) {
        // 32 fp32 of K per stage: lane half g supplies K = 16 g + 4 ks + e
        // to MFMA (ks, e); each 32x32x2 instruction consumes one K of each
        // half.  Whole vectors are cast before indexing: casting single
        // elements of the asm outputs made this compiler pass element 0
        // for every e.
        f32x4 ff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ff[i] = __builtin_bit_cast(f32x4, f[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        ff[bi][e], ff[4 + bj][e], acc[bi][bj], 0, 0, 0);
    };

    // Pipeline.  The ring holds operand tiles at positions (2 stage + op) % 5
    // (op 0: h, op 1: W).  While stage st computes, its two tiles and the h
    // tile of stage st + 1 are resident or landing, and the two free
    // positions (those of stage st - 1) take the W tile of stage st + 1
    // (copied during k-steps 0 and 1) and the h tile of stage st + 2 (k-steps
    // 2 and 3): four copies per k-step, one after every four MFMAs.  Fragment
    // reads run one k-step ahead of the MFMAs (fa, fb alternate).  Before the
    // barrier that ends stage st every wave waits for its copies of stage
    // st + 1 and for its last reads of stage st.  sched_barrier(0) keeps the
    // compiler from moving MFMAs across those waits and the reads that feed
    // the next k-step.
    int rd_h = 0, rd_w = 1;                            // positions of stage st
    int cp_w = 3, cp_h = 4;                            // W of st + 1, h of st + 2
    copy_h(0, 0); copy_h(1, 0); advance_h();           // h, stage 0
    copy_w(0, 1); copy_w(1, 1); advance_w();           // W, stage 0
    copy_h(0, 2); copy_h(1, 2); advance_h();           // h, stage 1
    wait_vmcnt<kDmaPerStage / 2>();                    // stage 0 (own copies)
    __syncthreads();                                   // ... everyone's
    u32x4 fa[8], fb[8];
    issue_frags(fa, rd_w, rd_h, 0);

    int st = 0;
    // row of A (vocabulary for the head) of acc register 4 q + i of block bi:
    // arow0 + bi 32 + q 8 + i
    const int64_t arow0 = vt_first * kTileV + wv * 128 + lhalf * 4;
    {
        constexpr int vt_local = 0;
        if constexpr (kMode == kF32StoreAcc) {
            // one base pointer per column, 32-bit row offsets (a tile spans
            // 256 rows of C)
            const uint32_t ldc = (uint32_t)ep.ldc;
            const int64_t mlim = v - arow0;                  // rows arow0 + mrel < v
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t cn = t0 + wt * 128 + bj * 32 + lrow;
                const bool cv = cn < n;
                const float* cb = ep.c + arow0 * ep.ldc + (cv ? cn : 0);
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int mrel = bi * 32 + (r >> 2) * 8 + (r & 3);
                        acc[bi][bj][r] = (cv && mrel < mlim) ? cb[(uint32_t)mrel * ldc] : 0.f;
                    }
                    asm volatile("" : "+a"(acc[bi][bj]));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;
        }

        for (int kb = 0; kb < nk; ++kb, ++st) {
            issue_frags(fb, rd_w, rd_h, 1);
            frags_ready<8>(fa);
            copy_w(0, cp_w);
            mfma_step(fa);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            issue_frags(fa, rd_w, rd_h, 2);
            frags_ready<8>(fb);
            copy_w(1, cp_w);
            mfma_step(fb);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            advance_w();
            issue_frags(fb, rd_w, rd_h, 3);
            frags_ready<8>(fa);
            copy_h(0, cp_h);
            mfma_step(fa);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<kDmaPerStage / 4>();            // all but h of st + 2, part 0
            frags_ready<0>(fb);
            asm volatile("s_barrier" ::: "memory");
            rd_h = next_pos(rd_h);
            rd_w = next_pos(rd_w);
            issue_frags(fa, rd_w, rd_h, 0);
            __builtin_amdgcn_sched_barrier(0);
            copy_h(1, cp_h);
            mfma_step(fb);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            advance_h();
            cp_w = next_pos(cp_w);
            cp_h = next_pos(cp_h);
        }

        if constexpr (kMode == kF32Fold) {
        // ---- epilogue of one vocabulary tile: online log-sum-exp + gather.
        // Per token column, the lane's 64 rows are folded block by block
        // (32-row MFMA blocks bi = 0..3, 16 rows per lane each) into the
        // running (max, sum-exp); inside a block the 16 exponentials are
        // summed by a fixed pairwise tree.  Rows past V (last tile only) are
        // -inf.  Branch-free apart from one uniform tail test per tile.
        const int64_t vbase_w = (vt_first + vt_local) * kTileV + wv * 128;
        const int64_t lim64 = v - vbase_w - lhalf * 4;    // rows < lim are valid
        const int lim = lim64 > 128 ? 128 : (int)lim64;
        auto fold = [&](auto masked_tag) {
            constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
                    float z[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        z[r] = acc[bi][bj][r];
                        if constexpr (kMasked) {
                            const int off = bi * 32 + (r >> 2) * 8 + (r & 3);
                            z[r] = off < lim ? z[r] : -INFINITY;
                        }
                    }
                    float bmax = z[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) bmax = fmaxf(bmax, z[r]);
                    const float m_new = fmaxf(m_run[bj], bmax);
                    // exponents as (z - m) c2: exactly 0 for the maximum, so
                    // its term is exactly 1 (a V = 1 row gets logp = 0 exactly)
                    const float mref = m_new == -INFINITY ? 0.f : m_new;
                    const float dsh = (m_run[bj] - mref) * c2;
                    const float scale = m_run[bj] == m_new ? 1.f : fast_exp2(dsh);
                    float e[16];
                    if constexpr (kEnt) {
                        float ea[16];
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float a = fmaxf((z[r] - mref) * c2, kArgFloor);
                            e[r] = fast_exp2(a);
                            ea[r] = e[r] * a;
                        }
#pragma unroll
                        for (int width = 8; width >= 1; width >>= 1)
#pragma unroll
                            for (int r = 0; r < width; ++r) ea[r] = ea[r] + ea[r + width];
                        const float uo = m_run[bj] == m_new
                                             ? u_run[bj]
                                             : (s_run[bj] > 0.f ? scale * fmaf(dsh, s_run[bj], u_run[bj])
                                                                : 0.f);
                        u_run[bj] = uo + ea[0];
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) e[r] = fast_exp2((z[r] - mref) * c2);
                    }
#pragma unroll
                    for (int width = 8; width >= 1; width >>= 1)
#pragma unroll
                        for (int r = 0; r < width; ++r) e[r] = e[r] + e[r + width];
                    s_run[bj] = fmaf(s_run[bj], scale, e[0]);
                    m_run[bj] = m_new;
                }
            }
        };
        if (lim < 128) fold(BoolConst<true>{});
        else fold(BoolConst<false>{});

        // gather: exactly one lane of the grid holds z[t, a_t]; rare, so one
        // divergent region per tile keeps the value in a register
        int tgt[4];
        bool any_tgt = false;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t rel = (int64_t)my_id[bj] - vbase_w;
            const bool mine = rel >= 0 && rel < 128 && (((rel & 31) >> 2) & 1) == lhalf;
            tgt[bj] = mine ? (int)((rel >> 5) * 16 + ((rel & 31) >> 3) * 4 + (rel & 3)) : -1;
            any_tgt |= mine;
        }
        if (any_tgt) {
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        zsel_reg[bj] = tgt[bj] == bi * 16 + r ? acc[bi][bj][r] : zsel_reg[bj];
            have_zsel |= any_tgt;
        }
        }
    }
    if constexpr (kMode != kF32Fold) {
        // the backward's tiles: drain the look-ahead reads and the extra
        // copies, then write the tile
        frags_ready<0>(fa);
        wait_vmcnt<0>();
        if constexpr (kMode == kF32Dz) {
            // dz = g_t ([v == a_t] - exp(z - lse_t)) for v < V, t < N; 0 in
            // the padding up to (Vp, Np).  Rows past V of the tile hold
            // finite logits of a clamped row, and their dz is selected away.
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t t = t0 + wt * 128 + bj * 32 + lrow;
                const bool tv = t < n;
                const float g = tv ? ep.g[t] : 0.f;
                const float l = tv ? ep.lse[t] : 0.f;
                const int32_t a = my_id[bj];
                const bool ok = tv && a >= 0 && (int64_t)a < v && g != 0.f;
                const bool t_in = t < ep.npad;
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t v0 = arow0 + bi * 32 + q * 8;   // four rows v0 .. v0 + 3
                        float d[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t vv = v0 + i;
                            const float pz = fast_exp2((acc[bi][bj][q * 4 + i] - l) * kLog2e);
                            const float dz = g * ((vv == (int64_t)a ? 1.f : 0.f) - pz);
                            d[i] = (ok && vv < v) ? dz : 0.f;
                        }
                        if (t_in && v0 < ep.vpad) {
                            if (ep.dz)
                                *(float4*)(ep.dz + t * ep.ldz + v0) = make_float4(d[0], d[1], d[2], d[3]);
                            if (ep.dzt) {
#pragma unroll
                                for (int i = 0; i < 4; ++i) ep.dzt[(v0 + i) * ep.lddzt + t] = d[i];
                            }
                        }
                    }
                }
            }
        } else {
            // C[m][n]: lanes of a row hold 32 consecutive n (128 bytes)
            const uint32_t ldc = (uint32_t)ep.ldc;
            const int64_t mlim = v - arow0;
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t cn = t0 + wt * 128 + bj * 32 + lrow;
                if (cn >= n) continue;
                float* cb = ep.c + arow0 * ep.ldc + cn;
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int mrel = bi * 32 + (r >> 2) * 8 + (r & 3);
                        if (mrel < mlim) cb[(uint32_t)mrel * ldc] = acc[bi][bj][r];
                    }
            }
        }
        return;
    }
    // drain: the last stage's look-ahead read and the extra copies; the ring
    // is reused for the wave exchange below
    frags_ready<0>(fa);
    wait_vmcnt<0>();
    __syncthreads();

    // ---- the selected logits this lane owns (one owner per token)
    if (have_zsel) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t rel = (int64_t)my_id[bj] - vt_first * kTileV - wv * 128;
            // owned iff the id lies in this chunk, in this wave's 128-row half
            // of its tile, in this lane's row set
            const int64_t chunk_rows = (int64_t)ntiles_here * kTileV;
            const int64_t in_chunk = (int64_t)my_id[bj] - vt_first * kTileV;
            if (in_chunk >= 0 && in_chunk < chunk_rows && ((in_chunk & 255) >> 7) == wv &&
                (((in_chunk & 31) >> 2) & 1) == lhalf)
                zsel[t0 + wt * 128 + bj * 32 + lrow] = zsel_reg[bj];
            (void)rel;
        }
    }

    // ---- end of chunk: merge half-waves, then the two vocabulary waves
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const float mo = __shfl_xor(m_run[bj], 32);
        const float so = __shfl_xor(s_run[bj], 32);
        if constexpr (kEnt) {
            const float uo = __shfl_xor(u_run[bj], 32);
            lse_combine3(m_run[bj], s_run[bj], u_run[bj], mo, so, uo, c2);
        } else {
            lse_combine(m_run[bj], s_run[bj], mo, so, c2);
        }
    }
    float2* xch = (float2*)lds;          // [token half][token]; the ring is drained
    float* xu = (float*)(lds + 2048);    // u, same index
    if (wv == 1 && lhalf == 0) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            xch[wt * 128 + bj * 32 + lrow] = make_float2(m_run[bj], s_run[bj]);
            if constexpr (kEnt) xu[wt * 128 + bj * 32 + lrow] = u_run[bj];
        }
    }
    __syncthreads();
    if (wv == 0 && lhalf == 0) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const float2 o = xch[wt * 128 + bj * 32 + lrow];
            float m = m_run[bj], s = s_run[bj], u = u_run[bj];
            const int64_t t = t0 + wt * 128 + bj * 32 + lrow;
            if constexpr (kEnt) {
                lse_combine3(m, s, u, o.x, o.y, xu[wt * 128 + bj * 32 + lrow], c2);
                if (t < n) upart[chunk * n + t] = u;
            } else {
                lse_combine(m, s, o.x, o.y, c2);
            }
            if (t < n) part[chunk * n + t] = make_float2(m, s);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16: 16x16x32 MFMAs.  A wave holds 128 vocabulary rows (8 blocks of 16)
// by NB token blocks of 16 as acc[bi][bj] (rows bi * 16 + .., tokens
// bj * 16 + ..).  A fragment (16 rows x 32 K): lane l holds row l & 15, K
// 8 (l >> 4) .. + 7; an output block: lane l holds rows 4 (l >> 4) + i of
// column l & 15.  The helpers below are the epilogue every bf16 kernel runs
// on such a wave tile, so that a logit's fold does not depend on which
// kernel (which token-tile width) computed it.

// Fold the wave tile's logits into the running per-token state.  Per token
// column bj the lane's 32 rows (bi = 0..7, i = 0..3) are folded as four
// groups of 8 (blocks 2p, 2p + 1) in ascending p; inside a group the block
// maximum first, then the 8 exponentials summed by a fixed pairwise tree.
// Rows with offset bi * 16 + i >= lim (past V, last tile only) are -inf.
template <bool kEnt, bool kMasked, int NB>
__device__ __forceinline__ void fold16(const f32x4 (&acc)[8][NB], int lim, float c2,
                                       float (&m_run)[NB], float (&s_run)[NB],
                                       float (&u_run)[NB]) {
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
#pragma unroll
        for (int part = 0; part < 4; ++part) {      // bi = 2 part, 2 part + 1
            float z[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int bi = part * 2 + (q >> 2), i = q & 3;
                z[q] = acc[bi][bj][i];
                if constexpr (kMasked) z[q] = bi * 16 + i < lim ? z[q] : -INFINITY;
            }
            float bmax = z[0];
#pragma unroll
            for (int q = 1; q < 8; ++q) bmax = fmaxf(bmax, z[q]);
            const float m_new = fmaxf(m_run[bj], bmax);
            // exponents as (z - m) c2: exactly 0 for the maximum, so its
            // term is exactly 1 (a V = 1 row gets logp = 0 exactly)
            const float mref = m_new == -INFINITY ? 0.f : m_new;
            const float dsh = (m_run[bj] - mref) * c2;
            const float scale = m_run[bj] == m_new ? 1.f : fast_exp2(dsh);
            float e[8];
            if constexpr (kEnt) {
                float ea[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float a = fmaxf((z[q] - mref) * c2, kArgFloor);
                    e[q] = fast_exp2(a);
                    ea[q] = e[q] * a;
                }
#pragma unroll
                for (int width = 4; width >= 1; width >>= 1)
#pragma unroll
                    for (int q = 0; q < width; ++q) ea[q] = ea[q] + ea[q + width];
                const float uo = m_run[bj] == m_new
                                     ? u_run[bj]
                                     : (s_run[bj] > 0.f ? scale * fmaf(dsh, s_run[bj], u_run[bj])
                                                        : 0.f);
                u_run[bj] = uo + ea[0];
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = fast_exp2((z[q] - mref) * c2);
            }
#pragma unroll
            for (int width = 4; width >= 1; width >>= 1)
#pragma unroll
                for (int q = 0; q < width; ++q) e[q] = e[q] + e[q + width];
            s_run[bj] = fmaf(s_run[bj], scale, e[0]);
            m_run[bj] = m_new;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Gather: the lane whose row set holds id my_id[bj] (relative row
// rel = id - vbase_w in [0, 128), row group (rel & 15) >> 2 == grp) keeps
// z[t, id] in zsel_reg[bj] and returns its index there (else -1).  Exactly
// one lane of the grid holds each token's selected logit.
template <int NB>
__device__ __forceinline__ void gather16(const f32x4 (&acc)[8][NB], const int32_t (&my_id)[NB],
                                         int64_t vbase_w, int grp, float (&zsel_reg)[NB],
                                         int (&tgt)[NB]) {
    bool any_tgt = false;
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
        const int64_t rel = (int64_t)my_id[bj] - vbase_w;
        const bool mine = rel >= 0 && rel < 128 && (int)((rel & 15) >> 2) == grp;
        tgt[bj] = mine ? (int)((rel >> 4) * 4 + (rel & 3)) : -1;
        any_tgt |= mine;
    }
    if (any_tgt) {
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) {
#pragma unroll
            for (int bi = 0; bi < 8; ++bi)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    zsel_reg[bj] = tgt[bj] == bi * 4 + i ? acc[bi][bj][i] : zsel_reg[bj];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The wave's four row groups of each token column, merged: xor 16, then 32.
template <bool kEnt, int NB>
__device__ __forceinline__ void merge_row_groups(float (&m_run)[NB], float (&s_run)[NB],
                                                 float (&u_run)[NB], float c2) {
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
#pragma unroll
        for (int sh = 16; sh <= 32; sh <<= 1) {
            const float mo = __shfl_xor(m_run[bj], sh);
            const float so = __shfl_xor(s_run[bj], sh);
            if constexpr (kEnt) {
                const float uo = __shfl_xor(u_run[bj], sh);
                lse_combine3(m_run[bj], s_run[bj], u_run[bj], mo, so, uo, c2);
            } else {
                lse_combine(m_run[bj], s_run[bj], mo, so, c2);
            }
        }
    }
}

// bf16 partials: one 256-vocabulary x 256-token tile per workgroup, eight
// waves, two per SIMD.
//
// Same tiles, vocabulary chunks (one tile each), LDS ring, copies and
// chunk-merge order as lmhead_partials_kernel (which serves fp32).  On this
// chip a 16x16x32 bf16 MFMA stream sustains 2.08 PFLOP/s against 1.75 for
// 32x32x16; and with two waves per SIMD one wave's MFMAs keep the matrix
// unit busy while the other waits on the issue of its buffer-to-LDS copies
// or at a barrier.  Wave w owns vocabulary rows (w & 1) * 128 .. + 127 and
// tokens (w >> 1) * 64 .. + 63 of the tile as 8 x 4 MFMA blocks (128
// accumulator registers, so two waves fit a SIMD).  A stage (128 bytes of K)
// is two k-steps; each wave copies 4 units of W and 4 of h (1 KiB each) per
// stage.
//
// Fragment registers: A[8] (one per row block), B0[4] and B1[4] (the column
// blocks of the stage's two k-steps).  Reads run ahead of the MFMAs:
//   ks0: read B1 (this stage's ks1); per row r: wait, 4 MFMAs (a W copy for
//        stage + 1 in rows 0-3), read A[r] <- ks1 row r.
//   ks1: rows 0-3: wait, 4 MFMAs, an h copy (stage + 2); then wait for this
//        wave's copies of stage + 1 and for all its reads, barrier, read B0
//        and A[0..3] <- next stage ks0; rows 4-7: 4 MFMAs, read A[r] <- next
//        stage ks0 row r.
// LDS reads of a wave complete in order; counting the reads issued after
// the one a row needs gives the waits: 11 for every ks0 row, 7 - r for ks1
// rows 0-3 (ks1 rows 4-7 need nothing new).  Past the last stage the copies
// wrap to K offset 0 and the reads continue into positions never used: every
// stage issues the same instructions, so the counts hold everywhere.  The
// look-ahead reads of the last stage are waited for right after the K loop,
// so that none of the fragment registers is live in the epilogue.
//
// kStore (the K-split schedule, never the batch-invariant path): the
// grid holds ksplit copies of the tile grid, copy s computing stages
// s nk .. (s + 1) nk - 1 of K (nk is per copy), and the epilogue stores the
// partial logits to slog[s][v][n] instead of folding them; a separate kernel
// adds the copies and folds.
template <bool kEnt, bool kStore = false>
__global__ void __launch_bounds__(2 * kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
lmhead8w_kernel(const unsigned char* __restrict__ h, int64_t ldh_b,
                const unsigned char* __restrict__ w, int64_t ldw_b,
                const int32_t* __restrict__ ids, int64_t n, int64_t v,
                int nk, int64_t nchunks, int64_t nttiles, float c2,
                float2* __restrict__ part, float* __restrict__ upart,
                float* __restrict__ zsel, int32_t* __restrict__ n_bad_ids,
                float* __restrict__ slog) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wv = wave & 1;        // vocabulary half of the tile (128 rows)
    const int wt = wave >> 1;       // token quarter of the tile (64 tokens)
    const int col = lane & 15;      // token column inside a 16 x 16 block
    const int grp = lane >> 4;      // row group: rows 4 grp .. 4 grp + 3 of a block

    if (blockIdx.x == 0 && tid == 0 && n_bad_ids) *n_bad_ids = 0;

    int64_t chunk, ttile;
    const int64_t tiles = nchunks * nttiles;
    const int64_t split = kStore ? (int64_t)blockIdx.x / tiles : 0;
    tile_of_block(kStore ? (int64_t)blockIdx.x % tiles : (int64_t)blockIdx.x,
                  kStore ? tiles : (int64_t)gridDim.x, nchunks, nttiles, chunk, ttile);
    const int64_t t0 = ttile * kTileT;
    const int64_t vbase = chunk * kTileV;
    if constexpr (kStore) {
        // this copy's K range: move both operands' bases to its first stage
        h += split * nk * kStageBytes;
        w += split * nk * kStageBytes;
    }

    // Copies: as in lmhead_partials_kernel, with eight waves: 8-row blocks
    // 4 wave .. 4 wave + 3 of both operands, swizzled chunks, rows past N or
    // V redirected to the last valid row.  Every access lies inside the
    // tensors and inside the descriptor's extent.
    uint32_t hoff[4], woff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int drow = (wave * 4 + j) * 8 + (lane >> 3);
        const uint32_t cb = (uint32_t)(((lane & 7) ^ ((drow >> 1) & 7)) * 16);
        const int64_t t = t0 + drow < n ? t0 + drow : n - 1;
        const int64_t r = vbase + drow < v ? vbase + drow : v - 1;
        hoff[j] = (uint32_t)((t - t0) * ldh_b) + cb;
        woff[j] = (uint32_t)((r - vbase) * ldw_b) + cb;
    }
    const int64_t hrows = (n - t0) < kTileT ? (n - t0) : kTileT;
    const int64_t wrows = (v - vbase) < kTileV ? (v - vbase) : kTileV;
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(h + t0 * ldh_b), (short)0,
        (int)((hrows - 1) * ldh_b + (int64_t)nk * kStageBytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + vbase * ldw_b), (short)0,
        (int)((wrows - 1) * ldw_b + (int64_t)nk * kStageBytes), kRsrcWord3);

    // fragment addresses: row col of a 16-row block, logical chunk ks*4 + grp
    const uint32_t lds_base = lds_addr(lds);
    const uint32_t kofs0 = (uint32_t)swz(col, 0 * 4 + grp);
    const uint32_t kofs1 = (uint32_t)swz(col, 1 * 4 + grp);
    const uint32_t a_half = (uint32_t)(wv * 128 * kStageBytes);   // this wave's W rows
    const uint32_t b_half = (uint32_t)(wt * 64 * kStageBytes);    // this wave's h rows

    int w_kb = 0, h_kb = 0;
    auto copy_w = [&](int j, int pos) {
        dma16_buf(wrs, lds + pos * kOperandBytes + (wave * 4 + j) * 1024, woff[j],
                  (uint32_t)(w_kb * kStageBytes));
    };
    auto copy_h = [&](int j, int pos) {
        dma16_buf(hrs, lds + pos * kOperandBytes + (wave * 4 + j) * 1024, hoff[j],
                  (uint32_t)(h_kb * kStageBytes));
    };
    auto advance_w = [&]() { if (++w_kb == nk) w_kb = 0; };
    auto advance_h = [&]() { if (++h_kb == nk) h_kb = 0; };
    auto next_pos = [](int p) { return p + 2 >= kPos ? p + 2 - kPos : p + 2; };

    f32x4 acc[8][4];
    u32x4 A[8], B0[4], B1[4];
    // reads of one k-step's fragments (block offsets as immediates)
    auto read_a = [&](int r, uint32_t base) {
        switch (r) {
            case 0: lds_read16<0 * 2048>(A[0], base); break;
            case 1: lds_read16<1 * 2048>(A[1], base); break;
            case 2: lds_read16<2 * 2048>(A[2], base); break;
            case 3: lds_read16<3 * 2048>(A[3], base); break;
            case 4: lds_read16<4 * 2048>(A[4], base); break;
            case 5: lds_read16<5 * 2048>(A[5], base); break;
            case 6: lds_read16<6 * 2048>(A[6], base); break;
            default: lds_read16<7 * 2048>(A[7], base); break;
        }
    };
    auto read_b = [&](u32x4 (&B)[4], uint32_t base) {
        lds_read16<0 * 2048>(B[0], base);
        lds_read16<1 * 2048>(B[1], base);
        lds_read16<2 * 2048>(B[2], base);
        lds_read16<3 * 2048>(B[3], base);
    };
    // tied-accumulator asm MFMAs (mfma_pipe.h)
    auto mfma = [&](int r, int bj, const u32x4& b) { mfma16_tied(acc[r][bj], A[r], b); };

    // Ring positions as in lmhead_partials_kernel: (2 stage + op) % 5.
    int rd_h = 0, rd_w = 1;
    int cp_w = 3, cp_h = 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_h(j, 0);
    advance_h();
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_w(j, 1);
    advance_w();
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_h(j, 2);
    advance_h();
#pragma unroll
    for (int bi = 0; bi < 8; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
    wait_vmcnt<4>();
    __syncthreads();
    {
        const uint32_t aw = lds_base + (uint32_t)(rd_w * kOperandBytes) + a_half;
        const uint32_t bh = lds_base + (uint32_t)(rd_h * kOperandBytes) + b_half;
        read_b(B0, bh + kofs0);
#pragma unroll
        for (int r = 0; r < 8; ++r) read_a(r, aw + kofs0);
    }

    for (int kb = 0; kb < nk; ++kb) {
        const uint32_t aw = lds_base + (uint32_t)(rd_w * kOperandBytes) + a_half;
        const uint32_t bh = lds_base + (uint32_t)(rd_h * kOperandBytes) + b_half;
        // ---- ks0: W(s+1) copies at rows 0-3
        read_b(B1, bh + kofs1);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r == 0) wait16_4<11>(A[0], B0);
            else wait16<11>(A[r]);
            mfma(r, 0, B0[0]); mfma(r, 1, B0[1]);
            if (r < 4) copy_w(r, cp_w);
            mfma(r, 2, B0[2]); mfma(r, 3, B0[3]);
            read_a(r, aw + kofs1);
        }
        advance_w();
        // ---- ks1, rows 0-3: h(s+2) copies
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r == 0) wait16_4<7>(A[0], B1);
            else if (r == 1) wait16<6>(A[1]);
            else if (r == 2) wait16<5>(A[2]);
            else wait16<4>(A[3]);
            mfma(r, 0, B1[0]); mfma(r, 1, B1[1]);
            copy_h(r, cp_h);
            mfma(r, 2, B1[2]); mfma(r, 3, B1[3]);
        }
        // stage + 1 resident (this wave's copies, then everyone's) and
        // every read of this stage done before its slots are reused
        wait_vmcnt<4>();
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(A[4]), "+v"(A[5]), "+v"(A[6]), "+v"(A[7]));
        asm volatile("s_barrier" ::: "memory");
        rd_h = next_pos(rd_h);
        rd_w = next_pos(rd_w);
        const uint32_t aw2 = lds_base + (uint32_t)(rd_w * kOperandBytes) + a_half;
        const uint32_t bh2 = lds_base + (uint32_t)(rd_h * kOperandBytes) + b_half;
        read_b(B0, bh2 + kofs0);
#pragma unroll
        for (int r = 0; r < 4; ++r) read_a(r, aw2 + kofs0);
        // ---- ks1, rows 4-7
#pragma unroll
        for (int r = 4; r < 8; ++r) {
            wait16<11>(A[r]);
            mfma(r, 0, B1[0]); mfma(r, 1, B1[1]); mfma(r, 2, B1[2]);
            if (r < 7) mfma(r, 3, B1[3]);
            else mfma16_tied_last(acc[7][3], A[7], B1[3],   // + the epilogue's wait
                                  __builtin_amdgcn_readfirstlane(kb == nk - 1));
            read_a(r, aw2 + kofs0);
        }
        advance_h();
        cp_w = next_pos(cp_w);
        cp_h = next_pos(cp_h);
    }
    // The 4 tokens of this lane (one per 16-column block) and their ids,
    // loaded here rather than before the K loop, where every register is
    // taken: from clamped rows, issued together, -1 for a column past N.
    // Their latency hides under the fold below.
    int32_t my_id[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const int64_t t = t0 + wt * 64 + bj * 16 + col;
        my_id[bj] = ids[t < n ? t : n - 1];
    }
    // the last stage's look-ahead reads: waited for here, so that no
    // fragment register is live (or still being written) in the epilogue
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(A[0]), "+v"(A[1]), "+v"(A[2]), "+v"(A[3]),
                 "+v"(A[4]), "+v"(A[5]), "+v"(A[6]), "+v"(A[7]));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(B0[0]), "+v"(B0[1]), "+v"(B0[2]), "+v"(B0[3]));

    if constexpr (kStore) {
        // partial logits of this K range: rows vbase + wv 128 + bi 16 + 4 grp
        // + i, token t0 + wt 64 + bj 16 + col (16 tokens of a row group are
        // 64 contiguous bytes)
        float* base = slog + split * v * n;
#pragma unroll
        for (int bi = 0; bi < 8; ++bi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = vbase + wv * 128 + bi * 16 + grp * 4 + i;
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const int64_t t = t0 + wt * 64 + bj * 16 + col;
                    if (row < v && t < n) base[row * n + t] = acc[bi][bj][i];
                }
            }
        wait_vmcnt<0>();
        return;
    }

    // ---- epilogue: online log-sum-exp + gather over the tile
    float m_run[4], s_run[4], u_run[4], zsel_reg[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        m_run[bj] = -INFINITY; s_run[bj] = 0.f; u_run[bj] = 0.f; zsel_reg[bj] = 0.f;
    }
    const int64_t vbase_w = vbase + wv * 128;
    const int64_t lim64 = v - vbase_w - grp * 4;     // row offsets bi*16 + i < lim are valid
    const int lim = lim64 > 128 ? 128 : (int)lim64;
    if (lim < 128) fold16<kEnt, true, 4>(acc, lim, c2, m_run, s_run, u_run);
    else fold16<kEnt, false, 4>(acc, lim, c2, m_run, s_run, u_run);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
        if (t0 + wt * 64 + bj * 16 + col >= n) my_id[bj] = -1;
    int tgt[4];
    gather16<4>(acc, my_id, vbase_w, grp, zsel_reg, tgt);
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
        if (tgt[bj] >= 0) zsel[t0 + wt * 64 + bj * 16 + col] = zsel_reg[bj];

    // ---- end of chunk: merge the four row groups, then the two vocabulary
    // waves.  The extra copies of the last stages land in the ring, which
    // the exchange reuses: wait for them first.
    merge_row_groups<kEnt, 4>(m_run, s_run, u_run, c2);
    wait_vmcnt<0>();
    __syncthreads();
    float2* xch = (float2*)lds;          // [token quarter][token]
    float* xu = (float*)(lds + 2048);    // u, same index
    if (wv == 1 && grp == 0) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            xch[wt * 64 + bj * 16 + col] = make_float2(m_run[bj], s_run[bj]);
            if constexpr (kEnt) xu[wt * 64 + bj * 16 + col] = u_run[bj];
        }
    }
    __syncthreads();
    if (wv == 0 && grp == 0) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const float2 o = xch[wt * 64 + bj * 16 + col];
            float m = m_run[bj], s = s_run[bj], u = u_run[bj];
            const int64_t t = t0 + wt * 64 + bj * 16 + col;
            if constexpr (kEnt) {
                lse_combine3(m, s, u, o.x, o.y, xu[wt * 64 + bj * 16 + col], c2);
                if (t < n) upart[chunk * n + t] = u;
            } else {
                lse_combine(m, s, o.x, o.y, c2);
            }
            if (t < n) part[chunk * n + t] = make_float2(m, s);
        }
    }
}

// bf16 partials for small batches: one wave per 128-row half of a
// vocabulary chunk and 16 NB tokens (NB = 1, 2 or 4 column blocks; the
// kernel also takes several token groups, unused while kNarrowMaxTokens is
// one group of 4 blocks).
//
// At a few tokens the 256-token tile of lmhead8w_kernel spends almost all
// of its MFMA work on padding, while the call is bound by reading W once
// (V D 2 bytes).  This kernel streams W through a two-slot LDS ring of its
// own, one wave per workgroup and no barrier, and at the Qwen3-8B shape
// 1187 independent waves keep the whole matrix in flight.  It computes each logit with the
// same instruction as lmhead8w_kernel (v_mfma_f32_16x16x32_bf16, W rows as
// the first source, tokens as the second, the same K -> lane assignment, k
// steps in ascending order from a zero accumulator) and folds it with the
// same helpers (fold16, gather16, merge_row_groups) in the same lane
// layout, so every per-token state it writes has the bits lmhead8w_kernel
// forms for the same half of the same chunk.  The only difference: the two
// halves of a chunk are separate waves here, so each writes its own state
// (hpart[2 chunk + half][n]) and the merge combines the pair in the order
// lmhead8w_kernel's exchange uses (half 0 first, half 1 merged into it).
// The MFMAs are tied-accumulator asm, as in lmhead8w_kernel (with the
// builtin the allocator moves all accumulators between registers every
// round, and each move waits for its MFMA); the wait states asm hides from
// the compiler's hazard recognizer are mfma_drain's after the loop, and the
// code as built is checked for MFMA hazards on every path.
//
// Operand path: k-step j of this wave (32 K; 2 per 128-byte stage) needs 8 A
// fragments (row block r: lane l holds row r*16 + (l & 15), K 8 (l >> 4) ..
// + 7) and NB B fragments.  Loading the A fragments straight from memory
// touches 16 rows x 64 bytes per instruction, half of each 128-byte line;
// measured on this chip a wave-per-128-rows read of the whole matrix in
// that shape moves 4.0 TB/s, in 8 rows x 128 bytes 5.8 TB/s.  So W goes to
// LDS by buffer-to-LDS copies of 8 rows x 128 bytes (XOR-swizzled chunks,
// as in the tile kernels) two stages ahead, and each k-step's A fragments
// are read back with ds_read_b128; the B fragments (a few tokens, in L2)
// are 16-byte buffer loads into a ring of three register sets.  Every
// stage issues the same copies and loads (past the last stage they repeat
// the last one, into a slot not read again), so the vmcnt waits count
// them.  The descriptors are built from the tensors' own pointers; W rows
// past V read as zero through the descriptor's range check, h rows past N
// are redirected to the last valid row, and results of either are masked
// or dropped.
//
// Work map: unit u = (chunk u >> 1, half u & 1), token group g.  Block b
// serves unit ((b >> 3) / ntg) * 8 + (b & 7) and group (b >> 3) % ntg: the
// groups of a unit run on one XCD (b & 7) next to each other, so W is read
// from HBM once and from that XCD's L2 by the other group.
constexpr int kNarrowMaxTokens = 64;   // above: token groups re-read W, and the
                                        // 256-token kernel is faster

template <bool kEnt, int NB>
__global__ void __launch_bounds__(64)
lmhead_narrow_kernel(const unsigned char* __restrict__ h, int64_t ldh_b,
                     const unsigned char* __restrict__ w, int64_t ldw_b,
                     const int32_t* __restrict__ ids, int64_t n, int64_t v, int nk,
                     int64_t nchunks, int ntg, float c2, float2* __restrict__ hpart,
                     float* __restrict__ hupart, float* __restrict__ zsel,
                     int32_t* __restrict__ n_bad_ids) {
    const int lane = threadIdx.x;
    const int col = lane & 15, grp = lane >> 4;
    if (blockIdx.x == 0 && lane == 0 && n_bad_ids) *n_bad_ids = 0;

    const int64_t q = blockIdx.x >> 3;
    const int g = (int)(q % ntg);
    const int64_t unit = (q / ntg) * 8 + (blockIdx.x & 7);
    if (unit >= 2 * nchunks) return;
    const int64_t chunk = unit >> 1;
    const int wv = (int)(unit & 1);
    const int64_t vbase_w = chunk * kTileV + wv * 128;
    const int64_t t0 = (int64_t)g * 16 * NB;
    if (vbase_w >= v) {
        // the upper half of a last chunk with at most 128 rows: the state
        // lmhead8w_kernel forms for a half with no valid row
        if (grp == 0) {
#pragma unroll
            for (int bj = 0; bj < NB; ++bj) {
                const int64_t t = t0 + bj * 16 + col;
                if (t < n) {
                    hpart[unit * n + t] = make_float2(-INFINITY, 0.f);
                    if constexpr (kEnt) hupart[unit * n + t] = 0.f;
                }
            }
        }
        return;
    }
    const int64_t wrows = (v - vbase_w) < 128 ? (v - vbase_w) : 128;
    const int64_t hrows = (n - t0) < 16 * NB ? (n - t0) : 16 * NB;
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(w + vbase_w * ldw_b), (short)0,
        (int)((wrows - 1) * ldw_b + (int64_t)nk * kStageBytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(h + t0 * ldh_b), (short)0,
        (int)((hrows - 1) * ldh_b + (int64_t)nk * kStageBytes), kRsrcWord3);
    // W: stage s (128 bytes of K, two k-steps) of the wave's 128 rows goes
    // to LDS slot s & 1 by 16 buffer-to-LDS copies of 8 rows x 128 bytes
    // (copy q: rows 8 q .. 8 q + 7; lane l writes 16 bytes at 16 l, i.e.
    // row 8 q + (l >> 3), physical chunk l & 7, which holds logical chunk
    // (l & 7) ^ ((row >> 1) & 7)).  The logical chunk depends on q only
    // through q & 1, so two per-lane offsets, plus the copy's rows, address
    // them.  The row offset stays in the per-lane offset, which the
    // descriptor's range check covers (the scalar offset, the stage's K
    // offset, is not checked): rows past V then read as zero, with no
    // access (their logits are masked in the fold).
    uint32_t avoff[2], boff[NB];
#pragma unroll
    for (int pq = 0; pq < 2; ++pq) {
        const int lc = (lane & 7) ^ ((4 * pq + (lane >> 4)) & 7);
        avoff[pq] = (uint32_t)((8 * pq + (lane >> 3)) * ldw_b) + (uint32_t)(lc * 16);
    }
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
        const int64_t row = bj * 16 + col < hrows ? bj * 16 + col : hrows - 1;
        boff[bj] = (uint32_t)(row * ldh_b) + (uint32_t)(grp * 16);
    }
    // fragment reads: row block rb (immediate 2048 rb), lane row col, logical
    // chunk 4 h + grp of k-step h: its physical chunk is the same in every
    // row block (the swizzle takes row bits 1-3, which rb does not change)
    uint32_t afrag[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        afrag[hh] = (uint32_t)(col * 128) + (uint32_t)((((4 * hh + grp) ^ (col >> 1)) & 7) * 16);
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * 16384];
    const uint32_t lds_base = lds_addr(lds);

    u32x4 A[2][8], B[3][2][NB];
    f32x4 acc[8][NB];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) acc[r][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

    // every stage issues the same loads (past the last stage they repeat
    // the last one, into a slot that is not read again): 16 copies, then
    // 2 NB h loads
    constexpr int L2 = 16 + 2 * NB;
    static_assert(L2 <= 63, "vmcnt range");
    // copies q0 .. q0 + 7 (rows 8 q0 .. 8 q0 + 63) of stage st
    auto issue_rows = [&](int st, auto q0_tag) {
        constexpr int q0 = decltype(q0_tag)::value;
        const int ss = __builtin_amdgcn_readfirstlane(st < nk ? st : nk - 1);
        unsigned char* slot = lds + (st & 1) * 16384;
#pragma unroll
        for (int q = q0; q < q0 + 8; ++q)
            dma16_buf(wrs, slot + q * 1024, avoff[q & 1] + (uint32_t)((q >> 1) * 16 * ldw_b),
                      (uint32_t)(ss * kStageBytes));
    };
    auto issue_h = [&](auto bslot_tag, int st) {
        constexpr int bs = decltype(bslot_tag)::value;
        const int ss = __builtin_amdgcn_readfirstlane(st < nk ? st : nk - 1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int bj = 0; bj < NB; ++bj)
                B[bs][hh][bj] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    hrs, boff[bj], (uint32_t)(ss * kStageBytes + hh * 64), 0));
    };
    auto issue = [&](auto bslot_tag, int st) {
        issue_rows(st, IntConst<0>{});
        issue_rows(st, IntConst<8>{});
        issue_h(bslot_tag, st);
    };
    // stage st: its copies and loads were issued two stages ago.  Wait for
    // them and read the 16 fragments, rows 0-63 first; as soon as those
    // reads are done their rows of the slot take stage st + 2's copies, then
    // the rest.  Then the stage's MFMAs: k-step 0 then 1, row blocks in
    // order, token blocks in order (the order lmhead8w_kernel's wave applies
    // to the same fragments).
    auto stage = [&](auto bslot_tag, int st) {
        constexpr int bs = decltype(bslot_tag)::value;
        wait_vmcnt<L2>();
        const uint32_t base = lds_base + (uint32_t)((st & 1) * 16384);
        const uint32_t a0 = base + afrag[0], a1 = base + afrag[1];
        lds_read16<0 * 2048>(A[0][0], a0);
        lds_read16<0 * 2048>(A[1][0], a1);
        lds_read16<1 * 2048>(A[0][1], a0);
        lds_read16<1 * 2048>(A[1][1], a1);
        lds_read16<2 * 2048>(A[0][2], a0);
        lds_read16<2 * 2048>(A[1][2], a1);
        lds_read16<3 * 2048>(A[0][3], a0);
        lds_read16<3 * 2048>(A[1][3], a1);
        lds_read16<4 * 2048>(A[0][4], a0);
        lds_read16<4 * 2048>(A[1][4], a1);
        lds_read16<5 * 2048>(A[0][5], a0);
        lds_read16<5 * 2048>(A[1][5], a1);
        lds_read16<6 * 2048>(A[0][6], a0);
        lds_read16<6 * 2048>(A[1][6], a1);
        lds_read16<7 * 2048>(A[0][7], a0);
        lds_read16<7 * 2048>(A[1][7], a1);
        // LDS operations of a wave complete in order: 8 outstanding means
        // the reads of rows 0-63 are done
        asm volatile("s_waitcnt lgkmcnt(8)"
                     : "+v"(A[0][0]), "+v"(A[1][0]), "+v"(A[0][1]), "+v"(A[1][1]),
                       "+v"(A[0][2]), "+v"(A[1][2]), "+v"(A[0][3]), "+v"(A[1][3]));
        __builtin_amdgcn_sched_barrier(0);
        issue_rows(st + 2, IntConst<0>{});
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(A[0][4]), "+v"(A[1][4]), "+v"(A[0][5]), "+v"(A[1][5]),
                       "+v"(A[0][6]), "+v"(A[1][6]), "+v"(A[0][7]), "+v"(A[1][7]));
        __builtin_amdgcn_sched_barrier(0);
        issue_rows(st + 2, IntConst<8>{});
        issue_h(IntConst<(bs + 2) % 3>{}, st + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int bj = 0; bj < NB; ++bj) mfma16_tied(acc[r][bj], A[hh][r], B[bs][hh][bj]);
        __builtin_amdgcn_sched_barrier(0);
    };
    issue(IntConst<0>{}, 0);
    issue(IntConst<1>{}, 1);
    // whole rounds of three stages (the h ring), then the remainder
    int st = 0;
    for (; st + 3 <= nk; st += 3) {
        stage(IntConst<0>{}, st);
        stage(IntConst<1>{}, st + 1);
        stage(IntConst<2>{}, st + 2);
    }
    const int rem = __builtin_amdgcn_readfirstlane(nk - st);
    if (rem >= 1) stage(IntConst<0>{}, st);
    if (rem >= 2) stage(IntConst<1>{}, st + 1);
    wait_vmcnt<0>();
    mfma_drain<NB>(acc);

    // ---- epilogue, as lmhead8w_kernel's for one wave
    float m_run[NB], s_run[NB], u_run[NB], zsel_reg[NB];
    int32_t my_id[NB];
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) {
        m_run[bj] = -INFINITY; s_run[bj] = 0.f; u_run[bj] = 0.f; zsel_reg[bj] = 0.f;
        const int64_t t = t0 + bj * 16 + col;
        my_id[bj] = t < n ? ids[t] : -1;
    }
    const int64_t lim64 = v - vbase_w - grp * 4;
    const int lim = lim64 > 128 ? 128 : (int)lim64;
    if (lim < 128) fold16<kEnt, true, NB>(acc, lim, c2, m_run, s_run, u_run);
    else fold16<kEnt, false, NB>(acc, lim, c2, m_run, s_run, u_run);
    int tgt[NB];
    gather16<NB>(acc, my_id, vbase_w, grp, zsel_reg, tgt);
#pragma unroll
    for (int bj = 0; bj < NB; ++bj)
        if (tgt[bj] >= 0) zsel[t0 + bj * 16 + col] = zsel_reg[bj];
    merge_row_groups<kEnt, NB>(m_run, s_run, u_run, c2);
    if (grp == 0) {
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) {
            const int64_t t = t0 + bj * 16 + col;
            if (t < n) {
                hpart[unit * n + t] = make_float2(m_run[bj], s_run[bj]);
                if constexpr (kEnt) hupart[unit * n + t] = u_run[bj];
            }
        }
    }
}

// The K-split schedule: adds the ksplit partial logits of each row
// (in ascending copy order) and folds a chunk's 256 rows into (max, sum-exp)
// per token, keeping the selected logit.  One thread per token, a block per
// (chunk, 64 tokens); the row loads do not depend on the fold, so they run
// ahead of it.
__global__ void __launch_bounds__(64)
splitk_combine_kernel(const float* __restrict__ slog, int ksplit,
                      const int32_t* __restrict__ ids, int64_t n, int64_t v, float c2,
                      float2* __restrict__ part, float* __restrict__ zsel) {
    const int64_t chunk = blockIdx.x;
    const int64_t t = (int64_t)blockIdx.y * 64 + threadIdx.x;
    if (t >= n) return;
    const int32_t id = ids[t];
    const int64_t r0 = chunk * kTileV;
    const int rows = (int)((v - r0) < kTileV ? (v - r0) : kTileV);
    float m = -INFINITY, s = 0.f;
#pragma unroll 8
    for (int r = 0; r < rows; ++r) {
        float z = slog[(r0 + r) * n + t];
        for (int sp = 1; sp < ksplit; ++sp) z += slog[((int64_t)sp * v + r0 + r) * n + t];
        if (r0 + r == (int64_t)id) zsel[t] = z;
        const float mn = fmaxf(m, z);
        const float sc = m == mn ? 1.f : fast_exp2((m - mn) * c2);
        s = fmaf(s, sc, fast_exp2((z - mn) * c2));
        m = mn;
    }
    part[chunk * n + t] = make_float2(m, s);
}

// Merge of the vocabulary-chunk partials.  A block serves 64 tokens with
// kMergeWaves waves: wave w folds chunks w, w + kMergeWaves, ... in ascending
// order for its 64 tokens (coalesced 8-byte loads, kMergeUnroll in flight),
// then wave 0 folds the kMergeWaves strands in order.  The order depends on
// the number of chunks only.
constexpr int kMergeWaves = 8;
// chunks in flight per strand step: 4 for the whole-chunk layout (many
// tokens per block keep the loads busy), 16 for the half-chunk layout of
// small batches, where a lane's loads are the only ones in flight
template <bool kHalves> struct MergeUnroll { static constexpr int value = kHalves ? 16 : 4; };
constexpr size_t kMergeTokenLdsMax = 64 * 1024;   // chunk states of one token in LDS

// With it = 1 / tau: lse = m it + ln s and logp = (z_a - m) it - ln s (the
// difference z_a - m is formed before the scale, so no two large terms
// cancel); entropy = ln 2 (log2 s - u / s) when kEnt.
//
// kHalves: the partials are per half chunk (lmhead_narrow_kernel): chunk c's
// state is half 2c with half 2c + 1 merged into it, the order in which
// lmhead8w_kernel's wave exchange forms it.
template <bool kEnt, bool kHalves>
__device__ __forceinline__ void load_chunk(const float2* __restrict__ part,
                                           const float* __restrict__ upart, int64_t c, int64_t n,
                                           int64_t tc, float c2, float2& p, float& q) {
    if constexpr (kHalves) {
        const float2 p0 = part[(2 * c) * n + tc], p1 = part[(2 * c + 1) * n + tc];
        float m = p0.x, s = p0.y, u = 0.f;
        if constexpr (kEnt) {
            u = upart[(2 * c) * n + tc];
            lse_combine3(m, s, u, p1.x, p1.y, upart[(2 * c + 1) * n + tc], c2);
        } else {
            lse_combine(m, s, p1.x, p1.y, c2);
        }
        p = make_float2(m, s);
        q = u;
    } else {
        p = part[c * n + tc];
        if constexpr (kEnt) q = upart[c * n + tc];
    }
}

template <bool kEnt, bool kHalves>
__global__ void __launch_bounds__(64 * kMergeWaves)
lse_merge_kernel(const float2* __restrict__ part, const float* __restrict__ upart,
                 const float* __restrict__ zsel, const int32_t* __restrict__ ids, int64_t n,
                 int64_t nchunks, int64_t v, float c2, float it, float* __restrict__ logp,
                 float* __restrict__ lse, float* __restrict__ ent,
                 int32_t* __restrict__ n_bad_ids) {
    __shared__ float2 strand[kMergeWaves][64];
    __shared__ float ustrand[kEnt ? kMergeWaves : 1][64];
    __shared__ int bad_count;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) bad_count = 0;
    const int64_t t = (int64_t)blockIdx.x * 64 + lane;
    const int64_t tc = t < n ? t : n - 1;
    float m = -INFINITY, s = 0.f, uu = 0.f;
    int64_t c = wave;
    constexpr int kMergeUnroll = MergeUnroll<kHalves>::value;
    for (; c + (kMergeUnroll - 1) * kMergeWaves < nchunks; c += kMergeUnroll * kMergeWaves) {
        float2 p[kMergeUnroll];
        float q[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u)
            load_chunk<kEnt, kHalves>(part, upart, c + u * kMergeWaves, n, tc, c2, p[u], q[u]);
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            if constexpr (kEnt) lse_combine3(m, s, uu, p[u].x, p[u].y, q[u], c2);
            else lse_combine(m, s, p[u].x, p[u].y, c2);
        }
    }
    for (; c < nchunks; c += kMergeWaves) {
        float2 p;
        float q = 0.f;
        load_chunk<kEnt, kHalves>(part, upart, c, n, tc, c2, p, q);
        if constexpr (kEnt) lse_combine3(m, s, uu, p.x, p.y, q, c2);
        else lse_combine(m, s, p.x, p.y, c2);
    }
    strand[wave][lane] = make_float2(m, s);
    if constexpr (kEnt) ustrand[wave][lane] = uu;
    __syncthreads();
    if (wave == 0 && t < n) {
        float mm = strand[0][lane].x, ss = strand[0][lane].y, us = 0.f;
        if constexpr (kEnt) us = ustrand[0][lane];
#pragma unroll
        for (int w = 1; w < kMergeWaves; ++w) {
            if constexpr (kEnt)
                lse_combine3(mm, ss, us, strand[w][lane].x, strand[w][lane].y, ustrand[w][lane], c2);
            else
                lse_combine(mm, ss, strand[w][lane].x, strand[w][lane].y, c2);
        }
        const float l2s = fast_log2(ss);
        const float lns = l2s * kLn2;
        const int32_t a = ids[t];
        const bool bad = a < 0 || (int64_t)a >= v;
        logp[t] = bad ? __builtin_nanf("") : fmaf(zsel[t] - mm, it, -lns);
        if (lse) lse[t] = fmaf(mm, it, lns);
        if constexpr (kEnt) ent[t] = (l2s - us / ss) * kLn2;
        if (bad) atomicAdd(&bad_count, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0 && n_bad_ids && bad_count) atomicAdd(n_bad_ids, bad_count);
}

// The same merge for the half-chunk partials of small batches, one block per
// token: the block first loads every chunk's pair of half states at once
// (combining each pair as load_chunk does) into LDS, then eight threads fold
// the eight strands (chunks w, w + 8, ... in ascending order) and thread 0
// folds the strands in order, the sequence lse_merge_kernel follows, so the
// bits are the same.  With a handful of tokens lse_merge_kernel's lanes have
// no loads but their own and wait a full memory latency per unrolled group;
// here one latency covers them all.
template <bool kEnt>
__global__ void __launch_bounds__(512)
lse_merge_token_kernel(const float2* __restrict__ part, const float* __restrict__ upart,
                       const float* __restrict__ zsel, const int32_t* __restrict__ ids, int64_t n,
                       int64_t nchunks, int64_t v, float c2, float it, float* __restrict__ logp,
                       float* __restrict__ lse, float* __restrict__ ent,
                       int32_t* __restrict__ n_bad_ids) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float2* cs = (float2*)smem;                              // [nchunks]
    float* cu = (float*)(smem + nchunks * sizeof(float2));   // [nchunks] when kEnt
    __shared__ float2 strand[kMergeWaves];
    __shared__ float ustrand[kMergeWaves];
    const int64_t t = blockIdx.x;
    for (int64_t c = threadIdx.x; c < nchunks; c += blockDim.x) {
        float2 p;
        float q = 0.f;
        load_chunk<kEnt, true>(part, upart, c, n, t, c2, p, q);
        cs[c] = p;
        if constexpr (kEnt) cu[c] = q;
    }
    __syncthreads();
    if (threadIdx.x < kMergeWaves) {
        const int w = threadIdx.x;
        float m = -INFINITY, s = 0.f, uu = 0.f;
        // unrolled so that the LDS reads of several chunks are in flight
        // ahead of the (sequential) folds
#pragma unroll 8
        for (int64_t c = w; c < nchunks; c += kMergeWaves) {
            const float2 p = cs[c];
            if constexpr (kEnt) lse_combine3(m, s, uu, p.x, p.y, cu[c], c2);
            else lse_combine(m, s, p.x, p.y, c2);
        }
        strand[w] = make_float2(m, s);
        ustrand[w] = uu;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mm = strand[0].x, ss = strand[0].y, us = 0.f;
        if constexpr (kEnt) us = ustrand[0];
#pragma unroll
        for (int w = 1; w < kMergeWaves; ++w) {
            if constexpr (kEnt)
                lse_combine3(mm, ss, us, strand[w].x, strand[w].y, ustrand[w], c2);
            else
                lse_combine(mm, ss, strand[w].x, strand[w].y, c2);
        }
        const float l2s = fast_log2(ss);
        const float lns = l2s * kLn2;
        const int32_t a = ids[t];
        const bool bad = a < 0 || (int64_t)a >= v;
        logp[t] = bad ? __builtin_nanf("") : fmaf(zsel[t] - mm, it, -lns);
        if (lse) lse[t] = fmaf(mm, it, lns);
        if constexpr (kEnt) ent[t] = (l2s - us / ss) * kLn2;
        if (bad && n_bad_ids) atomicAdd(n_bad_ids, 1);
    }
}

}  // namespace

bool make_logprob_plan(int64_t n, int64_t d, int64_t v, int dtype, unsigned flags,
                       bool entropy, LogprobPlan* p) {
    if (n < 0 || d <= 0 || v <= 0 || v > INT32_MAX || (dtype != 0 && dtype != 1) || flags > 2u)
        return false;
    p->n = n; p->d = d; p->v = v; p->dtype = dtype;
    p->nvtiles = (v + kTileV - 1) / kTileV;
    p->nttiles = (n + kTileT - 1) / kTileT;
    // every schedule: one tile per chunk (the K split of flags 2 splits K,
    // not the vocabulary)
    p->chunk_tiles = kInvariantChunkTiles;
    p->nchunks = (p->nvtiles + p->chunk_tiles - 1) / p->chunk_tiles;
    p->entropy = entropy;
    // the K split (flags 2), bf16, 33..256 tokens (one token tile, more than
    // a 32-token group): twice the workgroups of half the work; asked for,
    // it takes those sizes from the small-batch kernel too
    p->ksplit = (flags == 2u && dtype == 0 && !entropy && n > 32 && n <= kTileT &&
                 (d / 64) % 2 == 0) ? 2 : 1;
    p->narrow = dtype == 0 && n >= 1 && n <= kNarrowMaxTokens && p->ksplit == 1;
    p->nb = n <= 16 ? 1 : (n <= 32 ? 2 : 4);
    p->ntg = (int)((n + 16 * p->nb - 1) / (16 * p->nb));
    const size_t nparts = (size_t)p->nchunks * (p->narrow ? 2 : 1);
    p->part_bytes = align_up(nparts * (size_t)n * sizeof(float2), 256);
    p->zsel_off = p->part_bytes;
    p->upart_off = p->zsel_off + align_up((size_t)n * sizeof(float), 256);
    p->slog_off = p->upart_off + (entropy ? align_up(nparts * (size_t)n * sizeof(float), 256) : 0);
    p->total_bytes = p->slog_off +
                     (p->ksplit > 1 ? align_up((size_t)p->ksplit * (size_t)v * (size_t)n * sizeof(float), 256)
                                    : 0);
    if (p->total_bytes == 0) p->total_bytes = 256;
    return true;
}

ScoreScale make_score_scale(double temperature) {
    ScoreScale sc;
    sc.c2 = temperature == 1.0 ? kLog2e : (float)(1.4426950408889634 / temperature);
    sc.it = temperature == 1.0 ? 1.f : (float)(1.0 / temperature);
    return sc;
}

hipError_t launch_lmhead_partials(const LogprobPlan& p, const void* h, int64_t ldh,
                                  const void* w, int64_t ldw, const int32_t* ids,
                                  const ScoreScale& sc, void* workspace, int32_t* n_bad_ids,
                                  hipStream_t st) {
    const int64_t esz = p.dtype == 0 ? 2 : 4;
    const int nk = (int)(p.d * esz / kStageBytes);
    const int64_t grid = p.nchunks * p.nttiles;
    if (grid <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
    float2* part = (float2*)workspace;
    float* zsel = (float*)((unsigned char*)workspace + p.zsel_off);
    float* upart = p.entropy ? (float*)((unsigned char*)workspace + p.upart_off) : nullptr;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, st,
                           (const unsigned char*)h, ldh * esz, (const unsigned char*)w, ldw * esz,
                           ids, p.n, p.v, nk, p.chunk_tiles, p.nvtiles, p.nchunks, p.nttiles,
                           sc.c2, part, upart, zsel, n_bad_ids, F32Epi{});
    };
    if (p.dtype == 0 && p.narrow) {
        // units (chunk halves) rounded up to the 8 XCDs, times the token groups
        const int64_t blocks = (2 * p.nchunks + 7) / 8 * 8 * p.ntg;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        auto gon = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64), 0, st,
                               (const unsigned char*)h, ldh * esz, (const unsigned char*)w, ldw * esz,
                               ids, p.n, p.v, nk, p.nchunks, p.ntg, sc.c2, part, upart, zsel,
                               n_bad_ids);
        };
        if (p.entropy) {
            if (p.nb == 1) gon(lmhead_narrow_kernel<true, 1>);
            else if (p.nb == 2) gon(lmhead_narrow_kernel<true, 2>);
            else gon(lmhead_narrow_kernel<true, 4>);
        } else {
            if (p.nb == 1) gon(lmhead_narrow_kernel<false, 1>);
            else if (p.nb == 2) gon(lmhead_narrow_kernel<false, 2>);
            else gon(lmhead_narrow_kernel<false, 4>);
        }
    } else if (p.dtype == 0) {
        if (p.chunk_tiles != 1) return hipErrorInvalidValue;   // one tile per chunk
        if (p.ksplit > 1) {
            float* slog = (float*)((unsigned char*)workspace + p.slog_off);
            if (grid * p.ksplit > INT32_MAX) return hipErrorInvalidValue;
            hipLaunchKernelGGL((lmhead8w_kernel<false, true>), dim3((unsigned)(grid * p.ksplit)),
                               dim3(2 * kThreads), 0, st, (const unsigned char*)h, ldh * esz,
                               (const unsigned char*)w, ldw * esz, ids, p.n, p.v, nk / p.ksplit,
                               p.nchunks, p.nttiles, sc.c2, part, upart, zsel, n_bad_ids, slog);
            hipLaunchKernelGGL(splitk_combine_kernel, dim3((unsigned)p.nchunks,
                               (unsigned)((p.n + 63) / 64)), dim3(64), 0, st, slog, p.ksplit, ids,
                               p.n, p.v, sc.c2, part, zsel);
            return hipGetLastError();
        }
        auto go8 = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(2 * kThreads), 0, st,
                               (const unsigned char*)h, ldh * esz, (const unsigned char*)w, ldw * esz,
                               ids, p.n, p.v, nk, p.nchunks, p.nttiles, sc.c2, part, upart, zsel,
                               n_bad_ids, (float*)nullptr);
        };
        if (p.entropy) go8(lmhead8w_kernel<true>);
        else go8(lmhead8w_kernel<false>);
    } else {
        if (p.chunk_tiles != 1) return hipErrorInvalidValue;   // one tile per chunk
        if (p.entropy) go(lmhead_partials_kernel<true>);
        else go(lmhead_partials_kernel<false>);
    }
    return hipGetLastError();
}

hipError_t launch_f32_gemm(const F32Gemm& g, hipStream_t st) {
    if (g.m <= 0 || g.n <= 0 || g.k <= 0 || g.k % 32 != 0) return hipErrorInvalidValue;
    const int64_t mtiles = (g.m + kTileV - 1) / kTileV, ntiles = (g.n + kTileT - 1) / kTileT;
    const int64_t grid = mtiles * ntiles;
    if (grid > INT32_MAX || g.k / 32 > INT32_MAX) return hipErrorInvalidValue;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, st,
                           (const unsigned char*)g.b, g.ldb * 4, (const unsigned char*)g.a,
                           g.lda * 4, g.ids, g.n, g.m, (int)(g.k / 32), 1, mtiles, mtiles, ntiles,
                           kLog2e, (float2*)nullptr, (float*)nullptr, (float*)nullptr,
                           (int32_t*)nullptr, g.ep);
    };
    if (g.mode == kF32Dz) go(lmhead_partials_kernel<false, kF32Dz>);
    else if (g.mode == kF32Store) go(lmhead_partials_kernel<false, kF32Store>);
    else if (g.mode == kF32StoreAcc) go(lmhead_partials_kernel<false, kF32StoreAcc>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_lse_merge(const LogprobPlan& p, const int32_t* ids, const ScoreScale& sc,
                            const void* workspace, float* logp, float* lse, float* entropy,
                            int32_t* n_bad_ids, hipStream_t st) {
    const float2* part = (const float2*)workspace;
    const float* zsel = (const float*)((const unsigned char*)workspace + p.zsel_off);
    const float* upart = p.entropy ? (const float*)((const unsigned char*)workspace + p.upart_off)
                                   : nullptr;
    // small batches: one block per token, every chunk pair staged in LDS
    const size_t token_lds = (size_t)p.nchunks * (sizeof(float2) + (p.entropy ? sizeof(float) : 0));
    if (p.narrow && token_lds <= kMergeTokenLdsMax) {
        auto gt = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3((unsigned)p.n), dim3(512), token_lds, st, part, upart,
                               zsel, ids, p.n, p.nchunks, p.v, sc.c2, sc.it, logp, lse, entropy,
                               n_bad_ids);
        };
        if (p.entropy) gt(lse_merge_token_kernel<true>);
        else gt(lse_merge_token_kernel<false>);
        return hipGetLastError();
    }
    const int64_t blocks = (p.n + 63) / 64;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * kMergeWaves), 0, st, part, upart,
                           zsel, ids, p.n, p.nchunks, p.v, sc.c2, sc.it, logp, lse, entropy,
                           n_bad_ids);
    };
    if (p.entropy) {
        if (p.narrow) go(lse_merge_kernel<true, true>);
        else go(lse_merge_kernel<true, false>);
    } else {
        if (p.narrow) go(lse_merge_kernel<false, true>);
        else go(lse_merge_kernel<false, false>);
    }
    return hipGetLastError();
}

}  // namespace tim
