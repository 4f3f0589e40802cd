// bwd.hip — backward of the selected-token log-probability, and the PPO /
// GRPO clipped surrogate, for gfx950.
//
// Backward ("RL: Training Inference Mismatch", the "log p" chain,
// differentiated; its importance-sampling section's policy-gradient term is
// g_t grad log q_t).  With logp_t = z_t[a_t] - log sum_v exp z_t[v], z_t = W h_t
// and an upstream gradient g_t = dL/dlogp_t:
//     dz[t, v] = g_t ([v == a_t] - p_t[v]),  p_t = softmax(z_t)
//     dh = dz W           (K = vocabulary, ascending)
//     dW = dz^T h         (K = tokens, ascending)
// bf16 operands, fp32 accumulation; dz is rounded to bf16 once (as the
// logits' gradient enters a bf16 GEMM in a bf16 trainer).  Steps:
//   1. gemm8w<kEpiDz>: the logits of a 256 x 256 (vocabulary x token) tile,
//      recomputed as the bf16 forward forms them (16x16x32 MFMAs, same
//      operand order, ascending K from zero, fp32 accumulation); the
//      epilogue forms dz with the forward's lse and writes it twice, as
//      dz^T [Vp][Np] and dz [Np][Vp] (bf16, zero outside V x N; Vp, Np =
//      V, N rounded up to multiples of 64), so no transpose of dz is needed.
//   2. transpose_bf16: W^T [D][Vp] (zero-padded); gemm8w<kEpiStore>:
//      dh[t, d] = sum_v dz[t, v] W^T[d, v].
//   3. transpose_bf16: h^T [D][Np]; gemm8w<kEpiStore>:
//      dW[v, d] = sum_t dz^T[v, t] h^T[d, t].
// Every output element is one fp32 MFMA accumulator chain in ascending K, no
// split-K, no atomics: dh's row t depends only on token t (batch invariant),
// and dW in accumulate mode continues the chain from the stored value, so
// micro-batches of whole 64-token stages summed one after another give the
// bits of one batch.
//
// Surrogate ("Diagnosing Training Inference Mismatch ... (VeXact)", eq. (2)
// clipped surrogate, eq. (3) recompute / bypass ratios, eq. (5) zero-centred
// contribution; its compensation table's TIS rows: the truncated r_corr
// weight): per token loss = -w min(r A, clip(r, 1 - eps_lo, 1 + eps_hi) A),
// its derivative by logp, -w [unclipped] r A, scaled to the token mean.

#include "mfma_pipe.h"

#include <math.h>

namespace tim {
namespace {

using namespace mfma;

// ---------------------------------------------------------------------------
// Transpose of a bf16 matrix with zero padding
// ---------------------------------------------------------------------------

constexpr int kTrTile = 64;
constexpr int kTrThreads = 256;

// out[c][r] = in[r][c] for r < rows, c < cols; out[c][r] = 0 for
// rows <= r < out_cols.  T: uint16_t (bf16) or uint32_t (fp32); kV = 16 /
// sizeof(T) elements move in every global access.  Grid: (out_cols / 64,
// ceil(cols / 64)).  A thread loads kV consecutive elements of an input row
// into the LDS tile, then gathers kV consecutive rows of one tile column and
// stores them as kV consecutive elements of an output row.  Requires
// cols % kV == 0, out_cols % 64 == 0, in, out, ld_in and ld_out 16-byte
// aligned (in elements: multiples of kV), which the backward's operands
// meet (D % 64 == 0, 16-byte aligned rows, padded sizes).
template <typename T>
__global__ void __launch_bounds__(kTrThreads)
transpose_kernel(const T* __restrict__ in, int64_t ld_in, int64_t rows, int64_t cols,
                 T* __restrict__ out, int64_t ld_out, int64_t out_cols) {
    constexpr int kV = 16 / (int)sizeof(T);
    constexpr int kG = kTrTile / kV;             // kV-element groups per tile row
    constexpr int kRows = kTrThreads / kG;       // tile rows per pass
    constexpr int kPitch = kTrTile + kV;         // LDS row pitch: rows stay 16-byte aligned
    __shared__ __attribute__((aligned(16))) T tile[kTrTile][kPitch];
    const int64_t r0 = (int64_t)blockIdx.x * kTrTile, c0 = (int64_t)blockIdx.y * kTrTile;
    const int g = threadIdx.x % kG;
    const int q = threadIdx.x / kG;
#pragma unroll
    for (int k = 0; k < kTrTile / kRows; ++k) {
        const int lr = q + kRows * k;
        const int64_t r = r0 + lr, c = c0 + g * kV;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < rows && c < cols) v = *(const uint4*)(in + r * ld_in + c);
        *(uint4*)&tile[lr][g * kV] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTrTile / kRows; ++k) {
        const int lc = q + kRows * k;                  // tile column = output row
        const int64_t c = c0 + lc, r = r0 + g * kV;    // output row, first output column
        T e[kV];
#pragma unroll
        for (int j = 0; j < kV; ++j) e[j] = tile[g * kV + j][lc];
        if (c < cols && r < out_cols) {
            uint4 o;
            __builtin_memcpy(&o, e, 16);
            *(uint4*)(out + c * ld_out + r) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// NT GEMM tile kernel: C[m][n] = sum_k A[m][k] B[n][k], bf16, fp32 accumulate
// ---------------------------------------------------------------------------

// kEpiStore(Acc): C[m][n], a lane holding four consecutive n of one m;
// kEpiStoreT(Acc): C stored transposed, out[n][m], a lane holding four
// consecutive m of one n.  Acc: the chain continues from the stored value.
enum { kEpiDz = 0, kEpiStore = 1, kEpiStoreAcc = 2, kEpiStoreT = 3, kEpiStoreTAcc = 4 };

struct GemmArgs {
    const unsigned char* a; int64_t lda_b; int64_t m;   // A: m rows, K contiguous (bytes)
    // B: n rows, K contiguous; or, K-major kernels, [K][n] with row pitch
    // ldb_b bytes, rows k >= bk_rows read as zero
    const unsigned char* b; int64_t ldb_b; int64_t n;
    int64_t bk_rows;
    int nk;                                             // K / 64 stages
    int64_t mtiles, ntiles;
    // kEpiStore, kEpiStoreAcc: c 16-byte aligned, ldc and n multiples of 4
    float* c; int64_t ldc;
    // kEpiDz (A = W, B = h): logits of valid rows m < vtrue, n < ntrue
    const float* lse; const float* g; const int32_t* ids;
    int64_t vtrue, ntrue;
    uint16_t* dzt; int64_t lddz;                        // dz^T [Vp][Np], or null
    uint16_t* dz; int64_t ldz;                          // dz [Np][Vp], or null
    int64_t vpad, npad;
};

// Round a finite fp32 to bf16, nearest, ties to even.
__device__ __forceinline__ uint16_t bf16_rne(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

// XCD-aware order: each XCD gets a contiguous range of logical tiles, walked
// as groups of kGroupM row tiles by all column tiles, so the workgroups
// resident on one XCD share operand stages in its L2.  Only who computes a
// tile changes, never how.
constexpr int kGroupM = 4;
__device__ __forceinline__ void gemm_tile_of_block(int64_t mtiles, int64_t ntiles, int64_t& mt,
                                                   int64_t& nt) {
    const int64_t G = gridDim.x, b = blockIdx.x;
    const int64_t per = G >> 3, rem = G & 7, x = b & 7, i = b >> 3;
    const int64_t L = x * per + (x < rem ? x : rem) + i;
    const int64_t span = (int64_t)kGroupM * ntiles;
    const int64_t group = L / span;
    const int64_t first = group * kGroupM;
    const int64_t gm = mtiles - first < kGroupM ? mtiles - first : kGroupM;
    const int64_t within = L - group * span;
    mt = first + within % gm;
    nt = within / gm;
}

// Eight waves, two per SIMD, as the bf16 head kernel (its pipeline without
// the walk over vocabulary tiles): one 256 x 256 tile of C per workgroup;
// wave w owns A rows (w & 1) * 128 .. + 127 and B rows (w >> 1) * 64 .. + 63
// of the tile as 8 x 4 blocks of 16 x 16 (acc[bi][bj], 128 accumulator
// registers); 16x16x32 MFMAs, two k-steps per 128-byte stage, A of stage
// s + 1 and B of stage s + 2 copied while stage s computes, four copies of
// each per wave per stage.
//
// kEpiDz gives the MFMAs the operands in the head kernel's order (A = W
// fragments first, same K order from zero), so the recomputed logits are
// the ones the forward formed; a lane then holds rows 4 grp + i of column
// col of each block.  kEpiStore(Acc) swap the two sources (B fragments
// first), so that a lane holds four consecutive columns 4 grp .. 4 grp + 3
// of row col: one 16-byte store (and load) per block; kEpiStoreT(Acc) keep
// the order and store the block transposed, four consecutive rows of one
// column in one 16-byte store.
//
// kBT: B is stored K-major ([K][n], n contiguous: W itself for dh, dz for
// dW), so no transposed copy of it is needed.  A stage of it is 64 K rows
// of the tile's 256 columns (512 bytes each), copied two rows per
// buffer-to-LDS copy; the 32-byte column blocks of row r are XOR-swizzled
// with (r & 3) | ((r >> 3) & 1) << 2, so the eight rows that one half-wave
// of a transposing read touches land on eight distinct 32-byte bank groups.
// A fragment is two ds_read_b64_tr_b16 (lds_read_tr), which hand each lane the
// same eight K values of its column that the K-contiguous read hands it:
// the MFMAs, and so the results, are the same bit for bit.  Each fragment
// costs two LDS reads instead of one, so the waits count 7 A reads + 8 B
// reads (15, the largest lgkmcnt) where the K-contiguous kernel counts 11.
template <int kEpi, bool kBT = false>
__global__ void __launch_bounds__(2 * kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
gemm8w_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    constexpr bool kSwap = kEpi == kEpiStore || kEpi == kEpiStoreAcc;
    constexpr bool kStoreT = kEpi == kEpiStoreT || kEpi == kEpiStoreTAcc;
    constexpr int kWaitFull = kBT ? 15 : 11;     // 7 A reads + 4 B fragments

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wv = wave & 1;        // A half of the tile (128 rows)
    const int wt = wave >> 1;       // B quarter of the tile (64 rows)
    const int col = lane & 15;
    const int grp = lane >> 4;

    int64_t mt, nt;
    gemm_tile_of_block(p.mtiles, p.ntiles, mt, nt);
    // uniform tile indices keep the buffer descriptors in scalar registers
    const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)mt) * kTileV;
    const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((int)nt) * kTileT;
    const int64_t mw = m0 + wv * 128;     // first A row (row of C) of this wave
    const int64_t nw = n0 + wt * 64;      // first B row (column of C) of this wave
    const int nk = p.nk;

    f32x4 acc[8][4];
    if constexpr (kEpi == kEpiStoreTAcc) {
        // transposed layout: rows mw + bi 16 + 4 grp .. + 3 of column
        // nw + bj 16 + col are out[col][..]: one 16-byte load (m is a
        // multiple of 4)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t cn = nw + bj * 16 + col;
            const float* crow = p.c + (cn < p.n ? cn : 0) * p.ldc;
#pragma unroll
            for (int bi = 0; bi < 8; ++bi) {
                const int64_t r0 = mw + bi * 16 + grp * 4;
                float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
                if (cn < p.n && r0 < p.m) q = *(const float4*)(crow + r0);
                acc[bi][bj] = f32x4{q.x, q.y, q.z, q.w};
                asm volatile("" : "+a"(acc[bi][bj]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else if constexpr (kEpi == kEpiStoreAcc) {
        // the chain continues from the stored value (swapped layout: row
        // mw + bi 16 + col, columns nw + bj 16 + 4 grp .. + 3: one 16-byte
        // load; n is a multiple of 4)
#pragma unroll
        for (int bi = 0; bi < 8; ++bi) {
            const int64_t row = mw + bi * 16 + col;
            const float* crow = p.c + (row < p.m ? row : 0) * p.ldc;
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t c0 = nw + bj * 16 + grp * 4;
                float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
                if (row < p.m && c0 < p.n) q = *(const float4*)(crow + c0);
                acc[bi][bj] = f32x4{q.x, q.y, q.z, q.w};
                // into the accumulator registers now, not held in VGPRs
                asm volatile("" : "+a"(acc[bi][bj]));
            }
            // a few loads in flight at a time, not all 128 at once
            if (bi & 1) __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int bi = 0; bi < 8; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Copies: wave `wave` fills 8-row blocks 4 wave .. 4 wave + 3 of both
    // operand tiles (swizzled chunks); rows past m or n are redirected to the
    // last valid row (results discarded), so every access lies inside the
    // operands and inside the descriptors' extents.
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int drow = (wave * 4 + j) * 8 + (lane >> 3);
        const uint32_t cb = (uint32_t)(((lane & 7) ^ ((drow >> 1) & 7)) * 16);
        int64_t ra = m0 + drow, rb = n0 + drow;
        if (ra > p.m - 1) ra = p.m - 1;
        if (rb > p.n - 1) rb = p.n - 1;
        aoff[j] = (uint32_t)((ra - m0) * p.lda_b) + cb;
        if constexpr (kBT) {
            // K-major B: copy j of this wave holds stage rows 2 u, 2 u + 1
            // (u = 4 wave + j); lane l writes 16 bytes at l 16, i.e. row
            // 2 u + (l >> 5), physical 32-byte block (l & 31) >> 1, which
            // holds the logical block that the swizzle maps there
            const int r = 2 * (wave * 4 + j) + (lane >> 5);
            const int f = (r & 3) | (((r >> 3) & 1) << 2);
            const int lb = ((lane & 31) >> 1) ^ f;
            boff[j] = (uint32_t)(r * p.ldb_b) + (uint32_t)(lb * 32 + (lane & 1) * 16);
        } else {
            boff[j] = (uint32_t)((rb - n0) * p.ldb_b) + cb;
        }
    }
    const int64_t arows = (p.m - m0) < kTileV ? (p.m - m0) : kTileV;
    const int64_t brows = (p.n - n0) < kTileT ? (p.n - n0) : kTileT;
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.a + m0 * p.lda_b), (short)0,
        (int)((arows - 1) * p.lda_b + (int64_t)nk * kStageBytes), kRsrcWord3);
    // K-contiguous B: one descriptor for the tile's rows over all of K.
    // K-major B: one per stage (rebuilt in advance_b), over that stage's 64
    // rows and the tile's columns: rows past bk_rows and columns past n at
    // the last valid row lie outside it and read as zero, and no offset
    // grows with K (a [K][n] operand can exceed 4 GiB)
    auto b_stage_rsrc = [&](int kb) {
        const int64_t k0 = (int64_t)kb * 64;
        const int64_t nval = p.bk_rows - k0;
        int64_t ext = 0;
        // the range check is per dword (a dword that straddles the end
        // reads as zero): the last row's extent is rounded up to whole
        // dwords, which stays inside that row (dz rows are padded to 64
        // entries; W rows hold D, a multiple of 64)
        if (nval > 0) ext = ((nval < 64 ? nval : 64) - 1) * p.ldb_b + ((brows * 2 + 3) & ~(int64_t)3);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(p.b + k0 * p.ldb_b + n0 * 2), (short)0,
                                                 (int)ext, kRsrcWord3);
    };
    __amdgpu_buffer_rsrc_t brs;
    if constexpr (kBT)
        brs = b_stage_rsrc(0);
    else
        brs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.b + n0 * p.ldb_b), (short)0,
            (int)((brows - 1) * p.ldb_b + (int64_t)nk * kStageBytes), kRsrcWord3);

    // fragment addresses: row col of a 16-row block, logical chunk ks 4 + grp
    const uint32_t lds_base = lds_addr(lds);
    const uint32_t kofs0 = (uint32_t)swz(col, 0 * 4 + grp);
    const uint32_t kofs1 = (uint32_t)swz(col, 1 * 4 + grp);
    const uint32_t a_half = (uint32_t)(wv * 128 * kStageBytes);
    const uint32_t b_quarter = (uint32_t)(wt * 64 * kStageBytes);

    int a_kb = 0, b_kb = 0;
    auto copy_a = [&](int j, int pos) {
        dma16_buf(ars, lds + pos * kOperandBytes + (wave * 4 + j) * 1024, aoff[j],
                  (uint32_t)(a_kb * kStageBytes));
    };
    auto copy_b = [&](int j, int pos) {
        dma16_buf(brs, lds + pos * kOperandBytes + (wave * 4 + j) * 1024, boff[j],
                  kBT ? 0u : (uint32_t)(b_kb * kStageBytes));
    };
    auto advance_a = [&]() { if (++a_kb == nk) a_kb = 0; };
    auto advance_b = [&]() {
        if (++b_kb == nk) b_kb = 0;
        if constexpr (kBT) brs = b_stage_rsrc(b_kb);
    };
    auto next_pos = [](int q) { return q + 2 >= kPos ? q + 2 - kPos : q + 2; };

    // K-major B fragments: lane (g = l >> 4, p = l & 15) addresses stage
    // row 8 g + (p >> 2) (+ 4 for the upper four K, + 32 for k-step 1) at
    // the swizzled block of column block 4 wt + bj, 8 bytes at 4 (p & 3)
    uint32_t xb[4];
    if constexpr (kBT) {
        const int tg = lane >> 4, tq = (lane & 15) >> 2;
        const uint32_t f = (uint32_t)(tq | ((tg & 1) << 2));
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
            xb[bj] = (uint32_t)((8 * tg + tq) * 512) + ((((uint32_t)(4 * wt + bj)) ^ f) << 5) +
                     (uint32_t)((lane & 3) << 3);
    }
    u32x4 A[8], B0[4], B1[4];
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
    // base: the B ring position (K-major) or that plus the wave's quarter
    // and the k-step's chunk (K-contiguous); ks: the k-step (K-major only)
    auto read_b = [&](u32x4 (&B)[4], uint32_t base, auto ks) {
        if constexpr (kBT) {
            constexpr int o = decltype(ks)::value * 16384;
            lds_read_tr<o>(B[0], base + xb[0]);
            lds_read_tr<o>(B[1], base + xb[1]);
            lds_read_tr<o>(B[2], base + xb[2]);
            lds_read_tr<o>(B[3], base + xb[3]);
        } else {
            lds_read16<0 * 2048>(B[0], base);
            lds_read16<1 * 2048>(B[1], base);
            lds_read16<2 * 2048>(B[2], base);
            lds_read16<3 * 2048>(B[3], base);
        }
    };
    auto wait_b = [&](auto n, u32x4& a, u32x4 (&B)[4]) { wait16_4<decltype(n)::value>(a, B); };
    // tied-accumulator asm MFMAs (mfma_pipe.h); kEpiStore(Acc) swap the
    // sources
    auto mfma = [&](int r, int bj, const u32x4& b) {
        if constexpr (kSwap) mfma16_tied(acc[r][bj], b, A[r]);
        else mfma16_tied(acc[r][bj], A[r], b);
    };
    auto mfma_last = [&](const u32x4& b, int last) {
        if constexpr (kSwap) mfma16_tied_last(acc[7][3], b, A[7], last);
        else mfma16_tied_last(acc[7][3], A[7], b, last);
    };
    const uint32_t bsel0 = kBT ? 0u : b_quarter + kofs0;   // added to the ring position
    const uint32_t bsel1 = kBT ? 0u : b_quarter + kofs1;

    // kEpiDz: the per-token inputs of the epilogue, loaded before the K loop
    // so that their latency is hidden behind it
    float tok_g[4], tok_l[4];
    int32_t tok_a[4];
    if constexpr (kEpi == kEpiDz) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t t = nw + bj * 16 + col;
            const bool tv = t < p.ntrue;
            const int64_t tc = tv ? t : 0;
            tok_g[bj] = tv ? p.g[tc] : 0.f;
            tok_l[bj] = tv ? p.lse[tc] : 0.f;
            tok_a[bj] = tv ? p.ids[tc] : -1;
        }
    }

    // Ring positions (2 stage + op) % 5, op 0: B, op 1: A.  LDS reads of a
    // wave complete in order; the waits count the reads issued after the
    // one a row needs: 11 for every ks0 row, 7 - r for ks1 rows 0-3.
    int rd_b = 0, rd_a = 1;
    int cp_a = 3, cp_b = 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_b(j, 0);
    advance_b();
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_a(j, 1);
    advance_a();
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_b(j, 2);
    advance_b();
    wait_vmcnt<4>();
    __syncthreads();
    {
        const uint32_t aw = lds_base + (uint32_t)(rd_a * kOperandBytes) + a_half;
        const uint32_t bw = lds_base + (uint32_t)(rd_b * kOperandBytes);
        read_b(B0, bw + bsel0, IntConst<0>{});
#pragma unroll
        for (int r = 0; r < 8; ++r) read_a(r, aw + kofs0);
    }

    for (int kb = 0; kb < nk; ++kb) {
        const uint32_t aw = lds_base + (uint32_t)(rd_a * kOperandBytes) + a_half;
        const uint32_t bw = lds_base + (uint32_t)(rd_b * kOperandBytes);
        // ---- ks0: A(s+1) copies at rows 0-3
        read_b(B1, bw + bsel1, IntConst<1>{});
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r == 0) wait_b(IntConst<kWaitFull>{}, A[0], B0);
            else wait16<kWaitFull>(A[r]);
            mfma(r, 0, B0[0]); mfma(r, 1, B0[1]);
            if (r < 4) copy_a(r, cp_a);
            mfma(r, 2, B0[2]); mfma(r, 3, B0[3]);
            read_a(r, aw + kofs1);
        }
        advance_a();
        // ---- ks1, rows 0-3: B(s+2) copies
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r == 0) wait_b(IntConst<7>{}, A[0], B1);
            else if (r == 1) wait16<6>(A[1]);
            else if (r == 2) wait16<5>(A[2]);
            else wait16<4>(A[3]);
            mfma(r, 0, B1[0]); mfma(r, 1, B1[1]);
            copy_b(r, cp_b);
            mfma(r, 2, B1[2]); mfma(r, 3, B1[3]);
        }
        // stage + 1 resident (this wave's copies, then everyone's) and every
        // read of this stage done before its slots are reused
        wait_vmcnt<4>();
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(A[4]), "+v"(A[5]), "+v"(A[6]), "+v"(A[7]));
        asm volatile("s_barrier" ::: "memory");
        rd_b = next_pos(rd_b);
        rd_a = next_pos(rd_a);
        const uint32_t aw2 = lds_base + (uint32_t)(rd_a * kOperandBytes) + a_half;
        const uint32_t bw2 = lds_base + (uint32_t)(rd_b * kOperandBytes);
        read_b(B0, bw2 + bsel0, IntConst<0>{});
#pragma unroll
        for (int r = 0; r < 4; ++r) read_a(r, aw2 + kofs0);
        // ---- ks1, rows 4-7
#pragma unroll
        for (int r = 4; r < 8; ++r) {
            wait16<kWaitFull>(A[r]);
            mfma(r, 0, B1[0]); mfma(r, 1, B1[1]); mfma(r, 2, B1[2]);
            if (r < 7) mfma(r, 3, B1[3]);
            else mfma_last(B1[3], __builtin_amdgcn_readfirstlane(kb == nk - 1));   // + epilogue wait
            read_a(r, aw2 + kofs0);
        }
        advance_b();
        cp_a = next_pos(cp_a);
        cp_b = next_pos(cp_b);
    }
    // drain: the look-ahead reads and the extra copies (the LDS must be
    // quiet before the workgroup ends)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(A[0]), "+v"(A[1]), "+v"(A[2]), "+v"(A[3]),
                 "+v"(A[4]), "+v"(A[5]), "+v"(A[6]), "+v"(A[7]));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(B0[0]), "+v"(B0[1]), "+v"(B0[2]), "+v"(B0[3]));
    wait_vmcnt<0>();

    if constexpr (kStoreT) {
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int col_e = lane_e & 15, grp_e = lane_e >> 4;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t cn = nw + bj * 16 + col_e;
            if (cn >= p.n) continue;
            float* crow = p.c + cn * p.ldc;
#pragma unroll
            for (int bi = 0; bi < 8; ++bi) {
                const int64_t r0 = mw + bi * 16 + grp_e * 4;
                if (r0 < p.m)
                    *(float4*)(crow + r0) = make_float4(acc[bi][bj][0], acc[bi][bj][1],
                                                        acc[bi][bj][2], acc[bi][bj][3]);
            }
        }
    } else if constexpr (kEpi != kEpiDz) {
        // addresses formed anew (an opaque copy of the lane index): shared
        // with the loads above, they would stay live across the K loop
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int col_e = lane_e & 15, grp_e = lane_e >> 4;
#pragma unroll
        for (int bi = 0; bi < 8; ++bi) {
            const int64_t row = mw + bi * 16 + col_e;
            if (row >= p.m) continue;
            float* crow = p.c + row * p.ldc;
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t c0 = nw + bj * 16 + grp_e * 4;
                if (c0 < p.n)
                    *(float4*)(crow + c0) = make_float4(acc[bi][bj][0], acc[bi][bj][1],
                                                        acc[bi][bj][2], acc[bi][bj][3]);
            }
        }
    } else {
        // dz = g_t ([v == a_t] - exp(z - lse_t)) for v < V, t < N; 0 in the
        // padding (rows V..Vp-1, columns N..Np-1); an id outside [0, V)
        // contributes nothing.  A lane holds dz[t][v0 .. v0 + 3] of each
        // block: written to dz^T one element per row and to dz as one
        // 8-byte store (v0 is a multiple of 4 and Vp of 64).
        // Branch-free per element: rows past V of the tile hold finite
        // logits of a clamped row, and their dz is selected away.
        const int32_t vtrue = (int32_t)p.vtrue;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t t = nw + bj * 16 + col;
            const bool tv = t < p.ntrue;
            const float g = tok_g[bj], l = tok_l[bj];
            const int32_t a = tok_a[bj];
            const bool ok = tv && a >= 0 && a < vtrue && g != 0.f;
            const bool t_in = t < p.npad;
#pragma unroll
            for (int bi = 0; bi < 8; ++bi) {
                const int32_t v0 = (int32_t)(mw + bi * 16 + grp * 4);   // < 2^31 (V < 2^31)
                uint32_t q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t v = v0 + i;
                    const float pz = fast_exp2((acc[bi][bj][i] - l) * kLog2e);
                    const float dz = g * ((v == a ? 1.f : 0.f) - pz);
                    q[i] = (ok && v < vtrue) ? bf16_rne(dz) : 0u;
                }
                if (t_in && (int64_t)v0 < p.vpad) {
                    if (p.dzt) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) p.dzt[(v0 + i) * p.lddz + t] = (uint16_t)q[i];
                    }
                    if (p.dz)
                        *(uint2*)(p.dz + t * p.ldz + v0) = make_uint2(q[0] | (q[1] << 16),
                                                                      q[2] | (q[3] << 16));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// PPO / GRPO surrogate
// ---------------------------------------------------------------------------

constexpr int kPpoThreads = 256;
constexpr int kPpoMaxBlocks = 16384;
constexpr int kPpoGroup = 4;         // consecutive tokens per thread step: one 16-byte access
constexpr int kPpoUnroll = 2;        // groups per thread per loop trip, loads first

struct PpoPart {
    double loss, ratio, w, contrib;
    uint64_t nvalid, nclip, nnan, pad;
};

struct PpoArgs {
    const float *logp, *old_train, *old_rollout, *adv;
    const uint8_t* mask;
    int64_t n;
    double eps_lo, eps_hi, tis_c;
    double gscale;                   // > 0: gradient of gscale * sum; 0: unscaled (rescaled later)
    int bypass;
    float *loss, *grad, *ratio, *contrib;
    uint8_t* clipped;
};

struct PpoTok {
    float l, g, r, c;
    uint32_t clip;
};

// One token, fp64 from the fp32 inputs.
__device__ __forceinline__ PpoTok ppo_token(const PpoArgs& a, float lp, float ot, float orr,
                                            float ad, bool in, PpoPart& acc) {
    double l_t = 0, g_t = 0, r_t = 1, c_t = 0;
    uint32_t clip_t = 0;
    if (in) {
        const double old = a.bypass ? (double)orr : (double)ot;
        const double r = exp((double)lp - old);
        const double w = a.tis_c > 0.0 ? fmin(exp((double)ot - (double)orr), a.tis_c) : 1.0;
        const double adv = (double)ad;
        if (!isfinite(r) || !isfinite(w) || !isfinite(adv)) {
            acc.nnan++;
        } else {
            const double hi = 1.0 + a.eps_hi, lo = 1.0 - a.eps_lo;
            const double rc = r < lo ? lo : (r > hi ? hi : r);
            const double sur = fmin(r * adv, rc * adv);
            const bool active = (adv > 0.0 && r > hi) || (adv < 0.0 && r < lo);
            l_t = -w * sur;
            g_t = active ? 0.0 : -w * r * adv;
            if (a.gscale > 0.0) g_t *= a.gscale;
            r_t = r;
            c_t = -(r - 1.0) * adv;
            clip_t = active;
            acc.nvalid++;
            acc.nclip += active;
            acc.loss += l_t;
            acc.ratio += r;
            acc.w += w;
            acc.contrib += c_t;
        }
    }
    return PpoTok{(float)l_t, (float)g_t, (float)r_t, (float)c_t, clip_t};
}

// Thread tid of block b takes token groups g = b*256 + tid + j*stride
// (stride = grid*256), kPpoUnroll groups per loop trip with every load of
// the trip issued first; group g is tokens 4g .. 4g + 3, folded in
// ascending order.  kVec: every pointer is 16-byte aligned (the mask and the
// clip flags 4-byte aligned), so a whole group moves with one access per
// array; otherwise, and for the last group when n % 4 != 0, element by
// element.  Both variants assign and fold tokens identically, so their bits
// agree.  Block partials are folded by a fixed tree.
template <bool kVec>
__global__ void __launch_bounds__(kPpoThreads)
ppo_token_kernel(PpoArgs a, PpoPart* __restrict__ part) {
    __shared__ PpoPart sh[kPpoThreads];
    PpoPart acc{0, 0, 0, 0, 0, 0, 0, 0};
    const int64_t ng = (a.n + kPpoGroup - 1) / kPpoGroup;
    const int64_t stride = (int64_t)gridDim.x * kPpoThreads;
    for (int64_t base = (int64_t)blockIdx.x * kPpoThreads + threadIdx.x; base < ng;
         base += kPpoUnroll * stride) {
        float4 lp[kPpoUnroll], ot[kPpoUnroll], orr[kPpoUnroll], ad[kPpoUnroll];
        uint32_t mk[kPpoUnroll];
#pragma unroll
        for (int j = 0; j < kPpoUnroll; ++j) {
            const int64_t g = base + j * stride;
            const int64_t gc = g < ng ? g : base;              // base < ng: in bounds
            const int64_t t0 = gc * kPpoGroup;
            if (kVec && t0 + kPpoGroup <= a.n) {
                lp[j] = *(const float4*)(a.logp + t0);
                ot[j] = *(const float4*)(a.old_train + t0);
                orr[j] = *(const float4*)(a.old_rollout + t0);
                ad[j] = *(const float4*)(a.adv + t0);
                mk[j] = a.mask ? *(const uint32_t*)(a.mask + t0) : 0x01010101u;
            } else {
                float x[4][4];
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < kPpoGroup; ++i) {
                    const int64_t t = t0 + i < a.n ? t0 + i : a.n - 1;
                    x[0][i] = a.logp[t];
                    x[1][i] = a.old_train[t];
                    x[2][i] = a.old_rollout[t];
                    x[3][i] = a.adv[t];
                    m |= (uint32_t)(a.mask ? a.mask[t] : 1) << (8 * i);
                }
                lp[j] = make_float4(x[0][0], x[0][1], x[0][2], x[0][3]);
                ot[j] = make_float4(x[1][0], x[1][1], x[1][2], x[1][3]);
                orr[j] = make_float4(x[2][0], x[2][1], x[2][2], x[2][3]);
                ad[j] = make_float4(x[3][0], x[3][1], x[3][2], x[3][3]);
                mk[j] = m;
            }
        }
#pragma unroll
        for (int j = 0; j < kPpoUnroll; ++j) {
            const int64_t g = base + j * stride;
            if (g >= ng) continue;
            const int64_t t0 = g * kPpoGroup;
            const float lpv[4] = {lp[j].x, lp[j].y, lp[j].z, lp[j].w};
            const float otv[4] = {ot[j].x, ot[j].y, ot[j].z, ot[j].w};
            const float orv[4] = {orr[j].x, orr[j].y, orr[j].z, orr[j].w};
            const float adv[4] = {ad[j].x, ad[j].y, ad[j].z, ad[j].w};
            PpoTok o[kPpoGroup];
#pragma unroll
            for (int i = 0; i < kPpoGroup; ++i) {
                const bool in = t0 + i < a.n && ((mk[j] >> (8 * i)) & 0xffu) != 0;
                o[i] = ppo_token(a, lpv[i], otv[i], orv[i], adv[i], in, acc);
            }
            if (kVec && t0 + kPpoGroup <= a.n) {
                if (a.loss) *(float4*)(a.loss + t0) = make_float4(o[0].l, o[1].l, o[2].l, o[3].l);
                if (a.grad) *(float4*)(a.grad + t0) = make_float4(o[0].g, o[1].g, o[2].g, o[3].g);
                if (a.ratio) *(float4*)(a.ratio + t0) = make_float4(o[0].r, o[1].r, o[2].r, o[3].r);
                if (a.contrib)
                    *(float4*)(a.contrib + t0) = make_float4(o[0].c, o[1].c, o[2].c, o[3].c);
                if (a.clipped)
                    *(uint32_t*)(a.clipped + t0) =
                        o[0].clip | (o[1].clip << 8) | (o[2].clip << 16) | (o[3].clip << 24);
            } else {
#pragma unroll
                for (int i = 0; i < kPpoGroup; ++i) {
                    const int64_t t = t0 + i;
                    if (t >= a.n) break;
                    if (a.loss) a.loss[t] = o[i].l;
                    if (a.grad) a.grad[t] = o[i].g;
                    if (a.ratio) a.ratio[t] = o[i].r;
                    if (a.contrib) a.contrib[t] = o[i].c;
                    if (a.clipped) a.clipped[t] = (uint8_t)o[i].clip;
                }
            }
        }
    }
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kPpoThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            PpoPart& x = sh[threadIdx.x];
            const PpoPart& y = sh[threadIdx.x + s];
            x.loss += y.loss; x.ratio += y.ratio; x.w += y.w; x.contrib += y.contrib;
            x.nvalid += y.nvalid; x.nclip += y.nclip; x.nnan += y.nnan;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

// One block: blocks' partials folded in a fixed tree; the batch vector.
__global__ void __launch_bounds__(kPpoThreads)
ppo_final_kernel(const PpoPart* __restrict__ part, int nblk, double* __restrict__ batch,
                 double* __restrict__ inv_n) {
    __shared__ PpoPart sh[kPpoThreads];
    PpoPart acc{0, 0, 0, 0, 0, 0, 0, 0};
    for (int b = threadIdx.x; b < nblk; b += kPpoThreads) {
        const PpoPart& y = part[b];
        acc.loss += y.loss; acc.ratio += y.ratio; acc.w += y.w; acc.contrib += y.contrib;
        acc.nvalid += y.nvalid; acc.nclip += y.nclip; acc.nnan += y.nnan;
    }
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int s = kPpoThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            PpoPart& x = sh[threadIdx.x];
            const PpoPart& y = sh[threadIdx.x + s];
            x.loss += y.loss; x.ratio += y.ratio; x.w += y.w; x.contrib += y.contrib;
            x.nvalid += y.nvalid; x.nclip += y.nclip; x.nnan += y.nnan;
        }
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    const PpoPart& s = sh[0];
    const double nv = (double)s.nvalid;
    auto dv = [](double x, double y) { return y != 0.0 ? x / y : 0.0; };
    if (batch) {
        batch[kPpoOutMeanLoss] = dv(s.loss, nv);
        batch[kPpoOutClipFrac] = dv((double)s.nclip, nv);
        batch[kPpoOutMeanRatio] = dv(s.ratio, nv);
        batch[kPpoOutMeanTisW] = dv(s.w, nv);
        batch[kPpoOutMeanContrib] = dv(s.contrib, nv);
        batch[kPpoOutNValid] = nv;
        batch[kPpoOutNClipped] = (double)s.nclip;
        batch[kPpoOutNNan] = (double)s.nnan;
    }
    *inv_n = nv > 0 ? 1.0 / nv : 0.0;
}

// grad[t] *= 1 / n_valid (the derivative of the token mean); kVec: grad is
// 16-byte aligned and moves four values per access (the last n % 4 one by
// one).  The product is the same either way.
template <bool kVec>
__global__ void __launch_bounds__(kPpoThreads)
ppo_scale_kernel(float* __restrict__ grad, int64_t n, const double* __restrict__ inv_n) {
    const double s = *inv_n;
    const int64_t stride = (int64_t)gridDim.x * kPpoThreads;
    const int64_t tid = (int64_t)blockIdx.x * kPpoThreads + threadIdx.x;
    if constexpr (kVec) {
        const int64_t n4 = n / 4;
        for (int64_t i = tid; i < n4; i += stride) {
            float4 g = *(const float4*)(grad + 4 * i);
            g.x = (float)((double)g.x * s);
            g.y = (float)((double)g.y * s);
            g.z = (float)((double)g.z * s);
            g.w = (float)((double)g.w * s);
            *(float4*)(grad + 4 * i) = g;
        }
        if (tid < n - 4 * n4) grad[4 * n4 + tid] = (float)((double)grad[4 * n4 + tid] * s);
    } else {
        for (int64_t t = tid; t < n; t += stride) grad[t] = (float)((double)grad[t] * s);
    }
}

inline int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// x[0..n) = 0 (a kernel rather than a memset, so that a captured graph
// replays it like any other node)
__global__ void __launch_bounds__(256) fill_zero_kernel(float* __restrict__ x, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = 0.f;
}

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool make_backward_plan(int64_t n, int64_t d, int64_t v, int dtype, BackwardPlan* p) {
    if (n < 0 || d <= 0 || v <= 0 || v > INT32_MAX || n > INT32_MAX || (dtype != 0 && dtype != 1))
        return false;
    p->n = n; p->d = d; p->v = v; p->dtype = dtype;
    p->npad = round_up(n > 0 ? n : 1, 64);
    p->vpad = round_up(v, 64);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    if (dtype == 0) {
        p->wt_off = p->dzt_off = 0;                    // not used
        p->ht_off = take((size_t)d * p->npad * 2);
        p->dz_off = take((size_t)p->npad * p->vpad * 2);
    } else {
        p->wt_off = take((size_t)d * p->vpad * 4);
        p->ht_off = take((size_t)d * p->npad * 4);
        p->dzt_off = take((size_t)p->vpad * p->npad * 4);
        p->dz_off = take((size_t)p->npad * p->vpad * 4);
    }
    p->total_bytes = off;
    return true;
}

template <typename T>
static hipError_t launch_transpose(const T* in, int64_t ld_in, int64_t rows, int64_t cols, T* out,
                                   int64_t ld_out, int64_t out_cols, hipStream_t st) {
    constexpr int kV = 16 / (int)sizeof(T);
    const int64_t gx = (out_cols + kTrTile - 1) / kTrTile, gy = (cols + kTrTile - 1) / kTrTile;
    if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;
    if (cols % kV != 0 || out_cols % kTrTile != 0 || ld_in % kV != 0 || ld_out % kV != 0 ||
        (uintptr_t)in % 16 != 0 || (uintptr_t)out % 16 != 0)
        return hipErrorInvalidValue;                   // the kernel's 16-byte accesses
    hipLaunchKernelGGL(transpose_kernel<T>, dim3((unsigned)gx, (unsigned)gy), dim3(kTrThreads),
                       0, st, in, ld_in, rows, cols, out, ld_out, out_cols);
    return hipGetLastError();
}

static hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
    const int64_t grid = a.mtiles * a.ntiles;
    if (grid <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
    const dim3 block(2 * kThreads);
    if (epi == kEpiDz)
        hipLaunchKernelGGL((gemm8w_kernel<kEpiDz, false>), dim3((unsigned)grid), block, 0, st, a);
    else if (epi == kEpiStore)      // dh: B = W, K-major
        hipLaunchKernelGGL((gemm8w_kernel<kEpiStore, true>), dim3((unsigned)grid), block, 0, st, a);
    else if (epi == kEpiStoreT)     // dW: B = dz, K-major
        hipLaunchKernelGGL((gemm8w_kernel<kEpiStoreT, true>), dim3((unsigned)grid), block, 0, st, a);
    else
        hipLaunchKernelGGL((gemm8w_kernel<kEpiStoreTAcc, true>), dim3((unsigned)grid), block, 0, st,
                           a);
    return hipGetLastError();
}

// fp32 (the FP32 LM head's backward): the fp32 forward's tile kernel forms
// the logits with the forward's MFMA sequence and writes dz in fp32 in both
// layouts (no rounding: the head trains in fp32); W^T and h^T make the two
// products NT GEMMs of the same kernel.  Each output element is one fp32
// MFMA chain in ascending K, as in the bf16 path.
static hipError_t launch_backward_f32(const BackwardPlan& p, const float* h, int64_t ldh,
                                      const float* w, int64_t ldw, const int32_t* ids,
                                      const float* lse, const float* g, float* dh, float* dw,
                                      bool accumulate_dw, unsigned char* ws, hipStream_t st) {
    float* wt = (float*)(ws + p.wt_off);       // W^T [D][Vp]
    float* ht = (float*)(ws + p.ht_off);       // h^T [D][Np]
    float* dzt = (float*)(ws + p.dzt_off);     // dz^T [Vp][Np]
    float* dz = (float*)(ws + p.dz_off);       // dz [Np][Vp]
    hipError_t e;
    F32Gemm z{};
    z.mode = kF32Dz;
    z.a = w; z.lda = ldw; z.b = h; z.ldb = ldh; z.ids = ids;
    z.m = p.v; z.n = p.n; z.k = p.d;
    z.ep.lse = lse; z.ep.g = g;
    z.ep.dz = dh ? dz : nullptr; z.ep.ldz = p.vpad;
    z.ep.dzt = dw ? dzt : nullptr; z.ep.lddzt = p.npad;
    z.ep.vpad = p.vpad; z.ep.npad = p.npad;
    if ((e = launch_f32_gemm(z, st)) != hipSuccess) return e;
    if (dh) {
        // dh[t][d] = sum_v dz[t][v] W^T[d][v]
        if ((e = launch_transpose<uint32_t>((const uint32_t*)w, ldw, p.v, p.d, (uint32_t*)wt,
                                            p.vpad, p.vpad, st)) != hipSuccess)
            return e;
        F32Gemm a{};
        a.mode = kF32Store;
        a.a = dz; a.lda = p.vpad; a.b = wt; a.ldb = p.vpad;
        a.m = p.n; a.n = p.d; a.k = p.vpad;
        a.ep.c = dh; a.ep.ldc = p.d;
        if ((e = launch_f32_gemm(a, st)) != hipSuccess) return e;
    }
    if (dw) {
        // dW[v][d] = sum_t dz^T[v][t] h^T[d][t] (K = tokens, ascending)
        if ((e = launch_transpose<uint32_t>((const uint32_t*)h, ldh, p.n, p.d, (uint32_t*)ht,
                                            p.npad, p.npad, st)) != hipSuccess)
            return e;
        F32Gemm b{};
        b.mode = accumulate_dw ? kF32StoreAcc : kF32Store;
        b.a = dzt; b.lda = p.npad; b.b = ht; b.ldb = p.npad;
        b.m = p.v; b.n = p.d; b.k = p.npad;
        b.ep.c = dw; b.ep.ldc = p.d;
        if ((e = launch_f32_gemm(b, st)) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_logprob_backward(const BackwardPlan& p, const void* h, int64_t ldh,
                                   const void* w, int64_t ldw, const int32_t* ids,
                                   const float* lse, const float* g, float* dh, float* dw,
                                   bool accumulate_dw, void* workspace, hipStream_t st) {
    if (p.dtype == 1)
        return launch_backward_f32(p, (const float*)h, ldh, (const float*)w, ldw, ids, lse, g, dh,
                                   dw, accumulate_dw, (unsigned char*)workspace, st);
    unsigned char* ws = (unsigned char*)workspace;
    uint16_t* ht = (uint16_t*)(ws + p.ht_off);     // h^T [D][Np]
    uint16_t* dz = (uint16_t*)(ws + p.dz_off);     // dz [Np][Vp]
    hipError_t e;

    // 1. dz from the recomputed logits (A = W rows, B = h rows, K = D)
    GemmArgs z{};
    z.a = (const unsigned char*)w; z.lda_b = ldw * 2; z.m = p.v;
    z.b = (const unsigned char*)h; z.ldb_b = ldh * 2; z.n = p.n;
    z.nk = (int)(p.d / 64);
    z.mtiles = (p.vpad + kTileV - 1) / kTileV;
    z.ntiles = (p.npad + kTileT - 1) / kTileT;
    z.lse = lse; z.g = g; z.ids = ids; z.vtrue = p.v; z.ntrue = p.n;
    z.dzt = nullptr; z.lddz = 0;
    z.dz = dz; z.ldz = p.vpad;
    z.vpad = p.vpad; z.npad = p.npad;
    if ((e = launch_gemm(z, kEpiDz, st)) != hipSuccess) return e;

    if (dh) {
        // 2. dh = dz W (K = vocabulary; W read K-major, rows past V as zero)
        GemmArgs a{};
        a.a = (const unsigned char*)dz; a.lda_b = p.vpad * 2; a.m = p.n;
        a.b = (const unsigned char*)w; a.ldb_b = ldw * 2; a.n = p.d; a.bk_rows = p.v;
        a.nk = (int)(p.vpad / 64);
        a.mtiles = (p.n + kTileV - 1) / kTileV;
        a.ntiles = (p.d + kTileT - 1) / kTileT;
        a.c = dh; a.ldc = p.d;
        if ((e = launch_gemm(a, kEpiStore, st)) != hipSuccess) return e;
    }
    if (dw) {
        // 3. h^T, then dW^T = h^T dz computed as C[d][v] (K = tokens,
        //    ascending; dz read K-major) and stored transposed into dW[v][d]
        if ((e = launch_transpose<uint16_t>((const uint16_t*)h, ldh, p.n, p.d, ht, p.npad, p.npad, st)) != hipSuccess)
            return e;
        GemmArgs b{};
        b.a = (const unsigned char*)ht; b.lda_b = p.npad * 2; b.m = p.d;
        b.b = (const unsigned char*)dz; b.ldb_b = p.vpad * 2; b.n = p.v; b.bk_rows = p.n;
        b.nk = (int)(p.npad / 64);
        b.mtiles = (p.d + kTileV - 1) / kTileV;
        b.ntiles = (p.v + kTileT - 1) / kTileT;
        b.c = dw; b.ldc = p.d;
        if ((e = launch_gemm(b, accumulate_dw ? kEpiStoreTAcc : kEpiStoreT, st)) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n);
    return hipGetLastError();
}

size_t ppo_workspace_bytes() {
    return align_up(sizeof(PpoPart) * kPpoMaxBlocks, 256) + 256;
}

hipError_t launch_ppo_loss(const float* logp, const float* old_train, const float* old_rollout,
                           const float* adv, const uint8_t* mask, int64_t n, double eps_lo,
                           double eps_hi, int bypass, double tis_c, double grad_scale,
                           float* loss, float* grad, float* ratio, float* contrib,
                           uint8_t* clipped, double* batch, void* workspace, hipStream_t st) {
    PpoPart* part = (PpoPart*)workspace;
    double* inv_n = (double*)((unsigned char*)workspace + align_up(sizeof(PpoPart) * kPpoMaxBlocks, 256));
    // the block count is a function of n alone (it fixes the sum order)
    const int64_t per_blk = (int64_t)kPpoThreads * kPpoUnroll * kPpoGroup * 2;
    int64_t nblk = (n + per_blk - 1) / per_blk;
    if (nblk < 1) nblk = 1;
    if (nblk > kPpoMaxBlocks) nblk = kPpoMaxBlocks;
    PpoArgs a{logp, old_train, old_rollout, adv, mask, n, eps_lo, eps_hi, tis_c, grad_scale,
              bypass, loss, grad, ratio, contrib, clipped};
    auto al = [](const void* p, uintptr_t b) { return ((uintptr_t)p & (b - 1)) == 0; };
    const bool vec = al(logp, 16) && al(old_train, 16) && al(old_rollout, 16) && al(adv, 16) &&
                     al(mask, 4) && al(loss, 16) && al(grad, 16) && al(ratio, 16) &&
                     al(contrib, 16) && al(clipped, 4);
    if (vec)
        hipLaunchKernelGGL(ppo_token_kernel<true>, dim3((unsigned)nblk), dim3(kPpoThreads), 0, st,
                           a, part);
    else
        hipLaunchKernelGGL(ppo_token_kernel<false>, dim3((unsigned)nblk), dim3(kPpoThreads), 0, st,
                           a, part);
    hipLaunchKernelGGL(ppo_final_kernel, dim3(1), dim3(kPpoThreads), 0, st, (const PpoPart*)part,
                       (int)nblk, batch, inv_n);
    if (grad && n > 0 && !(grad_scale > 0.0))
    {
        if (al(grad, 16))
            hipLaunchKernelGGL(ppo_scale_kernel<true>, dim3((unsigned)nblk), dim3(kPpoThreads), 0,
                               st, grad, n, (const double*)inv_n);
        else
            hipLaunchKernelGGL(ppo_scale_kernel<false>, dim3((unsigned)nblk), dim3(kPpoThreads), 0,
                               st, grad, n, (const double*)inv_n);
    }
    return hipGetLastError();
}

}  // namespace tim
