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
//   1. transpose_bf16: W^T [D][Vp] and h^T [D][Np], zero-padded to multiples
//      of 64 along the contracted dimension.
//   2. gemm_nt<kEpiDz>: the logits of a 256 x 256 (vocabulary x token) tile,
//      recomputed in ascending K with fp32 accumulation (32x32x16 MFMAs; the
//      bf16 forward uses 16x16x32, so a logit can differ from the forward's
//      in its last bits); the epilogue forms dz with the forward's lse and writes
//      dz^T [Vp][Np] (bf16, zero outside V x N).
//   3. transpose_bf16: dz [Np][Vp].
//   4. gemm_nt<kEpiStore>: dh[t, d] = sum_v dz[t, v] W^T[d, v].
//   5. gemm_nt<kEpiStore>: dW[v, d] = sum_t dz^T[v, t] h^T[d, t].
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
// rows <= r < out_cols.  Grid: (ceil(out_cols / 64), ceil(cols / 64)).
__global__ void __launch_bounds__(kTrThreads)
transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t rows, int64_t cols,
                      uint16_t* __restrict__ out, int64_t ld_out, int64_t out_cols) {
    __shared__ uint16_t tile[kTrTile][kTrTile + 2];
    const int64_t r0 = (int64_t)blockIdx.x * kTrTile, c0 = (int64_t)blockIdx.y * kTrTile;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;       // 64 x 4
#pragma unroll
    for (int k = 0; k < kTrTile / 4; ++k) {
        const int lr = ty + 4 * k;
        const int64_t r = r0 + lr, c = c0 + tx;
        tile[lr][tx] = (r < rows && c < cols) ? in[r * ld_in + c] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTrTile / 4; ++k) {
        const int lc = ty + 4 * k;
        const int64_t c = c0 + lc, r = r0 + tx;
        if (c < cols && r < out_cols) out[c * ld_out + r] = tile[tx][lc];
    }
}

// ---------------------------------------------------------------------------
// NT GEMM tile kernel: C[m][n] = sum_k A[m][k] B[n][k], bf16, fp32 accumulate
// ---------------------------------------------------------------------------

enum { kEpiDz = 0, kEpiStore = 1, kEpiStoreAcc = 2 };

struct GemmArgs {
    const unsigned char* a; int64_t lda_b; int64_t m;   // A: m rows, K contiguous (bytes)
    const unsigned char* b; int64_t ldb_b; int64_t n;   // B: n rows, K contiguous
    int nk;                                             // K / 64 stages
    int64_t mtiles, ntiles;
    // kEpiStore
    float* c; int64_t ldc;
    // kEpiDz (A = W, B = h): logits of valid rows m < vtrue, n < ntrue
    const float* lse; const float* g; const int32_t* ids;
    int64_t vtrue, ntrue;
    uint16_t* dzt; int64_t lddz;                        // dz^T [Vp][Np]
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

template <int kEpi>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_nt_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wv = wave & 1;        // row half of the tile (128 rows of A)
    const int wt = wave >> 1;       // column half of the tile (128 rows of B)
    const int lrow = lane & 31;
    const int lhalf = lane >> 5;

    int64_t mt, nt;
    gemm_tile_of_block(p.mtiles, p.ntiles, mt, nt);
    // the tile indices are uniform; saying so keeps the buffer descriptors
    // built from them in scalar registers (else every copy is a waterfall loop)
    const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)mt) * kTileV;
    const int64_t n0 = (int64_t)__builtin_amdgcn_readfirstlane((int)nt) * kTileT;
    const int nk = p.nk;

    f32x16 acc[4][4];
    // output element of acc[bi][bj][r]: row m0 + wv*128 + bi*32 + (r/4)*8 +
    // lhalf*4 + r%4, column n0 + wt*128 + bj*32 + lrow
    auto row_of = [&](int bi, int r) -> int64_t {
        return m0 + wv * 128 + bi * 32 + (r >> 2) * 8 + lhalf * 4 + (r & 3);
    };
    auto col_of = [&](int bj) -> int64_t { return n0 + wt * 128 + bj * 32 + lrow; };
    if constexpr (kEpi == kEpiStoreAcc) {
        // the chain continues from the stored value
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = row_of(bi, r);
                const float* crow = p.c + (row < p.m ? row : 0) * p.ldc;
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) {
                    const int64_t col = col_of(bj);
                    acc[bi][bj][r] = (row < p.m && col < p.n) ? crow[col] : 0.f;
                }
                // a few loads in flight at a time: unbounded, the compiler
                // issues all 256 at once and spills their destinations
                if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
    } else {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;
    }

    // Copy assignment as in the forward kernel: wave `wave` fills 8-row
    // blocks 8 wave .. 8 wave + 7 of both operand tiles; rows past m or n are
    // redirected to the last valid row (results discarded), so every access
    // lies inside the operands and inside the descriptors' extents.
    uint32_t aoff[8], boff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int drow = (wave * 8 + j) * 8 + (lane >> 3);
        const uint32_t cb = (uint32_t)(((lane & 7) ^ ((drow >> 1) & 7)) * 16);
        int64_t ra = m0 + drow, rb = n0 + drow;
        if (ra > p.m - 1) ra = p.m - 1;
        if (rb > p.n - 1) rb = p.n - 1;
        aoff[j] = (uint32_t)((ra - m0) * p.lda_b) + cb;
        boff[j] = (uint32_t)((rb - n0) * p.ldb_b) + cb;
    }
    const int64_t arows = (p.m - m0) < kTileV ? (p.m - m0) : kTileV;
    const int64_t brows = (p.n - n0) < kTileT ? (p.n - n0) : kTileT;
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.a + m0 * p.lda_b), (short)0,
        (int)((arows - 1) * p.lda_b + (int64_t)nk * kStageBytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.b + n0 * p.ldb_b), (short)0,
        (int)((brows - 1) * p.ldb_b + (int64_t)nk * kStageBytes), kRsrcWord3);

    const uint32_t lds_base = lds_addr(lds);
    uint32_t kofs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kofs[ks] = (uint32_t)swz(lrow, ks * 2 + lhalf);

    // A of stage st + 1 and B of stage st + 2 are copied while stage st
    // computes; past the last stage both wrap to K offset 0 (valid rows into
    // positions that are never read again).
    int a_kb = 0, b_kb = 0;
    auto copy_a = [&](int part, int pos) {
        unsigned char* base = lds + pos * kOperandBytes;
        const uint32_t koff = (uint32_t)(a_kb * kStageBytes);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = part * 4 + jj;
            dma16_buf(ars, base + (wave * 8 + j) * 1024, aoff[j], koff);
        }
    };
    auto copy_b = [&](int part, int pos) {
        unsigned char* base = lds + pos * kOperandBytes;
        const uint32_t koff = (uint32_t)(b_kb * kStageBytes);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = part * 4 + jj;
            dma16_buf(brs, base + (wave * 8 + j) * 1024, boff[j], koff);
        }
    };
    auto advance_a = [&]() { if (++a_kb == nk) a_kb = 0; };
    auto advance_b = [&]() { if (++b_kb == nk) b_kb = 0; };
    auto next_pos = [](int q) { return q + 2 >= kPos ? q + 2 - kPos : q + 2; };
    auto issue_frags = [&](u32x4 (&f)[8], int pa, int pb, int ks) {
        lds_issue_8x16(f, lds_base + (uint32_t)(pa * kOperandBytes) + kofs[ks] + (uint32_t)(wv * 128 * kStageBytes),
                       lds_base + (uint32_t)(pb * kOperandBytes) + kofs[ks] + (uint32_t)(wt * 128 * kStageBytes));
    };
    auto mfma_step = [&](const u32x4 (&f)[8]) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, f[bi]), __builtin_bit_cast(bf16x8, f[4 + bj]),
                    acc[bi][bj], 0, 0, 0);
    };

    // Pipeline of the forward kernel (ring positions (2 stage + op) % 5, op 0:
    // B, op 1: A; four copies per k-step, one after every four MFMAs).
    int rd_b = 0, rd_a = 1;
    int cp_a = 3, cp_b = 4;
    copy_b(0, 0); copy_b(1, 0); advance_b();
    copy_a(0, 1); copy_a(1, 1); advance_a();
    copy_b(0, 2); copy_b(1, 2); advance_b();
    wait_vmcnt<kDmaPerStage / 2>();
    __syncthreads();
    u32x4 fa[8], fb[8];
    issue_frags(fa, rd_a, rd_b, 0);

    for (int kb = 0; kb < nk; ++kb) {
        issue_frags(fb, rd_a, rd_b, 1);
        frags_ready<8>(fa);
        copy_a(0, cp_a);
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
        issue_frags(fa, rd_a, rd_b, 2);
        frags_ready<8>(fb);
        copy_a(1, cp_a);
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
        advance_a();
        issue_frags(fb, rd_a, rd_b, 3);
        frags_ready<8>(fa);
        copy_b(0, cp_b);
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
        wait_vmcnt<kDmaPerStage / 4>();
        frags_ready<0>(fb);
        asm volatile("s_barrier" ::: "memory");
        rd_b = next_pos(rd_b);
        rd_a = next_pos(rd_a);
        issue_frags(fa, rd_a, rd_b, 0);
        __builtin_amdgcn_sched_barrier(0);
        copy_b(1, cp_b);
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
        advance_b();
        cp_a = next_pos(cp_a);
        cp_b = next_pos(cp_b);
    }
    // drain: the last look-ahead read and the extra copies
    frags_ready<0>(fa);
    wait_vmcnt<0>();

    if constexpr (kEpi != kEpiDz) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t col = col_of(bj);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = row_of(bi, r);
                    if (row < p.m && col < p.n) p.c[row * p.ldc + col] = acc[bi][bj][r];
                }
            }
    } else {
        // dz = g_t ([v == a_t] - exp(z - lse_t)) for v < V, t < N; 0 in the
        // padding (rows V..Vp-1, columns N..Np-1); an id outside [0, V)
        // contributes nothing
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t t = col_of(bj);
            if (t >= p.npad) continue;
            const bool tv = t < p.ntrue;
            const int64_t tc = tv ? t : 0;
            const float g = tv ? p.g[tc] : 0.f;
            const float l = tv ? p.lse[tc] : 0.f;
            const int32_t a = tv ? p.ids[tc] : -1;
            const bool ok = tv && a >= 0 && (int64_t)a < p.vtrue && g != 0.f;
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t v = row_of(bi, r);
                    if (v >= p.vpad) continue;
                    float dz = 0.f;
                    if (ok && v < p.vtrue) {
                        const float pz = fast_exp2((acc[bi][bj][r] - l) * kLog2e);
                        dz = g * ((v == (int64_t)a ? 1.f : 0.f) - pz);
                    }
                    p.dzt[v * p.lddz + t] = bf16_rne(dz);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// PPO / GRPO surrogate
// ---------------------------------------------------------------------------

constexpr int kPpoThreads = 256;
constexpr int kPpoMaxBlocks = 16384;
constexpr int kPpoUnroll = 4;        // tokens per thread per loop trip, loads first

struct PpoPart {
    double loss, ratio, w, contrib;
    uint64_t nvalid, nclip, nnan, pad;
};

struct PpoArgs {
    const float *logp, *old_train, *old_rollout, *adv;
    const uint8_t* mask;
    int64_t n;
    double eps_lo, eps_hi, tis_c;
    int bypass;
    float *loss, *grad, *ratio, *contrib;
    uint8_t* clipped;
};

// Per token, fp64 from the fp32 inputs; block partials in a fixed tree.
// Thread tid of block b takes tokens b*256 + tid + j*grid*256, kPpoUnroll of
// them per loop trip with every load issued first.
__device__ __forceinline__ void ppo_token(const PpoArgs& a, int64_t t, float lp, float ot,
                                          float orr, float ad, bool in, PpoPart& acc) {
    double l_t = 0, g_t = 0, r_t = 1, c_t = 0;
    int clip_t = 0;
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
    if (a.loss) a.loss[t] = (float)l_t;
    if (a.grad) a.grad[t] = (float)g_t;      // scaled by 1 / n_valid afterwards
    if (a.ratio) a.ratio[t] = (float)r_t;
    if (a.contrib) a.contrib[t] = (float)c_t;
    if (a.clipped) a.clipped[t] = (uint8_t)clip_t;
}

__global__ void __launch_bounds__(kPpoThreads)
ppo_token_kernel(PpoArgs a, PpoPart* __restrict__ part) {
    __shared__ PpoPart sh[kPpoThreads];
    PpoPart acc{0, 0, 0, 0, 0, 0, 0, 0};
    const int64_t stride = (int64_t)gridDim.x * kPpoThreads;
    for (int64_t base = (int64_t)blockIdx.x * kPpoThreads + threadIdx.x; base < a.n;
         base += kPpoUnroll * stride) {
        float lp[kPpoUnroll], ot[kPpoUnroll], orr[kPpoUnroll], ad[kPpoUnroll];
        bool in[kPpoUnroll];
#pragma unroll
        for (int j = 0; j < kPpoUnroll; ++j) {
            const int64_t t = base + j * stride;
            const int64_t tc = t < a.n ? t : base;             // base < n: in bounds
            lp[j] = a.logp[tc];
            ot[j] = a.old_train[tc];
            orr[j] = a.old_rollout[tc];
            ad[j] = a.adv[tc];
            const uint32_t mk = a.mask ? (uint32_t)(a.mask[tc] != 0) : 1u;   // no short-circuit
            in[j] = ((uint32_t)(t < a.n) & mk) != 0;
        }
#pragma unroll
        for (int j = 0; j < kPpoUnroll; ++j) {
            const int64_t t = base + j * stride;
            if (t < a.n) ppo_token(a, t, lp[j], ot[j], orr[j], ad[j], in[j], acc);
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

// grad[t] *= 1 / n_valid (the derivative of the token mean)
__global__ void __launch_bounds__(kPpoThreads)
ppo_scale_kernel(float* __restrict__ grad, int64_t n, const double* __restrict__ inv_n) {
    const double s = *inv_n;
    const int64_t stride = (int64_t)gridDim.x * kPpoThreads;
    for (int64_t t = (int64_t)blockIdx.x * kPpoThreads + threadIdx.x; t < n; t += stride)
        grad[t] = (float)((double)grad[t] * s);
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

bool make_backward_plan(int64_t n, int64_t d, int64_t v, BackwardPlan* p) {
    if (n < 0 || d <= 0 || v <= 0 || v > INT32_MAX || n > INT32_MAX) return false;
    p->n = n; p->d = d; p->v = v;
    p->npad = round_up(n > 0 ? n : 1, 64);
    p->vpad = round_up(v, 64);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    p->wt_off = take((size_t)d * p->vpad * 2);
    p->ht_off = take((size_t)d * p->npad * 2);
    p->dzt_off = take((size_t)p->vpad * p->npad * 2);
    p->dz_off = take((size_t)p->npad * p->vpad * 2);
    p->total_bytes = off;
    return true;
}

static hipError_t launch_transpose(const uint16_t* in, int64_t ld_in, int64_t rows, int64_t cols,
                                   uint16_t* out, int64_t ld_out, int64_t out_cols,
                                   hipStream_t st) {
    const int64_t gx = (out_cols + kTrTile - 1) / kTrTile, gy = (cols + kTrTile - 1) / kTrTile;
    if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kTrThreads),
                       0, st, in, ld_in, rows, cols, out, ld_out, out_cols);
    return hipGetLastError();
}

static hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
    const int64_t grid = a.mtiles * a.ntiles;
    if (grid <= 0 || grid > INT32_MAX) return hipErrorInvalidValue;
    if (epi == kEpiDz)
        hipLaunchKernelGGL(gemm_nt_kernel<kEpiDz>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    else if (epi == kEpiStore)
        hipLaunchKernelGGL(gemm_nt_kernel<kEpiStore>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(gemm_nt_kernel<kEpiStoreAcc>, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_logprob_backward(const BackwardPlan& p, const void* h, int64_t ldh,
                                   const void* w, int64_t ldw, const int32_t* ids,
                                   const float* lse, const float* g, float* dh, float* dw,
                                   bool accumulate_dw, void* workspace, hipStream_t st) {
    unsigned char* ws = (unsigned char*)workspace;
    uint16_t* wt = (uint16_t*)(ws + p.wt_off);     // W^T [D][Vp]
    uint16_t* ht = (uint16_t*)(ws + p.ht_off);     // h^T [D][Np]
    uint16_t* dzt = (uint16_t*)(ws + p.dzt_off);   // dz^T [Vp][Np]
    uint16_t* dz = (uint16_t*)(ws + p.dz_off);     // dz [Np][Vp]
    hipError_t e;

    // 1. dz^T from the recomputed logits (A = W rows, B = h rows, K = D)
    GemmArgs z{};
    z.a = (const unsigned char*)w; z.lda_b = ldw * 2; z.m = p.v;
    z.b = (const unsigned char*)h; z.ldb_b = ldh * 2; z.n = p.n;
    z.nk = (int)(p.d / 64);
    z.mtiles = (p.vpad + kTileV - 1) / kTileV;
    z.ntiles = (p.npad + kTileT - 1) / kTileT;
    z.lse = lse; z.g = g; z.ids = ids; z.vtrue = p.v; z.ntrue = p.n;
    z.dzt = dzt; z.lddz = p.npad; z.vpad = p.vpad; z.npad = p.npad;
    if ((e = launch_gemm(z, kEpiDz, st)) != hipSuccess) return e;

    if (dh) {
        // 2. dz = (dz^T)^T and W^T, then dh = dz W (K = vocabulary)
        if ((e = launch_transpose(dzt, p.npad, p.vpad, p.npad, dz, p.vpad, p.vpad, st)) != hipSuccess)
            return e;
        if ((e = launch_transpose((const uint16_t*)w, ldw, p.v, p.d, wt, p.vpad, p.vpad, st)) != hipSuccess)
            return e;
        GemmArgs a{};
        a.a = (const unsigned char*)dz; a.lda_b = p.vpad * 2; a.m = p.n;
        a.b = (const unsigned char*)wt; a.ldb_b = p.vpad * 2; a.n = p.d;
        a.nk = (int)(p.vpad / 64);
        a.mtiles = (p.n + kTileV - 1) / kTileV;
        a.ntiles = (p.d + kTileT - 1) / kTileT;
        a.c = dh; a.ldc = p.d;
        if ((e = launch_gemm(a, kEpiStore, st)) != hipSuccess) return e;
    }
    if (dw) {
        // 3. h^T, then dW = dz^T h (K = tokens, ascending)
        if ((e = launch_transpose((const uint16_t*)h, ldh, p.n, p.d, ht, p.npad, p.npad, st)) != hipSuccess)
            return e;
        GemmArgs b{};
        b.a = (const unsigned char*)dzt; b.lda_b = p.npad * 2; b.m = p.v;
        b.b = (const unsigned char*)ht; b.ldb_b = p.npad * 2; b.n = p.d;
        b.nk = (int)(p.npad / 64);
        b.mtiles = (p.v + kTileV - 1) / kTileV;
        b.ntiles = (p.d + kTileT - 1) / kTileT;
        b.c = dw; b.ldc = p.d;
        if ((e = launch_gemm(b, accumulate_dw ? kEpiStoreAcc : kEpiStore, st)) != hipSuccess) return e;
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
                           double eps_hi, int bypass, double tis_c, float* loss, float* grad,
                           float* ratio, float* contrib, uint8_t* clipped, double* batch,
                           void* workspace, hipStream_t st) {
    PpoPart* part = (PpoPart*)workspace;
    double* inv_n = (double*)((unsigned char*)workspace + align_up(sizeof(PpoPart) * kPpoMaxBlocks, 256));
    int64_t nblk = (n + kPpoThreads * kPpoUnroll * 4 - 1) / (kPpoThreads * kPpoUnroll * 4);
    if (nblk < 1) nblk = 1;
    if (nblk > kPpoMaxBlocks) nblk = kPpoMaxBlocks;
    PpoArgs a{logp, old_train, old_rollout, adv, mask, n, eps_lo, eps_hi, tis_c, bypass,
              loss, grad, ratio, contrib, clipped};
    hipLaunchKernelGGL(ppo_token_kernel, dim3((unsigned)nblk), dim3(kPpoThreads), 0, st, a, part);
    hipLaunchKernelGGL(ppo_final_kernel, dim3(1), dim3(kPpoThreads), 0, st, (const PpoPart*)part,
                       (int)nblk, batch, inv_n);
    if (grad && n > 0)
        hipLaunchKernelGGL(ppo_scale_kernel, dim3((unsigned)nblk), dim3(kPpoThreads), 0, st, grad,
                           n, (const double*)inv_n);
    return hipGetLastError();
}

}  // namespace tim
