// tim_internal.h — kernel launch interfaces shared by the C-ABI layer and
// the kernel translation units of libtim.so.  Not installed; not part of
// the public ABI (that is include/tim.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tim {

// ---------------------------------------------------------------------------
// LM-head log-probability kernels (lmhead.hip)
// ---------------------------------------------------------------------------

// Tile geometry of the fused contraction + online log-sum-exp kernel.
// A workgroup owns kTileV vocabulary rows x kTileT tokens of the logit
// matrix at a time and walks one vocabulary *chunk* (kChunkTiles tiles in
// the batch-invariant schedule) in ascending order, carrying a running
// (max, sum-exp) per token in registers.
constexpr int kTileV = 256;
constexpr int kTileT = 256;
constexpr int kStageBytes = 128;   // bytes of K per row per pipeline stage
constexpr int kThreads = 256;      // 4 waves of 64
constexpr int kInvariantChunkTiles = 1;   // 256 vocabulary entries per chunk

// Workspace layout of tim_logprob_forward (all offsets 256-byte aligned):
//   [0, part_bytes)           float2 partials[nchunks][n]: (max, sum-exp)
//   [zsel_off, +4n)           float  zsel[n]: the selected logit
struct LogprobPlan {
    int64_t n, d, v;
    int dtype;            // 0 bf16, 1 fp32
    int chunk_tiles;      // vocabulary tiles per chunk
    int64_t nvtiles;      // ceil(v / kTileV)
    int64_t nchunks;      // ceil(nvtiles / chunk_tiles)
    int64_t nttiles;      // ceil(n / kTileT)
    bool entropy;         // carry the entropy state u as well
    bool narrow;          // bf16, n <= 32: one wave per half chunk (lmhead_narrow_kernel),
                          // partials per half chunk
    int nb;               // narrow: token column blocks of 16 per wave (1 or 2)
    int ntg;              // narrow: token groups of 16 nb (1 or 2)
    int ksplit;           // K split (1: none); 2 only for TIM_SCHED_SPLIT_K, bf16,
                          // 32 < n <= 256, no entropy
    // workspace: float2 part[P][n] | float zsel[n] | float upart[P][n] |
    // float slog[ksplit][v][n] (ksplit > 1 only), with P = nchunks, or
    // 2 nchunks (one state per half chunk) when narrow
    size_t part_bytes, zsel_off, upart_off, slog_off, total_bytes;
};

// Fills `p`; returns false for sizes the library does not accept.
bool make_logprob_plan(int64_t n, int64_t d, int64_t v, int dtype, unsigned flags,
                       bool entropy, LogprobPlan* p);

// Temperature tau as the kernels use it: c2 = log2(e) / tau, it = 1 / tau
// (fp32, rounded once on the host; tau = 1 gives exactly log2(e) and 1).
struct ScoreScale {
    float c2, it;
};
ScoreScale make_score_scale(double temperature);

hipError_t launch_lmhead_partials(const LogprobPlan& p, const void* h, int64_t ldh,
                                  const void* w, int64_t ldw, const int32_t* ids,
                                  const ScoreScale& sc, void* workspace, int32_t* n_bad_ids,
                                  hipStream_t st);
hipError_t launch_lse_merge(const LogprobPlan& p, const int32_t* ids, const ScoreScale& sc,
                            const void* workspace, float* logp, float* lse, float* entropy,
                            int32_t* n_bad_ids, hipStream_t st);

// The fp32 head's tile kernel (lmhead.hip) as a GEMM for the fp32 backward:
// C[m][n] = sum_k A[m][k] B[n][k], A and B fp32 rows with K contiguous,
// the tile pipeline, MFMA sequence and K order of the fp32 forward.
enum { kF32Fold = 0, kF32Dz = 1, kF32Store = 2, kF32StoreAcc = 3 };
struct F32Epi {
    const float* lse; const float* g;   // kF32Dz: the forward's lse, dL/dlogp per token
    float* dz; int64_t ldz;             // kF32Dz: dz [Np][Vp], or null
    float* dzt; int64_t lddzt;          // kF32Dz: dz^T [Vp][Np], or null
    int64_t vpad, npad;                 // kF32Dz: padded sizes written (zeros past V, N)
    float* c; int64_t ldc;              // kF32Store(Acc): C [m][n]
};
struct F32Gemm {
    int mode;                           // kF32Dz, kF32Store or kF32StoreAcc
    const void* a; int64_t lda;         // A [m][k] (elements); W for kF32Dz
    const void* b; int64_t ldb;         // B [n][k]; h for kF32Dz
    const int32_t* ids;                 // kF32Dz: the selected ids
    int64_t m, n, k;                    // k a multiple of 32; kF32Dz: m = V, n = N
    F32Epi ep;
};
hipError_t launch_f32_gemm(const F32Gemm& g, hipStream_t st);

// RMSNorm (norm.hip): one wave per row, fp64 row sums, one rounding.
hipError_t launch_rmsnorm(const void* x, int64_t ldx, const void* gamma, int64_t n, int64_t d,
                          int dtype, double eps, void* y, int64_t ldy, float* rstd,
                          hipStream_t st);

// ---------------------------------------------------------------------------
// Mismatch statistics kernels (stats.hip)
// ---------------------------------------------------------------------------

// Tokens per sub-chunk.  Every sequence is cut into sub-chunks that start at
// the sequence's first token and every kSubChunk tokens after it, so a
// sequence's reduction order depends on nothing but its own length.
constexpr int kSubChunk = 1024;

struct StatsParamsDev {
    double clip_c, log_c, seq_lo, seq_hi, seq_k3_hi;
};

// Workspace layout of tim_mismatch_stats (offsets 256-byte aligned): one
// slot per possible sub-chunk (sequence j's sub-chunk k sits at slot
// floor(c_j / kSubChunk) + j + k, strictly increasing, fewer than
// floor(n / kSubChunk) + s + 1 slots), and per streaming wave the sum and
// maximum of |delta| over its tokens; then the finalize blocks' batch
// partials and their completion ticket.
struct StatsPlan {
    int64_t n, s;
    int64_t range;       // tokens per streaming wave (a multiple of 256)
    int64_t nwaves;      // streaming waves, >= 1
    int64_t nslots;      // sub-chunk slots
    int64_t nblk_fin;    // finalize blocks (256 sequences or streaming waves each)
    size_t slot_off, wpart_off, blk_off, ticket_off, total_bytes;
};

bool make_stats_plan(int64_t n, int64_t s, StatsPlan* p);

struct TokenOutPtrs {
    float *delta, *ratio, *k1, *k2, *k3, *tis_w;
    uint8_t* clipped;
};
struct SeqOutPtrs {
    int32_t *n_valid, *n_clipped, *n_nan;
    double *mean_delta, *mean_k1, *mean_k2, *mean_k3, *mean_tis_w;
    uint8_t *reject, *reject_k3;
};

hipError_t launch_mismatch_stats(const StatsPlan& p, const float* lt, const float* lr,
                                 const uint8_t* mask, const int32_t* cu,
                                 const StatsParamsDev& prm, const TokenOutPtrs& tok,
                                 const SeqOutPtrs& seq, double* batch, void* workspace,
                                 hipStream_t st);

// ---------------------------------------------------------------------------
// Extra mismatch metrics (extras.hip)
// ---------------------------------------------------------------------------

constexpr int kXMaxQ = 4;          // probabilities per call, both kinds together
constexpr int kXPasses = 6;        // radix-select passes over the tokens
constexpr int kXMaxBlocks = 512;   // blocks of a pass
constexpr int kXFusedMax = 8192;   // up to this many tokens, one block does everything

// Output vector layout (the TIM_X_* indices of tim.h).
constexpr int kXOutNValid = 0, kXOutNExtreme = 1, kXOutExtremeFrac = 2, kXOutMeanRelDiff = 3,
              kXOutRatioQ = 4, kXOutAbsQ = 8, kXOutFields = 12;

struct XParamsDev {
    double tok_tau;
    int32_t nrq, naq;      // ratio and |delta| probabilities; nrq + naq <= kXMaxQ
    double rq[kXMaxQ], aq[kXMaxQ];
};

// Workspace layout of tim_mismatch_extras (offsets 256-byte aligned): the
// select state, per-block histograms and key ranges, the summed histogram,
// per-block partial sums, and the per-block candidate regions with their
// counts and overflow flag.  nblk and cap depend on n only.
struct ExtrasPlan {
    int64_t n, nblk;
    bool fused;        // n <= kXFusedMax: one block, no workspace use
    uint32_t cap;      // keys per block in the candidate regions
    size_t state_off, bhist_off, bmm_off, ghist_off, part_off, cand_off, ccnt_off, cflag_off,
        shist_off, pmark_off, total_bytes;
};

bool make_extras_plan(int64_t n, ExtrasPlan* p);

hipError_t launch_mismatch_extras(const ExtrasPlan& p, const float* lt, const float* lr,
                                  const uint8_t* mask, const XParamsDev& prm, double* out,
                                  void* workspace, hipStream_t st);

// ---------------------------------------------------------------------------
// Backward of the log-probability and the PPO surrogate (bwd.hip)
// ---------------------------------------------------------------------------

// Workspace of tim_logprob_backward (offsets 256-byte aligned): W^T [D][Vp],
// h^T [D][Np], dz^T [Vp][Np] and dz [Np][Vp], bf16, with Vp and Np the
// vocabulary and token counts rounded up to multiples of 64.
struct BackwardPlan {
    int64_t n, d, v, npad, vpad;
    int dtype;                          // 0 bf16, 1 fp32
    // bf16: h^T, dz; fp32: W^T, h^T, dz^T, dz (each of the element type)
    size_t wt_off, ht_off, dzt_off, dz_off, total_bytes;
};

bool make_backward_plan(int64_t n, int64_t d, int64_t v, int dtype, BackwardPlan* p);

hipError_t launch_logprob_backward(const BackwardPlan& p, const void* h, int64_t ldh,
                                   const void* w, int64_t ldw, const int32_t* ids,
                                   const float* lse, const float* g, float* dh, float* dw,
                                   bool accumulate_dw, void* workspace, hipStream_t st);

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t st);

// Batch vector of tim_ppo_loss (the TIM_P_* indices of tim.h).
constexpr int kPpoOutMeanLoss = 0, kPpoOutClipFrac = 1, kPpoOutMeanRatio = 2,
              kPpoOutMeanTisW = 3, kPpoOutMeanContrib = 4, kPpoOutNValid = 5,
              kPpoOutNClipped = 6, kPpoOutNNan = 7, kPpoOutFields = 8;

size_t ppo_workspace_bytes();

hipError_t launch_ppo_loss(const float* logp, const float* old_train, const float* old_rollout,
                           const float* adv, const uint8_t* mask, int64_t n, double eps_lo,
                           double eps_hi, int bypass, double tis_c, double grad_scale,
                           float* loss, float* grad, float* ratio, float* contrib,
                           uint8_t* clipped, double* batch, void* workspace, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace tim
