// tim_api.hip — the C ABI of libtim.so (declared in include/tim.h): argument
// validation on the host, workspace sizing, and kernel launches on the
// caller's stream.  No device memory is allocated here and no call
// synchronises.

#include "tim.h"
#include "tim_internal.h"

#include <atomic>
#include <math.h>

// Scratch memory of tim_logprob_forward_noalloc, for callers that cannot
// allocate.  Every device the library's code object is loaded on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its address on a device comes from
// hipGetSymbolAddress (scratch_on_device below) and only that address is
// ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[TIM_NOALLOC_SCRATCH_BYTES];

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Device address of `scratch` on device `dev`, looked up on the first call
// for that device with the device current (then restored), and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

hipError_t scratch_on_device(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return hipSuccess;
}

// The tile kernels address an operand tile of `rows` rows through a buffer
// descriptor whose extent, (rows - 1) * ld_bytes + k_bytes, and per-lane
// 32-bit offsets must stay below 2^31.
inline bool tile_extent_ok(int64_t rows, int64_t ld_bytes, int64_t k_bytes) {
    return (rows - 1) * ld_bytes + k_bytes < ((int64_t)1 << 31);
}

}  // namespace

extern "C" {

int tim_abi_version(void) { return TIM_ABI_VERSION; }

const char* tim_status_string(int status) {
    switch (status) {
        case TIM_OK: return "TIM_OK: success";
        case TIM_EINVAL: return "TIM_EINVAL: invalid argument";
        case TIM_EUNSUPPORTED: return "TIM_EUNSUPPORTED: unsupported size, leading dimension or alignment";
        case TIM_EWORKSPACE: return "TIM_EWORKSPACE: workspace missing or too small";
        case TIM_EHIP: return "TIM_EHIP: HIP launch or runtime error";
        case TIM_ESCRATCH:
            return "TIM_ESCRATCH: the request needs more than the static scratch of "
                   "tim_logprob_forward_noalloc (TIM_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown tim_status";
    }
}

size_t tim_logprob_workspace_bytes(int64_t n, int64_t d, int64_t v, int dtype, unsigned flags) {
    tim::LogprobPlan p;
    if (!tim::make_logprob_plan(n, d, v, dtype, flags, false, &p)) return 0;
    return p.total_bytes;
}

namespace {

// Host checks of tim_logprob_forward and tim_logprob_forward_noalloc, in the
// order the header documents; fills the plan on success.
int forward_checks(const void* h, int64_t ldh, const void* w, int64_t ldw, const int32_t* ids,
                   int64_t n, int64_t d, int64_t v, int dtype, unsigned flags, const float* logp,
                   tim::LogprobPlan* p) {
    if (n < 0 || d <= 0 || v <= 0 || v > INT32_MAX || (dtype != TIM_BF16 && dtype != TIM_F32) ||
        flags > TIM_SCHED_SPLIT_K)
        return TIM_EINVAL;
    if (ldh < d || ldw < d) return TIM_EINVAL;
    if (n == 0) return TIM_OK;
    if (!h || !w || !ids || !logp) return TIM_EINVAL;
    const int64_t esz = dtype == TIM_BF16 ? 2 : 4;
    if (d % 64 != 0) return TIM_EUNSUPPORTED;
    if ((ldh * esz) % 16 != 0 || (ldw * esz) % 16 != 0) return TIM_EUNSUPPORTED;
    if (!aligned(h, 16) || !aligned(w, 16)) return TIM_EUNSUPPORTED;
    if (!tile_extent_ok(tim::kTileT, ldh * esz, d * esz) ||
        !tile_extent_ok(tim::kTileV, ldw * esz, d * esz))
        return TIM_EUNSUPPORTED;
    if (!tim::make_logprob_plan(n, d, v, dtype, flags, false, p)) return TIM_EINVAL;
    if (p->nchunks * p->nttiles > INT32_MAX) return TIM_EUNSUPPORTED;
    return TIM_OK;
}

int forward_launch(const tim::LogprobPlan& p, const void* h, int64_t ldh, const void* w,
                   int64_t ldw, const int32_t* ids, float* logp, float* lse, int32_t* n_bad_ids,
                   void* workspace, hipStream_t st) {
    const tim::ScoreScale sc = tim::make_score_scale(1.0);
    if (tim::launch_lmhead_partials(p, h, ldh, w, ldw, ids, sc, workspace, n_bad_ids, st) != hipSuccess)
        return TIM_EHIP;
    if (tim::launch_lse_merge(p, ids, sc, workspace, logp, lse, nullptr, n_bad_ids, st) != hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

}  // namespace

int tim_logprob_forward(const void* h, int64_t ldh, const void* w, int64_t ldw,
                        const int32_t* ids, int64_t n, int64_t d, int64_t v, int dtype,
                        unsigned flags, float* logp, float* lse, int32_t* n_bad_ids,
                        void* workspace, size_t workspace_bytes, void* stream) {
    tim::LogprobPlan p;
    const int chk = forward_checks(h, ldh, w, ldw, ids, n, d, v, dtype, flags, logp, &p);
    if (chk != TIM_OK || n == 0) return chk;
    if (!workspace || workspace_bytes < p.total_bytes) return TIM_EWORKSPACE;
    if (!aligned(workspace, 256)) return TIM_EUNSUPPORTED;
    return forward_launch(p, h, ldh, w, ldw, ids, logp, lse, n_bad_ids, workspace,
                          (hipStream_t)stream);
}

int tim_logprob_forward_noalloc(const void* h, int64_t ldh, const void* w, int64_t ldw,
                                const int32_t* ids, int64_t n, int64_t d, int64_t v, int dtype,
                                unsigned flags, float* logp, float* lse, int32_t* n_bad_ids,
                                void* stream) {
    tim::LogprobPlan p;
    const int chk = forward_checks(h, ldh, w, ldw, ids, n, d, v, dtype, flags, logp, &p);
    if (chk != TIM_OK || n == 0) return chk;
    if (p.total_bytes > TIM_NOALLOC_SCRATCH_BYTES) return TIM_ESCRATCH;
    hipStream_t st = (hipStream_t)stream;
    int dev = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess) return TIM_EHIP;
    void* ws = nullptr;
    if (scratch_on_device(dev, &ws) != hipSuccess) return TIM_EHIP;
    // Nothing here has to start at zero: every scratch byte a kernel of this
    // call reads was written earlier in the same call.
    return forward_launch(p, h, ldh, w, ldw, ids, logp, lse, n_bad_ids, ws, st);
}

int tim_rmsnorm(const void* x, int64_t ldx, const void* gamma, int64_t n, int64_t d, int dtype,
                double eps, void* y, int64_t ldy, float* rstd, void* stream) {
    if (n < 0 || d <= 0 || (dtype != TIM_BF16 && dtype != TIM_F32) || !(eps >= 0.0) ||
        !isfinite(eps) || ldx < d || ldy < d)
        return TIM_EINVAL;
    if (n == 0) return TIM_OK;
    if (!x || !gamma || !y) return TIM_EINVAL;
    if (tim::launch_rmsnorm(x, ldx, gamma, n, d, dtype, eps, y, ldy, rstd, (hipStream_t)stream) !=
        hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

namespace {

// Workspace of tim_logprob_forward_ex: the head's plan, then (with a norm)
// the normalised rows [n][d] of dtype.
bool ex_layout(int64_t n, int64_t d, int64_t v, int dtype, unsigned flags,
               const tim_forward_params* prm, bool with_entropy, tim::LogprobPlan* p,
               size_t* norm_off, size_t* total) {
    if (!prm || !(prm->temperature > 0.0) || !isfinite(prm->temperature)) return false;
    if (prm->norm_gamma && (!(prm->norm_eps >= 0.0) || !isfinite(prm->norm_eps))) return false;
    if (!tim::make_logprob_plan(n, d, v, dtype, flags, with_entropy, p)) return false;
    *norm_off = (p->total_bytes + 255) / 256 * 256;
    const size_t esz = dtype == TIM_BF16 ? 2 : 4;
    *total = *norm_off + (prm->norm_gamma ? ((size_t)n * (size_t)d * esz + 255) / 256 * 256 : 0);
    return true;
}

}  // namespace

size_t tim_logprob_ex_workspace_bytes(int64_t n, int64_t d, int64_t v, int dtype, unsigned flags,
                                      const tim_forward_params* params, int with_entropy) {
    tim::LogprobPlan p;
    size_t norm_off = 0, total = 0;
    if (!ex_layout(n, d, v, dtype, flags, params, with_entropy != 0, &p, &norm_off, &total))
        return 0;
    return total;
}

int tim_logprob_forward_ex(const void* h, int64_t ldh, const void* w, int64_t ldw,
                           const int32_t* ids, int64_t n, int64_t d, int64_t v, int dtype,
                           unsigned flags, const tim_forward_params* prm, float* logp, float* lse,
                           float* entropy, int32_t* n_bad_ids, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (n < 0 || d <= 0 || v <= 0 || v > INT32_MAX || (dtype != TIM_BF16 && dtype != TIM_F32) ||
        flags > TIM_SCHED_SPLIT_K || !prm)
        return TIM_EINVAL;
    if (!(prm->temperature > 0.0) || !isfinite(prm->temperature)) return TIM_EINVAL;
    if (prm->norm_gamma && (!(prm->norm_eps >= 0.0) || !isfinite(prm->norm_eps))) return TIM_EINVAL;
    if (ldh < d || ldw < d) return TIM_EINVAL;
    if (n == 0) return TIM_OK;
    if (!h || !w || !ids || !logp) return TIM_EINVAL;
    const int64_t esz = dtype == TIM_BF16 ? 2 : 4;
    if (d % 64 != 0) return TIM_EUNSUPPORTED;
    if ((ldw * esz) % 16 != 0 || !aligned(w, 16)) return TIM_EUNSUPPORTED;
    if (!prm->norm_gamma && ((ldh * esz) % 16 != 0 || !aligned(h, 16))) return TIM_EUNSUPPORTED;
    if (!tile_extent_ok(tim::kTileT, (prm->norm_gamma ? d : ldh) * esz, d * esz) ||
        !tile_extent_ok(tim::kTileV, ldw * esz, d * esz))
        return TIM_EUNSUPPORTED;
    tim::LogprobPlan p;
    size_t norm_off = 0, total = 0;
    if (!ex_layout(n, d, v, dtype, flags, prm, entropy != nullptr, &p, &norm_off, &total))
        return TIM_EINVAL;
    if (p.nchunks * p.nttiles > INT32_MAX) return TIM_EUNSUPPORTED;
    if (!workspace || workspace_bytes < total) return TIM_EWORKSPACE;
    if (!aligned(workspace, 256)) return TIM_EUNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    const void* rows = h;
    int64_t ldr = ldh;
    if (prm->norm_gamma) {
        void* hn = (unsigned char*)workspace + norm_off;
        if (tim::launch_rmsnorm(h, ldh, prm->norm_gamma, n, d, dtype, prm->norm_eps, hn, d,
                                nullptr, st) != hipSuccess)
            return TIM_EHIP;
        rows = hn;
        ldr = d;
    }
    const tim::ScoreScale sc = tim::make_score_scale(prm->temperature);
    if (tim::launch_lmhead_partials(p, rows, ldr, w, ldw, ids, sc, workspace, n_bad_ids, st) !=
        hipSuccess)
        return TIM_EHIP;
    if (tim::launch_lse_merge(p, ids, sc, workspace, logp, lse, entropy, n_bad_ids, st) != hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

size_t tim_stats_workspace_bytes(int64_t n, int64_t s) {
    tim::StatsPlan p;
    if (!tim::make_stats_plan(n, s, &p)) return 0;
    return p.total_bytes;
}

int tim_mismatch_stats(const float* logp_train, const float* logp_rollout, const uint8_t* mask,
                       const int32_t* cu_seqlens, int64_t n, int64_t s, const tim_stats_params* p,
                       const tim_token_out* tok, const tim_seq_out* seq, double* batch,
                       void* workspace, size_t workspace_bytes, void* stream) {
    if (n < 0 || s < 0 || !p) return TIM_EINVAL;
    if (!(p->tis_clip_c > 0.0) || !isfinite(p->tis_clip_c)) return TIM_EINVAL;
    if (!(p->seq_lo <= p->seq_hi) || isnan(p->seq_k3_hi)) return TIM_EINVAL;
    if (n > 0 && s < 1) return TIM_EINVAL;
    if (n == 0 && s == 0) return TIM_OK;
    if (n > 0 && (!logp_train || !logp_rollout)) return TIM_EINVAL;
    if (!cu_seqlens) return TIM_EINVAL;
    tim::StatsPlan plan;
    if (!tim::make_stats_plan(n, s, &plan)) return TIM_EUNSUPPORTED;
    if (!workspace || workspace_bytes < plan.total_bytes) return TIM_EWORKSPACE;
    if (!aligned(workspace, 256)) return TIM_EUNSUPPORTED;

    tim::StatsParamsDev prm;
    prm.clip_c = p->tis_clip_c;
    prm.log_c = log(p->tis_clip_c);
    prm.seq_lo = p->seq_lo;
    prm.seq_hi = p->seq_hi;
    prm.seq_k3_hi = p->seq_k3_hi;
    tim::TokenOutPtrs to{};
    if (tok) to = {tok->delta, tok->ratio, tok->k1, tok->k2, tok->k3, tok->tis_w, tok->clipped};
    tim::SeqOutPtrs so{};
    if (seq) so = {seq->n_valid, seq->n_clipped, seq->n_nan, seq->mean_delta, seq->mean_k1,
                   seq->mean_k2, seq->mean_k3, seq->mean_tis_w, seq->reject, seq->reject_k3};
    if (tim::launch_mismatch_stats(plan, logp_train, logp_rollout, mask, cu_seqlens, prm, to, so,
                                   batch, workspace, (hipStream_t)stream) != hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

size_t tim_extras_workspace_bytes(int64_t n) {
    tim::ExtrasPlan p;
    if (!tim::make_extras_plan(n, &p)) return 0;
    return p.total_bytes;
}

int tim_mismatch_extras(const float* logp_train, const float* logp_rollout, const uint8_t* mask,
                        int64_t n, const tim_extras_params* p, double* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
    static_assert(TIM_X_MAX_Q == tim::kXMaxQ && TIM_X_NFIELDS == tim::kXOutFields &&
                      TIM_X_RATIO_Q == tim::kXOutRatioQ && TIM_X_ABS_Q == tim::kXOutAbsQ,
                  "extras layout");
    if (n < 0 || !p || isnan(p->tok_tau)) return TIM_EINVAL;
    if (p->n_ratio_q < 0 || p->n_abs_q < 0 || p->n_ratio_q + p->n_abs_q > TIM_X_MAX_Q)
        return TIM_EINVAL;
    for (int i = 0; i < p->n_ratio_q; ++i)
        if (!(p->ratio_q[i] >= 0.0 && p->ratio_q[i] <= 1.0)) return TIM_EINVAL;
    for (int i = 0; i < p->n_abs_q; ++i)
        if (!(p->abs_q[i] >= 0.0 && p->abs_q[i] <= 1.0)) return TIM_EINVAL;
    if (n > 0 && (!logp_train || !logp_rollout)) return TIM_EINVAL;
    tim::ExtrasPlan plan;
    if (!tim::make_extras_plan(n, &plan)) return TIM_EUNSUPPORTED;
    if (!workspace || workspace_bytes < plan.total_bytes) return TIM_EWORKSPACE;
    if (!aligned(workspace, 256)) return TIM_EUNSUPPORTED;
    tim::XParamsDev prm{};
    prm.tok_tau = p->tok_tau;
    prm.nrq = p->n_ratio_q;
    prm.naq = p->n_abs_q;
    for (int i = 0; i < tim::kXMaxQ; ++i) {
        prm.rq[i] = i < p->n_ratio_q ? p->ratio_q[i] : 0.0;
        prm.aq[i] = i < p->n_abs_q ? p->abs_q[i] : 0.0;
    }
    if (tim::launch_mismatch_extras(plan, logp_train, logp_rollout, mask, prm, out, workspace,
                                    (hipStream_t)stream) != hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

size_t tim_logprob_backward_workspace_bytes(int64_t n, int64_t d, int64_t v, int dtype) {
    if (dtype != TIM_BF16 && dtype != TIM_F32) return 0;
    tim::BackwardPlan p;
    if (!tim::make_backward_plan(n, d, v, dtype, &p)) return 0;
    return p.total_bytes;
}

int tim_logprob_backward(const void* h, int64_t ldh, const void* w, int64_t ldw,
                         const int32_t* ids, const float* lse, const float* grad_logp,
                         int64_t n, int64_t d, int64_t v, int dtype, unsigned flags,
                         float* dh, float* dw, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (n < 0 || d <= 0 || v <= 0 || v > INT32_MAX || (dtype != TIM_BF16 && dtype != TIM_F32) ||
        flags > TIM_BWD_ACCUMULATE_DW)
        return TIM_EINVAL;
    if (ldh < d || ldw < d) return TIM_EINVAL;
    if ((dh && !aligned(dh, 16)) || (dw && !aligned(dw, 16))) return TIM_EUNSUPPORTED;
    if (n == 0 && !(dw && !(flags & TIM_BWD_ACCUMULATE_DW))) return TIM_OK;
    if (!w || (n > 0 && (!h || !ids || !lse || !grad_logp))) return TIM_EINVAL;
    if (d % 64 != 0) return TIM_EUNSUPPORTED;
    const int64_t esz = dtype == TIM_BF16 ? 2 : 4;
    if ((ldh * esz) % 16 != 0 || (ldw * esz) % 16 != 0) return TIM_EUNSUPPORTED;
    if ((h && !aligned(h, 16)) || !aligned(w, 16)) return TIM_EUNSUPPORTED;
    if (n > INT32_MAX) return TIM_EUNSUPPORTED;
    tim::BackwardPlan p;
    if (!tim::make_backward_plan(n, d, v, dtype, &p)) return TIM_EINVAL;
    // the three GEMMs' row tiles: W and h (K = D), dz and W (K = Vp, rows of
    // Vp elements), h^T and dz (K = Np, rows of Np elements)
    if (!tile_extent_ok(tim::kTileV, ldw * esz, d * esz) ||
        !tile_extent_ok(tim::kTileT, ldh * esz, d * esz) ||
        !tile_extent_ok(tim::kTileV, p.vpad * esz, p.vpad * esz) ||
        !tile_extent_ok(tim::kTileV, p.npad * esz, p.npad * esz))
        return TIM_EUNSUPPORTED;
    if (!workspace || workspace_bytes < p.total_bytes) return TIM_EWORKSPACE;
    if (!aligned(workspace, 256)) return TIM_EUNSUPPORTED;
    if (n == 0) {
        // a batch with no token: dh is empty and dw's sums are zero
        if (tim::launch_fill_zero(dw, v * d, (hipStream_t)stream) != hipSuccess) return TIM_EHIP;
        return TIM_OK;
    }
    if (tim::launch_logprob_backward(p, h, ldh, w, ldw, ids, lse, grad_logp, dh, dw,
                                     (flags & TIM_BWD_ACCUMULATE_DW) != 0, workspace,
                                     (hipStream_t)stream) != hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

size_t tim_ppo_workspace_bytes(int64_t n) {
    if (n < 0) return 0;
    return tim::ppo_workspace_bytes();
}

int tim_ppo_loss(const float* logp, const float* logp_old_train, const float* logp_old_rollout,
                 const float* advantages, const uint8_t* mask, int64_t n,
                 const tim_ppo_params* p, const tim_ppo_token_out* tok, double* batch,
                 void* workspace, size_t workspace_bytes, void* stream) {
    static_assert(TIM_P_NFIELDS == tim::kPpoOutFields, "ppo layout");
    if (n < 0 || !p) return TIM_EINVAL;
    if (!(p->eps_low >= 0.0) || !(p->eps_high >= 0.0) || isnan(p->tis_c) ||
        (p->bypass != 0 && p->bypass != 1) || !(p->grad_scale >= 0.0) || isinf(p->grad_scale))
        return TIM_EINVAL;
    if (n > 0 && (!logp || !logp_old_train || !logp_old_rollout || !advantages)) return TIM_EINVAL;
    if (!workspace || workspace_bytes < tim::ppo_workspace_bytes()) return TIM_EWORKSPACE;
    if (!aligned(workspace, 256)) return TIM_EUNSUPPORTED;
    tim_ppo_token_out t{};
    if (tok) t = *tok;
    if (tim::launch_ppo_loss(logp, logp_old_train, logp_old_rollout, advantages, mask, n,
                             p->eps_low, p->eps_high, p->bypass, p->tis_c, p->grad_scale,
                             t.loss, t.grad,
                             t.ratio, t.contrib, t.clipped, batch, workspace,
                             (hipStream_t)stream) != hipSuccess)
        return TIM_EHIP;
    return TIM_OK;
}

}  // extern "C"
