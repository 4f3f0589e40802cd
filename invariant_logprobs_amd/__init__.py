"""Batch-invariant selected-token log-probabilities and train/rollout mismatch
statistics on AMD Instinct MI355X (gfx950).

This module is the thin Python binding of ``libtim.so`` (C ABI in
``include/tim.h``).  It only marshals arguments: tensors must already live in
GPU memory, torch supplies the allocation of outputs and workspace and the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no CPU path: if the library is not built, or a tensor
is not on the GPU, a call raises.

Entry points (same names as the C ABI):

* :func:`tim_logprob_forward` -- ``logp[t] = log softmax(h[t] W^T)[ids[t]]``
  ("RL: Training Inference Mismatch", section "log p").
* :func:`tim_logprob_forward_ex` -- the same at a sampling temperature
  (``softmax(z / tau)``: "RL: Training Inference Mismatch", logits-processor
  section), with the entropy of that distribution and an optional RMSNorm
  of the input rows in front of the head.
* :func:`tim_rmsnorm` -- batch-invariant RMSNorm ("训推一致性与
  determinism", section 6 kernel table; VeXact methodology).
* :func:`tim_mismatch_stats` -- delta, ratio, k1/k2/k3, truncated IS weight,
  per-sequence means and geometric-mean-ratio rejection, batch aggregates
  ("Diagnosing Training Inference Mismatch ... (VeXact)", eq. (1) and its
  compensation table; "Train-Inference Consistency", sections 4-5), and the
  K3 form of the sequence rejection (srs-k3 rows of the same table).
* :func:`tim_logprob_backward` -- ``dh``, ``dW`` of ``L`` through the
  selected-token log-probability ("RL: Training Inference Mismatch", "log p"
  chain differentiated), deterministic, no atomics.
* :func:`tim_ppo_loss` -- the clipped surrogate with recompute / bypass
  ratios, truncated-r_corr TIS weight and zero-centred contribution
  (VeXact eqs. (2), (3), (5) and compensation table).
* :func:`tim_mismatch_extras` -- extreme-token rate, quantiles of the ratio
  and of ``|delta|`` ("训推一致性与 determinism", section 7, metric table)
  and the masked mean relative difference ("RL: Training Inference
  Mismatch", training/inference consistency).
"""
from __future__ import annotations

import ctypes
import functools
import math
import os
import threading
from typing import Optional

import torch

from .build import LIB_PATH

TIM_OK, TIM_EINVAL, TIM_EUNSUPPORTED, TIM_EWORKSPACE, TIM_EHIP, TIM_ESCRATCH = range(6)
TIM_BF16, TIM_F32 = 0, 1
TIM_SCHED_INVARIANT, TIM_SCHED_FREE, TIM_SCHED_SPLIT_K = 0, 1, 2
_SCHEDULES = {"invariant": TIM_SCHED_INVARIANT, "free": TIM_SCHED_FREE,
              "split_k": TIM_SCHED_SPLIT_K}

# Names of the batch aggregate vector, in TIM_B_* index order.  The
# is_approx_k3_kl / is_clip_ratio / is_nan_ratio names are the monitoring
# metrics of "Train-Inference Consistency", section 5.
BATCH_FIELDS = (
    "tok_mean_delta", "tok_mean_k1", "tok_mean_k2", "is_approx_k3_kl",
    "seq_mean_delta", "seq_mean_k1", "seq_mean_k2", "seq_mean_k3",
    "tok_mean_tis_w", "is_clip_ratio", "is_nan_ratio", "reject_frac",
    "mean_abs_delta", "max_abs_delta", "n_valid", "n_nan", "n_clipped",
    "n_seq_nonempty", "n_seq_rejected", "reject_k3_frac", "n_seq_rejected_k3",
)

# Names of the tim_mismatch_extras output vector, in TIM_X_* index order.
EXTRAS_FIELDS = (
    "n_valid", "n_extreme", "extreme_frac", "mean_rel_diff",
    "ratio_q0", "ratio_q1", "ratio_q2", "ratio_q3",
    "abs_q0", "abs_q1", "abs_q2", "abs_q3",
)
X_MAX_Q = 4
ABI_VERSION = 5
# Bytes of the static per-device scratch of tim_logprob_forward_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20
TIM_BWD_ACCUMULATE_DW = 1

# Names of the tim_ppo_loss batch vector, in TIM_P_* index order.
PPO_FIELDS = ("mean_loss", "clip_frac", "mean_ratio", "mean_tis_w", "mean_contrib",
              "n_valid", "n_clipped", "n_nan")

# Exported symbols of libtim.so (checked against include/tim.h by the tests).
EXPORTS = ("tim_abi_version", "tim_status_string", "tim_logprob_workspace_bytes",
           "tim_logprob_forward", "tim_stats_workspace_bytes", "tim_mismatch_stats",
           "tim_extras_workspace_bytes", "tim_mismatch_extras",
           "tim_logprob_backward_workspace_bytes", "tim_logprob_backward",
           "tim_ppo_workspace_bytes", "tim_ppo_loss", "tim_rmsnorm",
           "tim_logprob_ex_workspace_bytes", "tim_logprob_forward_ex",
           "tim_logprob_forward_noalloc")


class TimError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class _StatsParams(ctypes.Structure):
    _fields_ = [("tis_clip_c", ctypes.c_double), ("seq_lo", ctypes.c_double),
                ("seq_hi", ctypes.c_double), ("seq_k3_hi", ctypes.c_double)]


class _ExtrasParams(ctypes.Structure):
    _fields_ = [("tok_tau", ctypes.c_double), ("n_ratio_q", ctypes.c_int32),
                ("n_abs_q", ctypes.c_int32), ("ratio_q", ctypes.c_double * X_MAX_Q),
                ("abs_q", ctypes.c_double * X_MAX_Q)]


class _ForwardParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_double), ("norm_gamma", ctypes.c_void_p),
                ("norm_eps", ctypes.c_double)]


class _PpoParams(ctypes.Structure):
    _fields_ = [("eps_low", ctypes.c_double), ("eps_high", ctypes.c_double),
                ("bypass", ctypes.c_int32), ("tis_c", ctypes.c_double),
                ("grad_scale", ctypes.c_double)]


class _PpoTokenOut(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ("loss", "grad", "ratio", "contrib", "clipped")]


class _TokenOut(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("delta", "ratio", "k1", "k2", "k3", "tis_w", "clipped")]


class _SeqOut(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("n_valid", "n_clipped", "n_nan", "mean_delta", "mean_k1", "mean_k2",
                 "mean_k3", "mean_tis_w", "reject", "reject_k3")]


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libtim.so (built by ``invariant_logprobs_amd.build``); raise if absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m invariant_logprobs_amd.build` "
                               "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        lib.tim_abi_version.restype = ctypes.c_int
        lib.tim_status_string.restype = ctypes.c_char_p
        lib.tim_status_string.argtypes = [ctypes.c_int]
        lib.tim_logprob_workspace_bytes.restype = sz
        lib.tim_logprob_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_uint]
        lib.tim_logprob_forward.restype = ctypes.c_int
        lib.tim_logprob_forward.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, ctypes.c_int,
                                            ctypes.c_uint, vp, vp, vp, vp, sz, vp]
        lib.tim_logprob_forward_noalloc.restype = ctypes.c_int
        lib.tim_logprob_forward_noalloc.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64,
                                                    ctypes.c_int, ctypes.c_uint, vp, vp, vp, vp]
        lib.tim_rmsnorm.restype = ctypes.c_int
        lib.tim_rmsnorm.argtypes = [vp, i64, vp, i64, i64, ctypes.c_int, ctypes.c_double, vp, i64,
                                    vp, vp]
        lib.tim_logprob_ex_workspace_bytes.restype = sz
        lib.tim_logprob_ex_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_uint,
                                                       ctypes.POINTER(_ForwardParams), ctypes.c_int]
        lib.tim_logprob_forward_ex.restype = ctypes.c_int
        lib.tim_logprob_forward_ex.argtypes = [vp, i64, vp, i64, vp, i64, i64, i64, ctypes.c_int,
                                               ctypes.c_uint, ctypes.POINTER(_ForwardParams), vp,
                                               vp, vp, vp, vp, sz, vp]
        lib.tim_stats_workspace_bytes.restype = sz
        lib.tim_stats_workspace_bytes.argtypes = [i64, i64]
        lib.tim_mismatch_stats.restype = ctypes.c_int
        lib.tim_mismatch_stats.argtypes = [vp, vp, vp, vp, i64, i64,
                                           ctypes.POINTER(_StatsParams),
                                           ctypes.POINTER(_TokenOut), ctypes.POINTER(_SeqOut),
                                           vp, vp, sz, vp]
        lib.tim_extras_workspace_bytes.restype = sz
        lib.tim_extras_workspace_bytes.argtypes = [i64]
        lib.tim_mismatch_extras.restype = ctypes.c_int
        lib.tim_mismatch_extras.argtypes = [vp, vp, vp, i64, ctypes.POINTER(_ExtrasParams), vp,
                                            vp, sz, vp]
        lib.tim_logprob_backward_workspace_bytes.restype = sz
        lib.tim_logprob_backward_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
        lib.tim_logprob_backward.restype = ctypes.c_int
        lib.tim_logprob_backward.argtypes = [vp, i64, vp, i64, vp, vp, vp, i64, i64, i64,
                                             ctypes.c_int, ctypes.c_uint, vp, vp, vp, sz, vp]
        lib.tim_ppo_workspace_bytes.restype = sz
        lib.tim_ppo_workspace_bytes.argtypes = [i64]
        lib.tim_ppo_loss.restype = ctypes.c_int
        lib.tim_ppo_loss.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.POINTER(_PpoParams),
                                     ctypes.POINTER(_PpoTokenOut), vp, vp, sz, vp]
        if lib.tim_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.tim_abi_version()}, "
                               f"expected {ABI_VERSION}: rebuild it")
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().tim_status_string(int(status)).decode()


def _dptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _require_gpu(name: str, t: torch.Tensor):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a torch tensor in GPU memory")


def _stream_handle(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on_stream(fn):
    """Run a wrapper on the caller's ``stream=`` (a ``torch.cuda.Stream``)
    with torch's stream-ordered memory rules kept:

    * the given stream first waits for torch's current stream, so inputs
      written there are complete before the library reads them;
    * outputs and any internal workspace are allocated while the given
      stream is current, so torch's caching allocator ties them to it (an
      internal workspace freed on return is only reused by later work on
      the same stream, which runs after these kernels);
    * every tensor argument (inputs, ``out``, ``workspace``, ``dw``) is
      recorded on the given stream, so its memory is not handed to another
      allocation before the stream's kernels are done with it.

    Results live on the given stream: a caller that reads them on another
    stream makes that stream wait first, as with any torch tensor."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        if not isinstance(stream, torch.cuda.Stream):
            raise TypeError("stream must be a torch.cuda.Stream")
        cur = torch.cuda.current_stream(stream.device)
        if stream == cur:
            return fn(*args, **kwargs)
        stream.wait_stream(cur)
        with torch.cuda.stream(stream):
            res = fn(*args, **kwargs)
        for t in list(args) + list(kwargs.values()):
            if isinstance(t, torch.Tensor) and t.is_cuda:
                t.record_stream(stream)
        return res
    return wrapper


_DTYPES = {torch.bfloat16: TIM_BF16, torch.float32: TIM_F32}


def logprob_workspace_bytes(n: int, d: int, v: int, dtype: int, schedule: str = "invariant") -> int:
    flags = _SCHEDULES[schedule]
    return int(load_library().tim_logprob_workspace_bytes(n, d, v, dtype, flags))


def stats_workspace_bytes(n: int, s: int) -> int:
    return int(load_library().tim_stats_workspace_bytes(n, s))


@_on_stream
def tim_logprob_forward(h: torch.Tensor, w: torch.Tensor, ids: torch.Tensor, *,
                        schedule: str = "invariant", return_lse: bool = False,
                        out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """Selected-token log-probabilities ``logp[t] = log softmax(h[t] W^T)[ids[t]]``.

    ``h``: [N, D] and ``w``: [V, D], both bf16 or both fp32, rows contiguous
    (a leading dimension larger than D is allowed via a strided 2-D view).
    ``ids``: [N] int32.  Returns ``logp`` (fp32 [N]) or, with
    ``return_lse``, ``(logp, lse, n_bad_ids)``.  Asynchronous on ``stream``
    (default: torch's current stream).
    """
    lib = load_library()
    n, d, v = _check_forward_args(h, w, ids)
    dtype = _DTYPES[h.dtype]
    flags = _SCHEDULES[schedule]
    dev = h.device
    logp = out if out is not None else torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if return_lse else None
    nbad = torch.zeros(1, dtype=torch.int32, device=dev) if return_lse else None
    need = lib.tim_logprob_workspace_bytes(n, d, v, dtype, flags)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    st = lib.tim_logprob_forward(_dptr(h), h.stride(0), _dptr(w), w.stride(0), _dptr(ids),
                                 n, d, v, dtype, flags, _dptr(logp), _dptr(lse), _dptr(nbad),
                                 _dptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_logprob_forward")
    if return_lse:
        return logp, lse, nbad
    return logp


def _check_forward_args(h, w, ids):
    for name, t in (("h", h), ("w", w), ("ids", ids)):
        _require_gpu(name, t)
    if h.dtype not in _DTYPES or w.dtype != h.dtype:
        raise ValueError("h and w must share dtype bfloat16 or float32")
    if h.dim() != 2 or w.dim() != 2 or h.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("h and w must be 2-D with unit stride along D")
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous 1-D int32 tensor")
    n, d = h.shape
    v, d2 = w.shape
    if d2 != d or ids.shape[0] != n:
        raise ValueError(f"shape mismatch: h {tuple(h.shape)}, w {tuple(w.shape)}, ids {tuple(ids.shape)}")
    return n, d, v


def _check_out(name, t, n, dtype, dev):
    if t is not None and (not isinstance(t, torch.Tensor) or t.device != dev or t.dtype != dtype
                          or t.dim() != 1 or t.shape[0] < n or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous 1-D {dtype} tensor of at least {n} "
                         f"entries on {dev}")


@_on_stream
def tim_logprob_forward_noalloc(h: torch.Tensor, w: torch.Tensor, ids: torch.Tensor, *,
                                out: torch.Tensor, lse_out: Optional[torch.Tensor] = None,
                                n_bad_ids_out: Optional[torch.Tensor] = None,
                                schedule: str = "invariant", stream=None):
    """``tim_logprob_forward`` with the library's static per-device scratch
    instead of a workspace: no device memory is allocated, here or in the
    library.  The caller passes every output: ``out`` (fp32 [N]) and,
    optionally, ``lse_out`` (fp32 [N]) and ``n_bad_ids_out`` (int32 [1]).
    Raises ``TimError`` with ``TIM_ESCRATCH`` when the request needs more
    than ``NOALLOC_SCRATCH_BYTES``.  Calls that can overlap on one device
    race on the shared scratch."""
    lib = load_library()
    n, d, v = _check_forward_args(h, w, ids)
    dev = h.device
    _check_out("out", out, n, torch.float32, dev)
    if out is None:
        raise ValueError("out is required")
    _check_out("lse_out", lse_out, n, torch.float32, dev)
    _check_out("n_bad_ids_out", n_bad_ids_out, 1, torch.int32, dev)
    st = lib.tim_logprob_forward_noalloc(_dptr(h), h.stride(0), _dptr(w), w.stride(0),
                                         _dptr(ids), n, d, v, _DTYPES[h.dtype],
                                         _SCHEDULES[schedule], _dptr(out), _dptr(lse_out),
                                         _dptr(n_bad_ids_out), _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_logprob_forward_noalloc")
    return out


@_on_stream
def tim_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, *, eps: float = 1e-6,
                out: Optional[torch.Tensor] = None, return_rstd: bool = False, stream=None):
    """``y = gamma * x / sqrt(mean(x^2) + eps)`` per row of ``x`` [N, D]
    (bf16 or fp32, unit stride along D; ``gamma`` [D] of the same dtype).
    Returns ``y`` (same dtype, [N, D]) or ``(y, rstd)``."""
    lib = load_library()
    _require_gpu("x", x)
    _require_gpu("gamma", gamma)
    if x.dtype not in _DTYPES or gamma.dtype != x.dtype:
        raise ValueError("x and gamma must share dtype bfloat16 or float32")
    if x.dim() != 2 or x.stride(1) != 1 or gamma.dim() != 1 or not gamma.is_contiguous():
        raise ValueError("x must be 2-D with unit stride along D, gamma 1-D contiguous")
    n, d = x.shape
    if gamma.shape[0] != d:
        raise ValueError("gamma must have D entries")
    y = out if out is not None else torch.empty(n, d, dtype=x.dtype, device=x.device)
    if y.shape != (n, d) or y.dtype != x.dtype or y.stride(1) != 1:
        raise ValueError("out must be [N, D] of x's dtype with unit stride along D")
    rstd = torch.empty(n, dtype=torch.float32, device=x.device) if return_rstd else None
    st = lib.tim_rmsnorm(_dptr(x), x.stride(0), _dptr(gamma), n, d, _DTYPES[x.dtype], float(eps),
                         _dptr(y), y.stride(0), _dptr(rstd), _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_rmsnorm")
    return (y, rstd) if return_rstd else y


def logprob_ex_workspace_bytes(n: int, d: int, v: int, dtype: int, *, temperature: float = 1.0,
                               norm: bool = False, entropy: bool = False,
                               schedule: str = "invariant") -> int:
    flags = _SCHEDULES[schedule]
    prm = _ForwardParams(float(temperature), 1 if norm else None, 1e-6)
    return int(load_library().tim_logprob_ex_workspace_bytes(n, d, v, dtype, flags,
                                                             ctypes.byref(prm), int(entropy)))


@_on_stream
def tim_logprob_forward_ex(h: torch.Tensor, w: torch.Tensor, ids: torch.Tensor, *,
                           temperature: float = 1.0, norm_gamma: Optional[torch.Tensor] = None,
                           norm_eps: float = 1e-6, entropy: bool = False,
                           schedule: str = "invariant", workspace: Optional[torch.Tensor] = None,
                           stream=None) -> dict:
    """Scores at temperature ``tau``: ``logp = log softmax(z / tau)[ids]``
    with ``z = W norm(h)`` when ``norm_gamma`` is given (``h`` then holds the
    pre-norm rows), else ``z = W h``.  Returns a dict of GPU tensors:
    ``logp``, ``lse``, ``n_bad_ids`` and, with ``entropy``, ``entropy``."""
    lib = load_library()
    for name, t in (("h", h), ("w", w), ("ids", ids)):
        _require_gpu(name, t)
    if h.dtype not in _DTYPES or w.dtype != h.dtype:
        raise ValueError("h and w must share dtype bfloat16 or float32")
    if h.dim() != 2 or w.dim() != 2 or h.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("h and w must be 2-D with unit stride along D")
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous 1-D int32 tensor")
    n, d = h.shape
    v, d2 = w.shape
    if d2 != d or ids.shape[0] != n:
        raise ValueError(f"shape mismatch: h {tuple(h.shape)}, w {tuple(w.shape)}, ids {tuple(ids.shape)}")
    if norm_gamma is not None:
        _require_gpu("norm_gamma", norm_gamma)
        if norm_gamma.dtype != h.dtype or norm_gamma.shape != (d,) or not norm_gamma.is_contiguous():
            raise ValueError("norm_gamma must be a contiguous [D] tensor of h's dtype")
    dtype = _DTYPES[h.dtype]
    flags = _SCHEDULES[schedule]
    dev = h.device
    res = {"logp": torch.empty(n, dtype=torch.float32, device=dev),
           "lse": torch.empty(n, dtype=torch.float32, device=dev),
           "n_bad_ids": torch.zeros(1, dtype=torch.int32, device=dev)}
    if entropy:
        res["entropy"] = torch.empty(n, dtype=torch.float32, device=dev)
    prm = _ForwardParams(float(temperature), _dptr(norm_gamma), float(norm_eps))
    need = lib.tim_logprob_ex_workspace_bytes(n, d, v, dtype, flags, ctypes.byref(prm),
                                              int(entropy))
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    st = lib.tim_logprob_forward_ex(_dptr(h), h.stride(0), _dptr(w), w.stride(0), _dptr(ids),
                                    n, d, v, dtype, flags, ctypes.byref(prm), _dptr(res["logp"]),
                                    _dptr(res["lse"]), _dptr(res.get("entropy")),
                                    _dptr(res["n_bad_ids"]), _dptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_logprob_forward_ex")
    return res


@_on_stream
def tim_mismatch_stats(logp_train: torch.Tensor, logp_rollout: torch.Tensor,
                       mask: Optional[torch.Tensor], cu_seqlens: torch.Tensor, *,
                       tis_clip: float = 2.0, seq_bounds=(-0.01, 0.01),
                       seq_k3_max: float = math.inf,
                       token_outputs: bool = False, seq_outputs: bool = True,
                       check_cu_seqlens: bool = False,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Mismatch statistics between trainer and rollout log-probabilities.

    ``cu_seqlens`` must satisfy 0 = c0 <= c1 <= ... <= cs = n; the device does
    not check it (offsets outside [0, n] are clamped).  ``check_cu_seqlens``
    copies it to the host and raises ``ValueError`` if it does not (a debug
    aid: it synchronises with the device).

    ``seq_bounds`` are log-domain bounds on a sequence's mean delta; a
    geometric-mean-ratio window ``[a, b]`` is ``(log a, log b)``.  A sequence
    whose mean k3 exceeds ``seq_k3_max`` is K3-rejected (``inf``: never).  Returns a
    dict with ``"batch"`` (a tensor of ``len(BATCH_FIELDS)`` fp64 values on the
    GPU), and optionally ``"seq"`` and ``"token"`` dicts of GPU tensors.
    """
    lib = load_library()
    for name, t in (("logp_train", logp_train), ("logp_rollout", logp_rollout),
                    ("cu_seqlens", cu_seqlens)):
        _require_gpu(name, t)
    if mask is not None:
        _require_gpu("mask", mask)
        if mask.dtype != torch.uint8 or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 tensor")
    if logp_train.dtype != torch.float32 or logp_rollout.dtype != torch.float32:
        raise ValueError("log-probabilities must be float32")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor")
    if not (logp_train.is_contiguous() and logp_rollout.is_contiguous()):
        raise ValueError("log-probabilities must be contiguous")
    n = logp_train.numel()
    s = cu_seqlens.numel() - 1
    if logp_rollout.numel() != n or (mask is not None and mask.numel() != n) or s < 0:
        raise ValueError("inconsistent sizes")
    if check_cu_seqlens:
        _check_cu_seqlens(cu_seqlens, n)
    dev = logp_train.device
    res = {}
    batch = torch.empty(len(BATCH_FIELDS), dtype=torch.float64, device=dev)
    res["batch"] = batch
    tok = None
    if token_outputs:
        t = {k: torch.empty(n, dtype=torch.float32, device=dev)
             for k in ("delta", "ratio", "k1", "k2", "k3", "tis_w")}
        t["clipped"] = torch.empty(n, dtype=torch.uint8, device=dev)
        res["token"] = t
        tok = _TokenOut(*[_dptr(t[k]) for k in ("delta", "ratio", "k1", "k2", "k3", "tis_w",
                                                 "clipped")])
    seq = None
    if seq_outputs:
        q = {k: torch.empty(s, dtype=torch.int32, device=dev)
             for k in ("n_valid", "n_clipped", "n_nan")}
        q.update({k: torch.empty(s, dtype=torch.float64, device=dev)
                  for k in ("mean_delta", "mean_k1", "mean_k2", "mean_k3", "mean_tis_w")})
        q["reject"] = torch.empty(s, dtype=torch.uint8, device=dev)
        q["reject_k3"] = torch.empty(s, dtype=torch.uint8, device=dev)
        res["seq"] = q
        seq = _SeqOut(*[_dptr(q[k]) for k in ("n_valid", "n_clipped", "n_nan", "mean_delta",
                                               "mean_k1", "mean_k2", "mean_k3", "mean_tis_w",
                                               "reject", "reject_k3")])
    need = lib.tim_stats_workspace_bytes(n, s)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    prm = _StatsParams(float(tis_clip), float(seq_bounds[0]), float(seq_bounds[1]),
                       float(seq_k3_max))
    st = lib.tim_mismatch_stats(_dptr(logp_train), _dptr(logp_rollout), _dptr(mask),
                                _dptr(cu_seqlens), n, s, ctypes.byref(prm),
                                ctypes.byref(tok) if tok is not None else None,
                                ctypes.byref(seq) if seq is not None else None,
                                _dptr(batch), _dptr(workspace),
                                workspace.numel() * workspace.element_size(),
                                _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_mismatch_stats")
    return res


def _check_cu_seqlens(cu_seqlens: torch.Tensor, n: int):
    c = cu_seqlens.to("cpu").tolist()
    if not c or c[0] != 0 or c[-1] != n:
        raise ValueError(f"cu_seqlens must start at 0 and end at n = {n}")
    for j in range(1, len(c)):
        if c[j] < c[j - 1]:
            raise ValueError(f"cu_seqlens decreases at index {j}: {c[j - 1]} > {c[j]}")


def extras_workspace_bytes(n: int) -> int:
    return int(load_library().tim_extras_workspace_bytes(n))


@_on_stream
def tim_mismatch_extras(logp_train: torch.Tensor, logp_rollout: torch.Tensor,
                        mask: Optional[torch.Tensor], *, tok_tau: float,
                        ratio_q=(0.01, 0.5, 0.99), abs_q=(0.95,),
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Extreme-token rate, mean relative difference and quantiles.

    Returns a GPU fp64 tensor of ``len(EXTRAS_FIELDS)`` values; quantile
    ``ratio_q[i]`` of ``exp(delta)`` is at ``ratio_q{i}`` and quantile
    ``abs_q[i]`` of ``|delta|`` at ``abs_q{i}`` (see :func:`extras_dict`).
    """
    lib = load_library()
    _require_gpu("logp_train", logp_train)
    _require_gpu("logp_rollout", logp_rollout)
    if logp_train.dtype != torch.float32 or logp_rollout.dtype != torch.float32:
        raise ValueError("log-probabilities must be float32")
    if not (logp_train.is_contiguous() and logp_rollout.is_contiguous()):
        raise ValueError("log-probabilities must be contiguous")
    n = logp_train.numel()
    if logp_rollout.numel() != n:
        raise ValueError("inconsistent sizes")
    if mask is not None:
        _require_gpu("mask", mask)
        if mask.dtype != torch.uint8 or not mask.is_contiguous() or mask.numel() != n:
            raise ValueError("mask must be a contiguous uint8 tensor of n entries")
    ratio_q, abs_q = tuple(ratio_q), tuple(abs_q)
    if len(ratio_q) + len(abs_q) > X_MAX_Q:
        raise ValueError(f"at most {X_MAX_Q} probabilities per call")
    prm = _ExtrasParams(float(tok_tau), len(ratio_q), len(abs_q),
                        (ctypes.c_double * X_MAX_Q)(*(list(ratio_q) + [0.0] * (X_MAX_Q - len(ratio_q)))),
                        (ctypes.c_double * X_MAX_Q)(*(list(abs_q) + [0.0] * (X_MAX_Q - len(abs_q)))))
    dev = logp_train.device
    out = torch.empty(len(EXTRAS_FIELDS), dtype=torch.float64, device=dev)
    need = lib.tim_extras_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    st = lib.tim_mismatch_extras(_dptr(logp_train), _dptr(logp_rollout), _dptr(mask), n,
                                 ctypes.byref(prm), _dptr(out), _dptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_mismatch_extras")
    return out


def extras_dict(out: torch.Tensor, n_ratio_q: int = 3, n_abs_q: int = 1) -> dict:
    """Host dict of a tim_mismatch_extras output (synchronises)."""
    v = [float(x) for x in out.cpu().tolist()]
    res = dict(zip(EXTRAS_FIELDS[:4], v[:4]))
    res["ratio_q"] = v[4:4 + n_ratio_q]
    res["abs_q"] = v[8:8 + n_abs_q]
    return res


def backward_workspace_bytes(n: int, d: int, v: int, dtype: int = TIM_BF16) -> int:
    return int(load_library().tim_logprob_backward_workspace_bytes(n, d, v, dtype))


@_on_stream
def tim_logprob_backward(h: torch.Tensor, w: torch.Tensor, ids: torch.Tensor,
                         lse: torch.Tensor, grad_logp: torch.Tensor, *, want_dh: bool = True,
                         want_dw: bool = True, dw: Optional[torch.Tensor] = None,
                         accumulate_dw: bool = False, workspace: Optional[torch.Tensor] = None,
                         stream=None):
    """``(dh, dw)`` (fp32, ``[N, D]`` and ``[V, D]``) of ``L`` through
    ``logp = log softmax(h W^T)[ids]`` given ``grad_logp = dL/dlogp`` and the
    forward's ``lse``.  ``h`` and ``W`` both bf16 or both fp32.  With ``accumulate_dw`` the
    given ``dw`` is read and the sum over this batch's tokens continues from
    it."""
    lib = load_library()
    for name, t in (("h", h), ("w", w), ("ids", ids), ("lse", lse), ("grad_logp", grad_logp)):
        _require_gpu(name, t)
    if h.dtype != w.dtype or h.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("h and W must both be bfloat16 or both float32")
    dtype = TIM_BF16 if h.dtype == torch.bfloat16 else TIM_F32
    if h.dim() != 2 or w.dim() != 2 or h.shape[1] != w.shape[1]:
        raise ValueError("h must be [N, D] and w [V, D]")
    if h.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("h and w must have unit stride along D")
    n, d = h.shape
    v = w.shape[0]
    for name, t, dt in (("ids", ids, torch.int32), ("lse", lse, torch.float32),
                        ("grad_logp", grad_logp, torch.float32)):
        if t.dtype != dt or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous {dt} tensor of N entries")
    dev = h.device
    dh = torch.empty(n, d, dtype=torch.float32, device=dev) if want_dh else None
    if want_dw:
        if dw is None:
            if accumulate_dw:
                raise ValueError("accumulate_dw needs the dw tensor to continue from")
            dw = torch.empty(v, d, dtype=torch.float32, device=dev)
        elif dw.dtype != torch.float32 or not dw.is_contiguous() or tuple(dw.shape) != (v, d):
            raise ValueError("dw must be a contiguous fp32 [V, D] tensor")
    else:
        dw = None
    need = lib.tim_logprob_backward_workspace_bytes(n, d, v, dtype)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    flags = TIM_BWD_ACCUMULATE_DW if accumulate_dw else 0
    st = lib.tim_logprob_backward(_dptr(h), h.stride(0), _dptr(w), w.stride(0), _dptr(ids),
                                  _dptr(lse), _dptr(grad_logp), n, d, v, dtype, flags,
                                  _dptr(dh), _dptr(dw), _dptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_logprob_backward")
    return dh, dw


@_on_stream
def tim_ppo_loss(logp: torch.Tensor, logp_old_train: torch.Tensor,
                 logp_old_rollout: torch.Tensor, advantages: torch.Tensor,
                 mask: Optional[torch.Tensor], *, eps_low: float = 0.2, eps_high: float = 0.28,
                 bypass: bool = False, tis_c: float = 0.0, grad_scale: float = 0.0,
                 token_outputs: bool = True,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Clipped surrogate, gradient by ``logp`` of its token mean (or, with
    ``grad_scale > 0``, of ``grad_scale`` times its token sum, in one pass),
    ratios, zero-centred contributions and clip flags (GPU tensors), and the
    batch vector (``"batch"``, ``PPO_FIELDS`` order)."""
    lib = load_library()
    ins = (logp, logp_old_train, logp_old_rollout, advantages)
    for name, t in zip(("logp", "logp_old_train", "logp_old_rollout", "advantages"), ins):
        _require_gpu(name, t)
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    n = logp.numel()
    if any(t.numel() != n for t in ins):
        raise ValueError("inconsistent sizes")
    if mask is not None:
        _require_gpu("mask", mask)
        if mask.dtype != torch.uint8 or not mask.is_contiguous() or mask.numel() != n:
            raise ValueError("mask must be a contiguous uint8 tensor of n entries")
    dev = logp.device
    res = {"batch": torch.empty(len(PPO_FIELDS), dtype=torch.float64, device=dev)}
    tok = None
    if token_outputs:
        t = {k: torch.empty(n, dtype=torch.float32, device=dev)
             for k in ("loss", "grad", "ratio", "contrib")}
        t["clipped"] = torch.empty(n, dtype=torch.uint8, device=dev)
        res["token"] = t
        tok = _PpoTokenOut(*[_dptr(t[k]) for k in ("loss", "grad", "ratio", "contrib", "clipped")])
    need = lib.tim_ppo_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    prm = _PpoParams(float(eps_low), float(eps_high), int(bool(bypass)), float(tis_c),
                     float(grad_scale))
    st = lib.tim_ppo_loss(*[_dptr(x) for x in ins], _dptr(mask), n, ctypes.byref(prm),
                          ctypes.byref(tok) if tok is not None else None, _dptr(res["batch"]),
                          _dptr(workspace), workspace.numel() * workspace.element_size(),
                          _stream_handle(stream))
    if st != TIM_OK:
        raise TimError(st, "tim_ppo_loss")
    return res


def batch_dict(batch: torch.Tensor) -> dict:
    """Host dict {name: value} of a batch aggregate tensor (synchronises)."""
    return dict(zip(BATCH_FIELDS, (float(x) for x in batch.cpu().tolist())))


def log_window(lo_ratio: float, hi_ratio: float):
    """Log-domain bounds of a geometric-mean-ratio window ``[lo, hi]``."""
    return (math.log(lo_ratio), math.log(hi_ratio))
