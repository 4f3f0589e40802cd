"""fp64 CPU oracle for selected-token log-probabilities and mismatch statistics.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library
path (``invariant_logprobs_amd``) never imports it, and this package imports
nothing from the library: the two share no code.

The arithmetic lives in ``tim_oracle.c`` (plain C, fp64, sequential sums in
the order the definitions give).  This module only builds that file with gcc
and marshals numpy arrays into it.

Functions and the passages they follow:

* :func:`logprob` -- ``logp_t = z_t[a_t] - log sum_v exp z_t[v]`` with
  ``z_t = W h_t``: "RL: Training Inference Mismatch", section "log p".
* :func:`logprob_ex` -- the same at a sampling temperature ``tau`` (the
  softmax of ``z / tau``) with the entropy of that distribution: "RL:
  Training Inference Mismatch", logits-processor section; entropy as a
  monitored quantity: "训推一致性与 determinism", section 2.
* :func:`rmsnorm` -- ``y = gamma * x / sqrt(mean(x^2) + eps)`` per row
  ("训推一致性与 determinism", section 6 kernel table; VeXact methodology,
  batch-invariant RMSNorm).
* :func:`mismatch_stats` -- token-level TIM ``delta = train - rollout``
  ("Diagnosing Training Inference Mismatch ... (VeXact)", eq. (1)), ratio,
  k1/k2/k3 ("RL: Training Inference Mismatch", KL-estimator table), TIS
  weight and clip flag ("Train-Inference Consistency", section 4), per-sequence
  and batch means (same "RL" page, monitoring flow), geometric-mean-ratio
  rejection and its K3 form (VeXact compensation table, srs-k1 / srs-k3).
* :func:`mismatch_extras` -- extreme-token rate, quantiles of the ratio and
  of ``|delta|`` ("训推一致性与 determinism", section 7, metric table) and
  the masked mean of ``|lt - lr| / (|lt| + 1e-8)`` ("RL: Training Inference
  Mismatch", training/inference consistency).
* :func:`logprob_backward` -- ``dz = g ([v == a] - softmax(z))``, ``dh = dz W``,
  ``dW = dz^T h``: the "log p" chain of "RL: Training Inference Mismatch",
  differentiated.
* :func:`ppo_loss` -- the clipped surrogate (VeXact eq. (2)) with the
  recompute / bypass ratios (eq. (3)), the truncated-r_corr TIS weight (its
  compensation table), the zero-centred contribution (eq. (5)) and the
  gradient by the log-probability.
* :func:`bf16_decode`, :func:`bf16_round_rne` -- bf16 <-> double, ties to
  even ("Train-infer mismatch for Open-weight MoE RL", figure "Rounding
  depends on the order of additions").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tim_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_OUT_DIR, "libtim_oracle.so")

BF16 = 0
F32 = 1
# default thread cap: the oracle shares its host with the GPU job
MAX_THREADS = 16

# Batch vector field names, in index order (restated from the definitions;
# not imported from the library).
BATCH_FIELDS = (
    "tok_mean_delta", "tok_mean_k1", "tok_mean_k2", "tok_mean_k3",
    "seq_mean_delta", "seq_mean_k1", "seq_mean_k2", "seq_mean_k3",
    "tok_mean_tis_w", "clip_ratio", "nan_ratio", "reject_frac",
    "mean_abs_delta", "max_abs_delta", "n_valid", "n_nan", "n_clipped",
    "n_seq_nonempty", "n_seq_rejected", "reject_k3_frac", "n_seq_rejected_k3",
)
# Output vector of :func:`mismatch_extras`, in index order.
EXTRAS_FIELDS = (
    "n_valid", "n_extreme", "extreme_frac", "mean_rel_diff",
    "ratio_q0", "ratio_q1", "ratio_q2", "ratio_q3",
    "abs_q0", "abs_q1", "abs_q2", "abs_q3",
)
MAX_Q = 4
# Batch vector of :func:`ppo_loss`, in index order.
PPO_FIELDS = ("mean_loss", "clip_frac", "mean_ratio", "mean_tis_w", "mean_contrib",
              "n_valid", "n_clipped", "n_nan")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile ``tim_oracle.c`` into ``_build/libtim_oracle.so`` with gcc."""
    os.makedirs(_OUT_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = build(force=False)
        lib = ctypes.CDLL(path)
        c_i64, c_int, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.or_bf16_decode.restype = ctypes.c_double
        lib.or_bf16_decode.argtypes = [ctypes.c_uint16]
        lib.or_bf16_round_rne.restype = ctypes.c_uint16
        lib.or_bf16_round_rne.argtypes = [ctypes.c_double]
        lib.or_available_cpus.restype = c_int
        lib.or_batch_nfields.restype = c_int
        lib.or_logprob_rows_ex.restype = c_int
        lib.or_logprob_rows_ex.argtypes = [vp, c_i64, vp, c_i64, vp, c_int, c_i64,
                                           c_i64, vp, c_i64, ctypes.c_double, vp, vp, vp, vp,
                                           c_int]
        lib.or_rmsnorm.restype = c_int
        lib.or_rmsnorm.argtypes = [vp, c_i64, vp, c_int, c_i64, c_i64, ctypes.c_double, vp, vp]
        lib.or_bf16_round_rne_n.restype = None
        lib.or_bf16_round_rne_n.argtypes = [vp, vp, c_i64]
        lib.or_logprob_rows.restype = c_int
        lib.or_logprob_rows.argtypes = [vp, c_i64, vp, c_i64, vp, c_int, c_i64,
                                        c_i64, vp, c_i64, vp, vp, vp, c_int]
        lib.or_mismatch_stats.restype = c_int
        lib.or_mismatch_stats.argtypes = [vp, vp, vp, vp, c_i64, c_i64,
                                          ctypes.c_double, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double] + [vp] * 18
        lib.or_mismatch_extras.restype = c_int
        lib.or_mismatch_extras.argtypes = [vp, vp, vp, c_i64, ctypes.c_double, vp, c_int,
                                           vp, c_int, vp]
        lib.or_extras_nfields.restype = c_int
        lib.or_logprob_backward.restype = c_int
        lib.or_logprob_backward.argtypes = [vp, c_i64, vp, c_i64, vp, vp, c_int, c_i64, c_i64,
                                            c_i64, vp, c_i64, vp, vp, c_i64, vp, c_int]
        lib.or_ppo_loss.restype = c_int
        lib.or_ppo_loss.argtypes = [vp, vp, vp, vp, vp, c_i64, ctypes.c_double,
                                    ctypes.c_double, c_int, ctypes.c_double,
                                    ctypes.c_double] + [vp] * 6
        lib.or_ppo_nfields.restype = c_int
        assert lib.or_batch_nfields() == len(BATCH_FIELDS)
        assert lib.or_extras_nfields() == len(EXTRAS_FIELDS)
        assert lib.or_ppo_nfields() == len(PPO_FIELDS)
        _lib = lib
        return lib


def available_cpus() -> int:
    return int(_load().or_available_cpus())


def _ptr(a):
    return None if a is None else a.ctypes.data


def _as_host_array(x, dtype):
    """numpy (or CPU torch) -> C-contiguous numpy array of ``dtype``."""
    if hasattr(x, "detach"):  # torch tensor: raw bits for bf16
        import torch  # local: only needed when called with tensors
        x = x.detach().cpu()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16).numpy().view(np.uint16)
        else:
            x = x.numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def bf16_decode(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.or_bf16_decode(int(v)) for v in b], dtype=np.float64)


def bf16_round_rne(x) -> np.ndarray:
    """Bits of the bf16 nearest to each element (ties to even), same shape."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().or_bf16_round_rne_n(_ptr(a), _ptr(out), a.size)
    return out


def rmsnorm(x, gamma, *, dtype: int, eps: float):
    """fp64 ``(y [N, D], rstd [N])`` of ``y = gamma * x * rstd``,
    ``rstd = 1 / sqrt(mean(x^2) + eps)``.  bf16 inputs as uint16 bits (or
    bf16 torch tensors), fp32 as float32."""
    el = np.uint16 if dtype == BF16 else np.float32
    x = _as_host_array(x, el)
    gamma = _as_host_array(gamma, el)
    n, d = x.shape
    assert gamma.shape == (d,)
    y = np.empty((n, d), np.float64)
    rstd = np.empty(n, np.float64)
    if _load().or_rmsnorm(_ptr(x), d, _ptr(gamma), dtype, n, d, float(eps), _ptr(y),
                          _ptr(rstd)) != 0:
        raise ValueError("or_rmsnorm rejected its arguments")
    return y, rstd


def logprob_ex(h, w, ids, *, dtype: int, temperature: float = 1.0, rows=None,
               nthreads: int = 0) -> dict:
    """fp64 ``logp``, ``lse``, ``zsel`` (= ``z_a / tau``) and ``entropy`` of
    ``softmax(z / tau)`` for token rows ``rows`` (default: all)."""
    el = np.uint16 if dtype == BF16 else np.float32
    h = _as_host_array(h, el)
    w = _as_host_array(w, el)
    ids = _as_host_array(ids, np.int32)
    n, d = h.shape
    v, d2 = w.shape
    assert d == d2 and ids.shape == (n,)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = n if rows_arr is None else rows_arr.size
    out = {k: np.empty(nr, np.float64) for k in ("logp", "lse", "zsel", "entropy")}
    if nr == 0:
        return out
    if nthreads <= 0:
        nthreads = min(available_cpus(), MAX_THREADS)
    used = _load().or_logprob_rows_ex(_ptr(h), d, _ptr(w), d, _ptr(ids), dtype, d, v,
                                      _ptr(rows_arr), nr, float(temperature),
                                      _ptr(out["logp"]), _ptr(out["lse"]), _ptr(out["zsel"]),
                                      _ptr(out["entropy"]), int(nthreads))
    if used < 0:
        raise ValueError("or_logprob_rows_ex rejected its arguments")
    return out


def logprob(h, w, ids, *, dtype: int, rows=None, nthreads: int = 0):
    """fp64 ``(logp, lse, zsel)`` for token rows ``rows`` (default: all).

    ``h``: [N, D] and ``w``: [V, D]; for ``dtype == BF16`` pass uint16 bit
    patterns (or bf16 torch tensors), for ``F32`` float32.  ``ids``: [N]
    int32.  Returns float64 arrays indexed like ``rows`` and the number of
    threads used.
    """
    el = np.uint16 if dtype == BF16 else np.float32
    h = _as_host_array(h, el)
    w = _as_host_array(w, el)
    ids = _as_host_array(ids, np.int32)
    n, d = h.shape
    v, d2 = w.shape
    assert d == d2 and ids.shape == (n,)
    if rows is None:
        rows_arr = None
        nr = n
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows_arr.ndim == 1 and (rows_arr.size == 0 or
                                       (rows_arr.min() >= 0 and rows_arr.max() < n))
        nr = rows_arr.size
    logp = np.empty(nr, np.float64)
    lse = np.empty(nr, np.float64)
    zsel = np.empty(nr, np.float64)
    if nr == 0:
        return logp, lse, zsel, 0
    if nthreads <= 0:
        nthreads = min(available_cpus(), MAX_THREADS)
    used = _load().or_logprob_rows(_ptr(h), d, _ptr(w), d, _ptr(ids), dtype, d, v,
                                   _ptr(rows_arr), nr, _ptr(logp), _ptr(lse),
                                   _ptr(zsel), int(nthreads))
    if used < 0:
        raise ValueError("or_logprob_rows rejected its arguments")
    return logp, lse, zsel, used


def mismatch_stats(lt, lr, mask, cu_seqlens, *, clip_c: float, seq_lo: float,
                   seq_hi: float, seq_k3_hi: float = float("inf"),
                   token_outputs: bool = True) -> dict:
    """fp64 token, sequence and batch statistics (see module docstring).

    A sequence with a valid token is rejected when its mean delta is outside
    ``[seq_lo, seq_hi]`` (``seq["reject"]``) and K3-rejected when its mean k3
    exceeds ``seq_k3_hi`` (``seq["reject_k3"]``).
    """
    lt = _as_host_array(lt, np.float32)
    lr = _as_host_array(lr, np.float32)
    cu = _as_host_array(cu_seqlens, np.int32)
    m = None if mask is None else _as_host_array(mask, np.uint8)
    n = lt.size
    s = cu.size - 1
    if token_outputs:
        tok = {k: np.empty(n, np.float64) for k in ("delta", "ratio", "k1", "k2", "k3", "tis_w")}
        tok["clipped"] = np.empty(n, np.uint8)
    else:   # large inputs: sequence and batch results only
        tok = {k: None for k in ("delta", "ratio", "k1", "k2", "k3", "tis_w", "clipped")}
    seq = {k: np.empty(s, np.int32) for k in ("n_valid", "n_clipped", "n_nan")}
    seq.update({k: np.empty(s, np.float64) for k in
                ("mean_delta", "mean_k1", "mean_k2", "mean_k3", "mean_tis_w")})
    seq["reject"] = np.empty(s, np.uint8)
    seq["reject_k3"] = np.empty(s, np.uint8)
    batch = np.empty(len(BATCH_FIELDS), np.float64)
    rc = _load().or_mismatch_stats(
        _ptr(lt), _ptr(lr), _ptr(m), _ptr(cu), n, s, float(clip_c), float(seq_lo),
        float(seq_hi), float(seq_k3_hi),
        _ptr(tok["delta"]), _ptr(tok["ratio"]), _ptr(tok["k1"]), _ptr(tok["k2"]),
        _ptr(tok["k3"]), _ptr(tok["tis_w"]), _ptr(tok["clipped"]),
        _ptr(seq["n_valid"]), _ptr(seq["n_clipped"]), _ptr(seq["n_nan"]),
        _ptr(seq["mean_delta"]), _ptr(seq["mean_k1"]), _ptr(seq["mean_k2"]),
        _ptr(seq["mean_k3"]), _ptr(seq["mean_tis_w"]), _ptr(seq["reject"]),
        _ptr(seq["reject_k3"]), _ptr(batch))
    if rc != 0:
        raise ValueError("or_mismatch_stats rejected its arguments")
    return {"token": tok, "seq": seq,
            "batch": dict(zip(BATCH_FIELDS, (float(x) for x in batch)))}


def mismatch_extras(lt, lr, mask, *, tok_tau: float, ratio_q=(), abs_q=()) -> dict:
    """fp64 extreme-token rate, mean relative difference and quantiles.

    Returns ``{"n_valid", "n_extreme", "extreme_frac", "mean_rel_diff",
    "ratio_q": [...], "abs_q": [...], "vector": np.ndarray}`` where the
    quantile lists follow ``ratio_q`` / ``abs_q`` and ``vector`` is the full
    output in ``EXTRAS_FIELDS`` order.
    """
    lt = _as_host_array(lt, np.float32)
    lr = _as_host_array(lr, np.float32)
    m = None if mask is None else _as_host_array(mask, np.uint8)
    n = lt.size
    rq = np.ascontiguousarray(ratio_q, dtype=np.float64)
    aq = np.ascontiguousarray(abs_q, dtype=np.float64)
    out = np.empty(len(EXTRAS_FIELDS), np.float64)
    rc = _load().or_mismatch_extras(_ptr(lt), _ptr(lr), _ptr(m), n, float(tok_tau),
                                    _ptr(rq) if rq.size else None, int(rq.size),
                                    _ptr(aq) if aq.size else None, int(aq.size), _ptr(out))
    if rc != 0:
        raise ValueError("or_mismatch_extras rejected its arguments")
    res = dict(zip(EXTRAS_FIELDS[:4], (float(x) for x in out[:4])))
    res["ratio_q"] = [float(x) for x in out[4:4 + rq.size]]
    res["abs_q"] = [float(x) for x in out[8:8 + aq.size]]
    res["vector"] = out
    return res


def logprob_backward(h, w, ids, g, *, dtype: int, dh_rows=None, dw_rows=None, nthreads: int = 0):
    """fp64 ``(dh[dh_rows], dW[dw_rows])`` for the upstream gradient ``g``
    (``dL/dlogp``, one value per token); rows default to all.  Only tokens with
    ``g != 0`` cost anything."""
    el = np.uint16 if dtype == BF16 else np.float32
    h = _as_host_array(h, el)
    w = _as_host_array(w, el)
    ids = _as_host_array(ids, np.int32)
    g = _as_host_array(g, np.float64)
    n, d = h.shape
    v, d2 = w.shape
    assert d == d2 and ids.shape == (n,) and g.shape == (n,)
    dh_rows = np.arange(n, dtype=np.int64) if dh_rows is None else \
        np.ascontiguousarray(dh_rows, dtype=np.int64)
    dw_rows = np.arange(v, dtype=np.int64) if dw_rows is None else \
        np.ascontiguousarray(dw_rows, dtype=np.int64)
    dh = np.empty((dh_rows.size, d), np.float64)
    dw = np.empty((dw_rows.size, d), np.float64)
    if nthreads <= 0:
        nthreads = min(available_cpus(), MAX_THREADS)
    rc = _load().or_logprob_backward(_ptr(h), d, _ptr(w), d, _ptr(ids), _ptr(g), dtype, n, d, v,
                                     _ptr(dh_rows), dh_rows.size, _ptr(dh), _ptr(dw_rows),
                                     dw_rows.size, _ptr(dw), int(nthreads))
    if rc != 0:
        raise ValueError("or_logprob_backward rejected its arguments")
    return dh, dw


def ppo_loss(logp, old_train, old_rollout, adv, mask, *, eps_lo: float, eps_hi: float,
             bypass: bool = False, tis_c: float = 0.0, grad_scale: float = 0.0,
             token_outputs: bool = True) -> dict:
    """fp64 per-token loss, gradient (of the token mean, or of
    ``grad_scale`` times the token sum when it is > 0), ratio, contribution
    and clip flag, and the batch vector (``PPO_FIELDS``)."""
    arrs = [_as_host_array(x, np.float32) for x in (logp, old_train, old_rollout, adv)]
    m = None if mask is None else _as_host_array(mask, np.uint8)
    n = arrs[0].size
    if token_outputs:
        out = {k: np.empty(n, np.float64) for k in ("loss", "grad", "ratio", "contrib")}
        out["clipped"] = np.empty(n, np.uint8)
    else:   # large inputs: the batch vector only
        out = {k: None for k in ("loss", "grad", "ratio", "contrib", "clipped")}
    batch = np.empty(len(PPO_FIELDS), np.float64)
    rc = _load().or_ppo_loss(*[_ptr(a) for a in arrs], _ptr(m), n, float(eps_lo), float(eps_hi),
                             int(bool(bypass)), float(tis_c), float(grad_scale),
                             _ptr(out["loss"]), _ptr(out["grad"]),
                             _ptr(out["ratio"]), _ptr(out["contrib"]), _ptr(out["clipped"]),
                             _ptr(batch))
    if rc != 0:
        raise ValueError("or_ppo_loss rejected its arguments")
    out["batch"] = dict(zip(PPO_FIELDS, (float(x) for x in batch)))
    return out
