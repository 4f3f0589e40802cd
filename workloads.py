"""Seeded synthetic workloads for selected-token scoring and mismatch statistics.

This module is shared by the tests, the smoke check and the benchmark.  It
only *makes inputs*: it holds neither the library's kernels nor the oracle's
arithmetic, and neither side of a parity check reads anything from it except
the arrays it returns.

What the inputs stand for.  The pages describe an RL loop in which a rollout
engine samples response tokens and records the log-probability of each
sampled token, and a trainer later recomputes that log-probability from the
same hidden states ("Train-Inference Consistency", section 1; "RL: Training
Inference Mismatch", section on the recommended debugging procedure).  No
model, checkpoint or dataset is used here.  Instead:

* ``h`` (final hidden states) and ``W`` (LM-head weight) are Gaussian with the
  per-workload standard deviations below, drawn with torch's seeded generator
  on the device that generates them, then rounded to bf16 (round-to-nearest-
  even, torch's conversion) for bf16 workloads.
* The *sampler* plays the rollout engine: it computes fp32 logits with a
  library matmul, draws one uniform per row and takes the inverse CDF of the
  row's softmax (temperature 1, no logits processors), and records that
  token's fp32 log-probability as the rollout engine would.  This recorded
  value is an input of the statistics; it is never used as an expected value.
* The rollout log-probability handed to the statistics is the sampler's
  record plus the injected mismatch of each workload: Gaussian per-token
  noise, optional per-sequence drift, optional spikes.

Every random draw comes from its own generator stream derived from the
workload seed with ``numpy.random.SeedSequence(seed).spawn``, in the fixed
order ``STREAMS``.  Small workloads are always generated on the CPU (bit-
reproducible on any machine); large ones on the GPU when one is present.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

STREAMS = ("h", "w", "ids", "noise", "spike_pos", "spike_sign", "drift", "lengths",
           "lt", "nan_pos", "x_pre", "row_scale", "gamma")


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    n: int
    d: int
    v: int
    dtype: str              # "bf16" or "f32"
    seq_lens: tuple         # explicit lengths, or () for the lognormal law
    n_seqs: int
    h_std: float
    w_std: float
    noise_std: float
    drift_std: float = 0.0
    spike_frac: float = 0.0
    spike_mag: float = 0.0
    prompt_frac: float = 0.0  # leading fraction of each sequence with mask 0
    clip_c: float = 2.0
    seq_lo: float = -0.01
    seq_hi: float = 0.01
    # K3-form rejection bound on a sequence's mean k3, and the extreme-token
    # threshold on |delta|; the pages give neither value.  5e-5 is the k3 of
    # a constant log-ratio of 0.01 to leading order (0.01^2 / 2), the K3
    # counterpart of the +-0.01 window; 0.1 flags the injected spikes and not
    # the per-token noise.
    seq_k3_hi: float = 5e-5
    tok_tau: float = 0.1
    seed: int = 0
    gen_on_cpu: bool = True
    desc: str = ""


# Bounds of the geometric-mean-ratio window [0.99, 1.01] in the log domain.
LOG_099 = math.log(0.99)
LOG_101 = math.log(1.01)

SPECS = {
    "tiny": Spec("tiny", 64, 256, 1024, "f32", (16,) * 4, 4, 1.0, 0.05, 1e-3,
                 seed=0, desc="N=64 (4x16), D=256, V=1024, fp32"),
    "small": Spec("small", 2048, 2048, 32000, "bf16", (256,) * 8, 8, 1.0, 0.02, 2e-3,
                  spike_frac=0.01, spike_mag=0.5, prompt_frac=0.1, seed=1,
                  desc="N=2048 (8x256), D=2048, V=32000, bf16"),
    "qwen3_8b": Spec("qwen3_8b", 8192, 4096, 151936, "bf16", (512,) * 16, 16, 1.0, 0.02,
                     1e-3, seed=2, gen_on_cpu=False,
                     desc="Qwen3-8B-shaped head: N=8192 (16x512), D=4096, V=151936, bf16"),
    "fp32_head": Spec("fp32_head", 4096, 4096, 151936, "f32", (512,) * 8, 8, 1.0, 0.02,
                      1e-3, seed=3, gen_on_cpu=False,
                      desc="FP32 LM head: N=4096 (8x512), D=4096, V=151936, fp32"),
    "dsv3": Spec("dsv3", 32768, 7168, 129280, "bf16", (), 64, 1.0, 0.02, 2e-3,
                 drift_std=5e-3, seq_lo=LOG_099, seq_hi=LOG_101, seed=4, gen_on_cpu=False,
                 desc="DeepSeek-V3-shaped head: N=32768 (64 lognormal), D=7168, V=129280, bf16"),
}


@dataclasses.dataclass
class Workload:
    spec: Spec
    h: torch.Tensor            # [N, D] bf16 or fp32
    w: torch.Tensor            # [V, D] bf16 or fp32
    ids: torch.Tensor          # [N] int32
    logp_sampler: torch.Tensor  # [N] fp32: the sampler's own record (no noise)
    logp_rollout: torch.Tensor  # [N] fp32: record + injected mismatch
    mask: Optional[torch.Tensor]  # [N] uint8 or None
    cu_seqlens: torch.Tensor   # [S+1] int32

    @property
    def n(self):
        return self.spec.n


def stream_seeds(seed: int) -> dict:
    """One 63-bit seed per named stream, in ``STREAMS`` order."""
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: int(c.generate_state(1, np.uint64)[0] >> np.uint64(1))
            for name, c in zip(STREAMS, children)}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def lognormal_lengths(n_total: int, n_seqs: int, seed: int, median: int = 512,
                      sigma: float = 0.5, lo: int = 128, hi: int = 4096) -> np.ndarray:
    """Lengths ``clip(median * exp(sigma z), lo, hi)`` rescaled to sum to
    ``n_total`` by largest-remainder rounding and re-clipped (repeated until
    the sum is exact)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    raw = np.clip(median * np.exp(sigma * rng.standard_normal(n_seqs)), lo, hi)
    if not (lo * n_seqs <= n_total <= hi * n_seqs):
        raise ValueError("n_total cannot be split into n_seqs lengths in [lo, hi]")
    lens = raw.copy()
    for _ in range(100):
        target = lens * (n_total / lens.sum())
        base = np.floor(target).astype(np.int64)
        rem = n_total - int(base.sum())
        order = np.argsort(-(target - base), kind="stable")
        base[order[:rem]] += 1
        clipped = np.clip(base, lo, hi)
        if clipped.sum() == n_total:
            return clipped.astype(np.int32)
        lens = clipped.astype(np.float64)
    raise RuntimeError("length rescaling did not converge")


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, np.int64)
    np.cumsum(np.asarray(lens, np.int64), out=cu[1:])
    return cu.astype(np.int32)


def sample_ids(h: torch.Tensor, w: torch.Tensor, u: torch.Tensor, rows_per_chunk: int = 2048):
    """Rollout-engine stand-in: draw ids from softmax(h W^T) by inverse CDF of
    the uniforms ``u`` and return ``(ids int32, recorded fp32 logp)``."""
    dev = h.device
    wt = w.float().t().contiguous()  # [D, V]
    n = h.shape[0]
    ids = torch.empty(n, dtype=torch.int32, device=dev)
    rec = torch.empty(n, dtype=torch.float32, device=dev)
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        z = torch.mm(h[r0:r1].float(), wt)                      # fp32 logits
        cdf = torch.cumsum(torch.softmax(z, dim=-1), dim=-1)
        target = (u[r0:r1] * cdf[:, -1]).unsqueeze(1).contiguous()
        a = torch.searchsorted(cdf, target).squeeze(1).clamp_(max=z.shape[1] - 1)
        ids[r0:r1] = a.to(torch.int32)
        rec[r0:r1] = torch.log_softmax(z, dim=-1).gather(1, a.unsqueeze(1)).squeeze(1)
        del z, cdf
    return ids, rec


def make(name: str, device: Optional[str] = None) -> Workload:
    """Build workload ``name`` (a key of ``SPECS``) and place it on ``device``
    (default: cuda if available, else cpu)."""
    spec = SPECS[name]
    if device is None:
        device = "cuda" if torch.cuda.is_available() else "cpu"
    gdev = "cpu" if (spec.gen_on_cpu or not torch.cuda.is_available()) else device
    seeds = stream_seeds(spec.seed)
    el = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

    h = torch.randn(spec.n, spec.d, generator=_gen(seeds["h"], gdev), device=gdev)
    h.mul_(spec.h_std)
    h = h.to(el)
    w = torch.randn(spec.v, spec.d, generator=_gen(seeds["w"], gdev), device=gdev)
    w.mul_(spec.w_std)
    w = w.to(el)
    u = torch.rand(spec.n, generator=_gen(seeds["ids"], gdev), device=gdev,
                   dtype=torch.float64).float()
    ids, rec = sample_ids(h, w, u)

    if spec.seq_lens:
        lens = np.asarray(spec.seq_lens, np.int32)
    else:
        lens = lognormal_lengths(spec.n, spec.n_seqs, seeds["lengths"])
    assert int(lens.sum()) == spec.n and len(lens) == spec.n_seqs
    cu = cu_from_lengths(lens)

    mismatch = torch.randn(spec.n, generator=_gen(seeds["noise"], gdev), device=gdev)
    mismatch.mul_(spec.noise_std)
    if spec.drift_std > 0:
        drift = torch.randn(spec.n_seqs, generator=_gen(seeds["drift"], gdev), device=gdev)
        drift.mul_(spec.drift_std)
        seq_of = torch.repeat_interleave(torch.arange(spec.n_seqs, device=gdev),
                                         torch.as_tensor(lens, dtype=torch.int64, device=gdev))
        mismatch.add_(drift[seq_of])
    if spec.spike_frac > 0:
        k = int(round(spec.spike_frac * spec.n))
        pos = torch.randperm(spec.n, generator=_gen(seeds["spike_pos"], gdev), device=gdev)[:k]
        sign = torch.randint(0, 2, (k,), generator=_gen(seeds["spike_sign"], gdev),
                             device=gdev).float().mul_(2).sub_(1)
        mismatch[pos] += spec.spike_mag * sign
    lr = (rec + mismatch).float()

    mask = None
    if spec.prompt_frac > 0:
        m = np.ones(spec.n, np.uint8)
        for j in range(spec.n_seqs):
            m[cu[j]: cu[j] + int(round(spec.prompt_frac * lens[j]))] = 0
        mask = torch.from_numpy(m)

    def to(x):
        return None if x is None else x.to(device)
    return Workload(spec, to(h), to(w), to(ids), to(rec), to(lr), to(mask),
                    torch.from_numpy(cu).to(device))


def stats_scale(n: int, seed: int = 7, device: Optional[str] = None,
                spike_frac: float = 1e-3, nan_frac: float = 1e-4, prompt_frac: float = 0.1):
    """Statistics-only workload of ``n`` tokens with the DeepSeek-V3-shaped
    workload's length and mismatch laws (lognormal lengths, median 512,
    128..4096; per-sequence drift N(0, 5e-3^2); per-token N(0, 2e-3^2)), plus
    spikes of +1.0 in delta (above log 2, so truncation triggers), NaN
    rollout entries and a zero mask on the leading 10% of each sequence.

    The trainer-side log-probabilities are drawn directly (no model):
    ``lt = -|N(0, 3^2)|``.  Returns ``(lt, lr, mask, cu_seqlens)``.
    """
    if device is None:
        device = "cuda" if torch.cuda.is_available() else "cpu"
    seeds = stream_seeds(seed)
    rng = np.random.Generator(np.random.PCG64(seeds["lengths"]))
    draw = np.clip(512 * np.exp(0.5 * rng.standard_normal(n // 128 + 1)), 128, 4096)
    draw = draw.astype(np.int64)
    ends = np.cumsum(draw)
    k = int(np.searchsorted(ends, n))      # first sequence reaching n
    lens = draw[:k + 1].copy()
    lens[k] = n - (int(ends[k - 1]) if k > 0 else 0)   # last one truncated
    lens = lens.astype(np.int32)
    cu = cu_from_lengths(lens)
    s = len(lens)
    lt = torch.randn(n, generator=_gen(seeds["lt"], device), device=device).abs_().mul_(-3.0)
    eps = torch.randn(n, generator=_gen(seeds["noise"], device), device=device).mul_(2e-3)
    drift = torch.randn(s, generator=_gen(seeds["drift"], device), device=device).mul_(5e-3)
    lens_t = torch.as_tensor(lens, dtype=torch.int64, device=device)
    seq_of = torch.repeat_interleave(torch.arange(s, device=device), lens_t)
    mismatch = eps + drift[seq_of]
    k = int(round(spike_frac * n))
    if k:
        pos = torch.randint(0, n, (k,), generator=_gen(seeds["spike_pos"], device),
                            device=device)
        mismatch[pos] = -1.0           # delta = lt - lr = +1.0
    lr = lt + mismatch
    k = int(round(nan_frac * n))
    if k:
        pos = torch.randint(0, n, (k,), generator=_gen(seeds["nan_pos"], device),
                            device=device)
        lr[pos] = float("nan")
    start = torch.as_tensor(cu[:-1], dtype=torch.int64, device=device)[seq_of]
    pos_in_seq = torch.arange(n, device=device) - start
    prompt = torch.round(lens_t.double() * prompt_frac).long()[seq_of]
    mask = (pos_in_seq >= prompt).to(torch.uint8)
    return lt.float(), lr.float(), mask, torch.from_numpy(cu).to(device)


def pre_norm(n: int, d: int, seed: int, dtype=torch.bfloat16, device: Optional[str] = None):
    """Pre-norm final hidden states ``x`` [n, d] and an RMSNorm gain ``gamma``
    [d] for the norm in front of the head.  ``x = s_t * N(0, 1)`` with a
    per-row scale ``s_t = 8 exp(0.5 z_t)`` (rows of different loudness, as
    residual streams are) and four fixed channels (0, 1, d/2, d - 1) ten
    times louder (a few outlier channels); ``gamma = 1 + N(0, 0.2^2)``.  Both
    rounded to ``dtype`` (torch's conversion: nearest, ties to even).
    Returns ``(x, gamma)``."""
    if device is None:
        device = "cuda" if torch.cuda.is_available() else "cpu"
    seeds = stream_seeds(seed)
    x = torch.randn(n, d, generator=_gen(seeds["x_pre"], device), device=device)
    rs = torch.randn(n, generator=_gen(seeds["row_scale"], device), device=device)
    x.mul_((8.0 * torch.exp(0.5 * rs))[:, None])
    x[:, [0, 1, d // 2, d - 1]] *= 10.0
    gamma = 1.0 + 0.2 * torch.randn(d, generator=_gen(seeds["gamma"], device), device=device)
    return x.to(dtype), gamma.to(dtype)


def sweep_slices(n: int, batch: int):
    """Consecutive ``[start, end)`` slices of ``batch`` rows covering ``n``."""
    return [(s, min(n, s + batch)) for s in range(0, n, batch)]


def random_slices(n: int, seed: int, max_batch: int = 1000):
    """A seeded random partition of ``[0, n)`` into slices of 1..max_batch rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out, s = [], 0
    while s < n:
        b = int(rng.integers(1, max_batch + 1))
        out.append((s, min(n, s + b)))
        s += b
    return out
