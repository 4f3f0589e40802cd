"""GPU parity and invariance of the RMSNorm in front of the head and of
temperature-scaled scoring with entropy (tim_rmsnorm, tim_logprob_forward_ex).

Every GPU value comes from the HIP library through its C ABI and is compared
with the fp64 oracle on the same seeded inputs: bf16 RMSNorm outputs code for
code (both sides round the same fp64 value once, ties to even), logp / lse
within 2e-4 and the entropy within 2e-4 (1 + H); or with itself across batch
splits, layouts and entry points (bit-exact).
"""
import sys

import numpy as np
import pytest
import torch

import invariant_logprobs_amd as tim
import oracle
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
TOL_LOGP = 2e-4
EPS = 1e-6


def say(msg):
    print(f"[norm-temp-gpu] {msg}", flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def odt(t):
    return oracle.BF16 if t.dtype == torch.bfloat16 else oracle.F32


def oracle_norm_codes(x, g, eps):
    """The oracle's normalised rows, rounded once to x's dtype (as bits)."""
    y, rstd = oracle.rmsnorm(x.cpu(), g.cpu(), dtype=odt(x), eps=eps)
    if x.dtype == torch.bfloat16:
        return oracle.bf16_round_rne(y), y, rstd
    return y.astype(np.float32).view(np.int32), y, rstd


def near_tie(y, dtype):
    """Entries whose fp64 value lies within 1e-12 (relative) of a rounding
    midpoint of the output type: there the last bit may go either way."""
    if dtype == torch.bfloat16:
        lo = oracle.bf16_decode(oracle.bf16_round_rne(y).ravel()).reshape(y.shape)
        keep = 8                                   # significant bits
    else:
        lo = y.astype(np.float32).astype(np.float64)
        keep = 24
    _, e = np.frexp(lo)                            # lo = m 2^e, 0.5 <= |m| < 1
    ulp = np.ldexp(1.0, e - keep)
    return np.abs(np.abs(y - lo) - ulp / 2) <= 1e-12 * np.abs(y)


def check_norm(x, g, y_gpu, rstd_gpu, label):
    codes, y, rstd = oracle_norm_codes(x, g, EPS)
    got = bits(y_gpu).cpu().numpy()
    if x.dtype == torch.bfloat16:
        got = got.view(np.uint16)
    diff = got != codes
    ties = near_tie(y, x.dtype)
    say(f"{label}: {diff.sum()} codes differ, {ties.sum()} near ties, of {codes.size}")
    assert not np.any(diff & ~ties), f"{label}: codes differ away from a rounding tie"
    if rstd_gpu is not None:
        np.testing.assert_allclose(rstd_gpu.double().cpu().numpy(), rstd, rtol=2e-7)


@pytest.mark.parametrize("n,d,dtype,ldx", [(37, 200, torch.bfloat16, 200),
                                           (300, 4096, torch.bfloat16, 4096),
                                           (64, 4096, torch.bfloat16, 4160),
                                           (50, 1000, torch.float32, 1000),
                                           (129, 7168, torch.float32, 7168),
                                           # register-resident rows: the limits of
                                           # each variant and the next width past them
                                           (40, 4096, torch.float32, 4096),
                                           (21, 4104, torch.float32, 4104),
                                           (33, 7168, torch.bfloat16, 7168),
                                           (20, 8192, torch.bfloat16, 8192),
                                           (17, 8200, torch.bfloat16, 8200),
                                           (9, 4100, torch.bfloat16, 4100)])
def test_rmsnorm_parity(n, d, dtype, ldx):
    x_full, g = workloads.pre_norm(n, ldx, seed=n + d, dtype=dtype, device=DEV)
    x = x_full[:, :d]
    g = g[:d].contiguous()
    y, rstd = tim.tim_rmsnorm(x, g, eps=EPS, return_rstd=True)
    torch.cuda.synchronize()
    check_norm(x, g, y, rstd, f"n={n} d={d} {dtype} ldx={ldx}")


def test_rmsnorm_rows_do_not_depend_on_batch_or_layout():
    n, d = 200, 4096
    x, g = workloads.pre_norm(n, d, seed=11, device=DEV)
    y = tim.tim_rmsnorm(x, g)
    # a slice of rows scored on its own
    y_s = tim.tim_rmsnorm(x[37:161].contiguous(), g)
    # the same rows at an address that is not 16-byte aligned (element-wise loads)
    buf = torch.empty(n * d + 1, dtype=x.dtype, device=DEV)
    xu = buf[1:].view(n, d)
    xu.copy_(x)
    y_u = tim.tim_rmsnorm(xu, g)
    y_2 = tim.tim_rmsnorm(x, g)
    torch.cuda.synchronize()
    assert torch.equal(bits(y_s), bits(y[37:161]))
    assert torch.equal(bits(y_u), bits(y))
    assert torch.equal(bits(y_2), bits(y))


def test_rmsnorm_degenerate_rows():
    d = 256
    x = torch.zeros(4, d, dtype=torch.bfloat16, device=DEV)
    x[1] = 3.0
    x[2, ::2], x[2, 1::2] = 1e-30, -1e-30        # tiny: eps dominates
    x[3, 5] = 1e4                                  # one loud entry
    g = torch.linspace(0.5, 1.5, d, device=DEV).to(torch.bfloat16)
    y, rstd = tim.tim_rmsnorm(x, g, eps=EPS, return_rstd=True)
    torch.cuda.synchronize()
    check_norm(x, g, y, rstd, "degenerate rows")
    assert torch.all(y[0] == 0)


def _case(n, d, v, seed, dtype=torch.bfloat16):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn(n, d, generator=gen).to(dtype)
    w = (torch.randn(v, d, generator=gen) * 0.05).to(dtype)
    ids = torch.randint(0, v, (n,), generator=gen, dtype=torch.int32)
    return h.to(DEV), w.to(DEV), ids.to(DEV)


def check_ex(res, ref, label, rows=None):
    rows = slice(None) if rows is None else rows
    lp = res["logp"].double().cpu().numpy()[rows]
    ls = res["lse"].double().cpu().numpy()[rows]
    ok = np.isfinite(ref["logp"])
    e_lp = np.abs(lp[ok] - ref["logp"][ok])
    e_ls = np.abs(ls - ref["lse"])
    msg = f"{label}: max |dlogp| {e_lp.max():.2e}, |dlse| {e_ls.max():.2e}"
    assert np.all(np.isnan(lp[~ok]))
    assert e_lp.max() <= TOL_LOGP and e_ls.max() <= TOL_LOGP, msg
    if "entropy" in res:
        en = res["entropy"].double().cpu().numpy()[rows]
        e_en = np.abs(en - ref["entropy"]) / (1 + ref["entropy"])
        msg += f", |dH|/(1+H) {e_en.max():.2e}"
        assert e_en.max() <= TOL_LOGP, msg
    say(msg)


@pytest.mark.parametrize("tau", [0.7, 1.0, 1.6])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_temperature_and_entropy_parity(tau, dtype):
    n, d, v = 300, 256, 2000
    h, w, ids = _case(n, d, v, seed=int(tau * 10), dtype=dtype)
    ids[7] = v + 3                                  # out of range: NaN logp, counted
    res = tim.tim_logprob_forward_ex(h, w, ids, temperature=tau, entropy=True)
    torch.cuda.synchronize()
    ref = oracle.logprob_ex(h.cpu(), w.cpu(), ids.cpu(), dtype=odt(h), temperature=tau)
    check_ex(res, ref, f"tau={tau} {dtype}")
    assert int(res["n_bad_ids"].item()) == 1


def test_tau_one_is_the_plain_forward_bitwise():
    n, d, v = 700, 512, 5000
    h, w, ids = _case(n, d, v, seed=3)
    lp, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    a = tim.tim_logprob_forward_ex(h, w, ids, temperature=1.0)
    b = tim.tim_logprob_forward_ex(h, w, ids, temperature=1.0, entropy=True)
    torch.cuda.synchronize()
    for r in (a, b):
        assert torch.equal(bits(r["logp"]), bits(lp))
        assert torch.equal(bits(r["lse"]), bits(lse))


def test_entropy_edge_cases():
    d = 64
    # V = 1: the only token has probability 1
    h, w, ids = _case(5, d, 1, seed=4)
    r = tim.tim_logprob_forward_ex(h, w, torch.zeros(5, dtype=torch.int32, device=DEV),
                                   temperature=0.5, entropy=True)
    torch.cuda.synchronize()
    assert torch.all(r["logp"] == 0) and torch.all(r["entropy"] == 0)
    # equal logits: H = log V at any temperature
    w0 = torch.zeros(777, d, dtype=torch.bfloat16, device=DEV)
    r = tim.tim_logprob_forward_ex(h, w0, torch.zeros(5, dtype=torch.int32, device=DEV),
                                   temperature=3.0, entropy=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(r["entropy"].double().cpu().numpy(), np.log(777), rtol=1e-5)
    np.testing.assert_allclose(r["logp"].double().cpu().numpy(), -np.log(777), rtol=1e-5)


def test_ex_rows_do_not_depend_on_the_batch():
    n, d, v = 520, 256, 3000
    x, g = workloads.pre_norm(n, d, seed=5, device=DEV)
    _, w, ids = _case(n, d, v, seed=5)
    kw = dict(temperature=0.7, entropy=True, norm_gamma=g, norm_eps=EPS)
    full = tim.tim_logprob_forward_ex(x, w, ids, **kw)
    again = tim.tim_logprob_forward_ex(x, w, ids, **kw)
    parts = [tim.tim_logprob_forward_ex(x[a:b].contiguous(), w, ids[a:b].contiguous(), **kw)
             for a, b in ((0, 1), (1, 21), (21, 257), (257, 520))]
    # the fused norm equals the norm followed by the head
    hn = tim.tim_rmsnorm(x, g, eps=EPS)
    sep = tim.tim_logprob_forward_ex(hn, w, ids, temperature=0.7, entropy=True)
    torch.cuda.synchronize()
    for k in ("logp", "lse", "entropy"):
        assert torch.equal(bits(full[k]), bits(again[k])), k
        assert torch.equal(bits(torch.cat([p[k] for p in parts])), bits(full[k])), k
        assert torch.equal(bits(sep[k]), bits(full[k])), k


def test_full_size_norm_temperature_entropy():
    # the Qwen3-8B-shaped head (N = 8192, D = 4096, V = 151936) with pre-norm
    # rows, tau = 0.7 and the entropy; the oracle scores 16 sampled rows
    w8 = workloads.make("qwen3_8b", device=DEV)
    w, ids = w8.w, w8.ids
    n, d = ids.shape[0], w.shape[1]
    x, g = workloads.pre_norm(n, d, seed=2, device=DEV)
    say("full size: fused norm + head at tau 0.7")
    res = tim.tim_logprob_forward_ex(x, w, ids, temperature=0.7, entropy=True, norm_gamma=g,
                                     norm_eps=EPS)
    hn = tim.tim_rmsnorm(x, g, eps=EPS)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(9).choice(n, 16, replace=False))
    rows[-1] = n - 1
    xr = x[torch.as_tensor(rows, device=DEV)]
    codes, _, _ = oracle_norm_codes(xr, g, EPS)
    got = hn[torch.as_tensor(rows, device=DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, codes), "normalised rows differ from the oracle's codes"
    say("full size: oracle rows")
    ref = oracle.logprob_ex(codes, w.cpu(), ids.cpu()[torch.as_tensor(rows)], dtype=oracle.BF16,
                            temperature=0.7)
    check_ex(res, ref, "full size", rows=rows)
