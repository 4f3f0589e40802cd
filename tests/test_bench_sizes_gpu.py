"""Parity at the sizes and launch configurations bench.py times for the
HBM-bound entry points: the statistics, the clipped surrogate and the extra
metrics at 2^28 tokens (the statistics workload, seed 7), and the RMSNorm at
2^18 rows of 4096.  The oracle computes every sequence and batch value of
the statistics and the surrogate's batch vector over all tokens, the
surrogate's per-token outputs and the norm's rows on a sample, and the extra
metrics (quantiles over every valid token) over all tokens.
"""
import math
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
N = 1 << 28
_inputs = {}


def say(msg):
    print(f"[bench-sizes] {msg}", flush=True)
    sys.stdout.flush()


def stats_inputs():
    if "stats" not in _inputs:
        say("generating the 2^28-token statistics workload")
        _inputs["stats"] = workloads.stats_scale(N, seed=7, device=DEV)
        torch.cuda.synchronize()
    return _inputs["stats"]


def test_stats_at_2p28_all_sequences_and_batch():
    lt, lr, mask, cu = stats_inputs()
    lo, hi = math.log(0.99), math.log(1.01)
    res = tim.tim_mismatch_stats(lt, lr, mask, cu, tis_clip=2.0, seq_bounds=(lo, hi),
                                 seq_k3_max=5e-5)
    torch.cuda.synchronize()
    say("oracle over 2^28 tokens")
    ref = oracle.mismatch_stats(lt.cpu(), lr.cpu(), mask.cpu(), cu.cpu(), clip_c=2.0, seq_lo=lo,
                                seq_hi=hi, seq_k3_hi=5e-5, token_outputs=False)
    s, r = res["seq"], ref["seq"]
    md = r["mean_delta"][r["n_valid"] > 0]
    margin = np.minimum(np.abs(md - lo), np.abs(md - hi)).min()
    say(f"{len(md)} sequences; smallest distance of a mean to a bound {margin:.3e}")
    assert margin > 1e-12
    for k in ("n_valid", "n_clipped", "n_nan", "reject", "reject_k3"):
        np.testing.assert_array_equal(s[k].cpu().numpy(), r[k], err_msg=k)
    for k in ("mean_delta", "mean_k1", "mean_k2", "mean_k3", "mean_tis_w"):
        np.testing.assert_allclose(s[k].cpu().numpy(), r[k], rtol=1e-3, atol=1e-12, err_msg=k)
    got = tim.batch_dict(res["batch"])
    for k_ours, k_ref in zip(tim.BATCH_FIELDS, oracle.BATCH_FIELDS):
        a, b = got[k_ours], ref["batch"][k_ref]
        if k_ours.startswith("n_") or k_ours in ("is_clip_ratio", "is_nan_ratio", "reject_frac",
                                                 "max_abs_delta", "reject_k3_frac"):
            assert a == b, f"{k_ours}: {a} vs {b}"
        else:
            assert abs(a - b) <= 1e-3 * abs(b) + 1e-12, f"{k_ours}: {a} vs {b}"


def test_extras_at_2p28_against_the_oracle():
    """The extra metrics over all 2^28 tokens against the oracle's, computed
    over the same host copies (its quantiles sort every valid token)."""
    lt, lr, mask, _ = stats_inputs()
    rq, aq = (0.01, 0.5, 0.99), (0.95,)
    out = tim.tim_mismatch_extras(lt, lr, mask, tok_tau=0.1, ratio_q=rq, abs_q=aq)
    got = tim.extras_dict(out, len(rq), len(aq))
    say("oracle extra metrics over 2^28 tokens")
    ref = oracle.mismatch_extras(lt.cpu(), lr.cpu(), mask.cpu(), tok_tau=0.1, ratio_q=rq,
                                 abs_q=aq)
    say(f"oracle done: ratio quantiles {ref['ratio_q']}, |delta| p95 {ref['abs_q'][0]:.6g}")
    assert got["n_valid"] == ref["n_valid"] and got["n_extreme"] == ref["n_extreme"]
    assert got["extreme_frac"] == ref["extreme_frac"]
    # the relative-difference mean sums in a different order on each side
    assert got["mean_rel_diff"] == pytest.approx(ref["mean_rel_diff"], rel=1e-9)
    # ratio quantiles interpolate exp(delta): the device exp and libm's may
    # differ by an ulp at each order statistic
    for v, want in zip(got["ratio_q"], ref["ratio_q"]):
        assert v == pytest.approx(want, rel=1.6e-15, abs=0)
    # |delta| is exact on both sides and the interpolation is the same
    # sequence of fp64 operations: equal
    assert got["abs_q"] == ref["abs_q"]
    say(f"ratio quantiles {got['ratio_q']}, |delta| p95 {got['abs_q'][0]:.6g}")


def test_ppo_at_2p28_batch_and_sampled_tokens():
    n = N
    g = torch.Generator(device=DEV).manual_seed(12)
    ot = -torch.rand(n, generator=g, device=DEV) * 4
    orr = ot + torch.randn(n, generator=g, device=DEV) * 0.05
    lp = ot + torch.randn(n, generator=g, device=DEV) * 0.3
    adv = torch.randn(n, generator=g, device=DEV)
    mask = (torch.rand(n, generator=g, device=DEV) < 0.9).to(torch.uint8)
    res = tim.tim_ppo_loss(lp, ot, orr, adv, mask, eps_low=0.2, eps_high=0.28, tis_c=2.0)
    torch.cuda.synchronize()
    say("oracle batch over 2^28 tokens")
    host = [x.cpu() for x in (lp, ot, orr, adv, mask)]
    ref = oracle.ppo_loss(*host, eps_lo=0.2, eps_hi=0.28, tis_c=2.0, token_outputs=False)
    got = dict(zip(tim.PPO_FIELDS, res["batch"].cpu().tolist()))
    for k in tim.PPO_FIELDS:
        if k.startswith("n_") or k == "clip_frac":
            assert got[k] == ref["batch"][k], k
        else:
            assert got[k] == pytest.approx(ref["batch"][k], rel=1e-9, abs=1e-300), k
    idx = np.sort(np.random.default_rng(3).choice(n, 100_000, replace=False))
    sub = [h.numpy()[idx] for h in host]
    ref_s = oracle.ppo_loss(*sub, eps_lo=0.2, eps_hi=0.28, tis_c=2.0)
    t = res["token"]
    ti = torch.as_tensor(idx, device=DEV)
    np.testing.assert_array_equal(t["clipped"][ti].cpu().numpy(), ref_s["clipped"])
    for k in ("loss", "ratio", "contrib"):
        np.testing.assert_allclose(t[k][ti].double().cpu().numpy(), ref_s[k], rtol=1e-6,
                                   atol=1e-30, err_msg=k)
    # the sample's gradients are of the sample's own token mean: rescale to the full batch's
    scale = ref_s["batch"]["n_valid"] / ref["batch"]["n_valid"]
    np.testing.assert_allclose(t["grad"][ti].double().cpu().numpy(), ref_s["grad"] * scale,
                               rtol=1e-6, atol=1e-30)


def test_rmsnorm_at_2p18_rows_sampled():
    n, d = 1 << 18, 4096
    x, gamma = workloads.pre_norm(n, d, seed=3, device=DEV)
    y = tim.tim_rmsnorm(x, gamma, eps=1e-6)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(4).choice(n, 256, replace=False))
    rows[-1] = n - 1
    ti = torch.as_tensor(rows, device=DEV)
    yr, _ = oracle.rmsnorm(x[ti].cpu(), gamma.cpu(), dtype=oracle.BF16, eps=1e-6)
    codes = oracle.bf16_round_rne(yr)
    got = y[ti].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, codes), f"{(got != codes).sum()} codes differ"
