"""GPU parity of tim_mismatch_extras against the fp64 oracle on identical
inputs: counts and the |delta| quantiles bit-exact (both sides select the same
fp64 order statistics and interpolate with the same three roundings), ratio
quantiles within a few ulps (the device and host exp differ by at most an
ulp), the mean relative difference within the summation-order bound
2 m 2^-53 for m valid tokens;
plus the K3-form sequence rejection of tim_mismatch_stats, and run-to-run
determinism.
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
RQ = (0.01, 0.5, 0.99)
AQ = (0.95,)


def say(msg):
    print(f"[extras-gpu] {msg}", flush=True)
    sys.stdout.flush()


def check(lt, lr, mask, tau, rq=RQ, aq=AQ, label=""):
    out = tim.tim_mismatch_extras(lt, lr, mask, tok_tau=tau, ratio_q=rq, abs_q=aq)
    torch.cuda.synchronize()
    got = tim.extras_dict(out, len(rq), len(aq))
    ref = oracle.mismatch_extras(lt.cpu(), lr.cpu(), None if mask is None else mask.cpu(),
                                 tok_tau=tau, ratio_q=rq, abs_q=aq)
    say(f"{label}: n_valid {got['n_valid']:.0f}, extreme {got['extreme_frac']:.3e}, "
        f"rel {got['mean_rel_diff']:.3e}, ratio q {got['ratio_q']}, |d| q {got['abs_q']}")
    assert got["n_valid"] == ref["n_valid"], label
    assert got["n_extreme"] == ref["n_extreme"], label
    assert got["extreme_frac"] == ref["extreme_frac"], label
    # a sum of m positive terms in any order is within (m - 1) u of the exact
    # sum (u = 2^-53); the two sides add in different orders
    tol = 2 * max(got["n_valid"], 1) * 2.0 ** -53
    assert got["mean_rel_diff"] == pytest.approx(ref["mean_rel_diff"], rel=tol, abs=0), label
    assert got["abs_q"] == ref["abs_q"], f"{label}: {got['abs_q']} vs {ref['abs_q']}"
    np.testing.assert_allclose(got["ratio_q"], ref["ratio_q"], rtol=4e-16 * 4, atol=0,
                               err_msg=label)
    # unused slots are zero
    v = out.cpu().numpy()
    assert np.all(v[4 + len(rq):8] == 0) and np.all(v[8 + len(aq):12] == 0)
    return got, out


@pytest.mark.parametrize("name", ["tiny", "small", "qwen3_8b", "dsv3"])
def test_workload_extras_parity(name):
    w = workloads.make(name, device=DEV)
    say(f"workload {name}")
    check(w.logp_sampler, w.logp_rollout, w.mask, w.spec.tok_tau, label=name)


@pytest.mark.parametrize("n", [1, 7, 1000, 8192, 8193, 16384 + 37, 200_003, 1 << 22, (1 << 25) + 7])
def test_stress_extras_parity(n):
    # lognormal lengths, per-sequence drift, spikes of +1, NaN entries and a
    # masked prompt; sizes across one block, many blocks and a ragged tail
    lt, lr, mask, _ = workloads.stats_scale(max(n, 1), seed=31 + n % 97, device=DEV)
    check(lt[:n].contiguous(), lr[:n].contiguous(), mask[:n].contiguous(), 0.1,
          label=f"stress n={n}")


def test_unmasked_and_probability_edges():
    lt, lr, _, _ = workloads.stats_scale(50_000, seed=3, device=DEV)
    check(lt, lr, None, 0.05, rq=(0.0, 1.0), aq=(0.0, 1.0), label="q = 0, 1")
    got, _ = check(lt, lr, None, 0.05, rq=(), aq=(0.25, 0.5, 0.75, 0.999), label="abs only")
    got, _ = check(lt, lr, None, 0.05, rq=(0.3, 0.6, 0.9, 0.97), aq=(), label="ratio only")
    got, _ = check(lt, lr, None, 0.05, rq=(), aq=(), label="no quantiles")


def test_empty_all_masked_single_and_zero_mismatch():
    z = torch.zeros(0, device=DEV)
    out = tim.tim_mismatch_extras(z, z, None, tok_tau=0.1)
    assert torch.all(out.cpu() == 0)
    lt, lr, mask, _ = workloads.stats_scale(40_000, seed=4, device=DEV)
    out = tim.tim_mismatch_extras(lt, lr, torch.zeros_like(mask), tok_tau=0.1)
    assert torch.all(out.cpu() == 0)
    one = torch.zeros_like(mask)
    one[12345] = 1
    lr1 = lr.clone()
    lr1[12345] = lt[12345] - 0.25          # finite delta at the one valid token
    check(lt, lr1, one, 0.1, label="single valid token")
    # zero mismatch: every delta 0, resolved by the key-range test in one pass
    got, _ = check(lt, lt, mask, 0.1, label="zero mismatch")
    assert got["ratio_q"] == [1.0, 1.0, 1.0] and got["abs_q"] == [0.0]
    assert got["extreme_frac"] == 0 and got["mean_rel_diff"] == 0


def test_keys_differing_only_in_the_last_bits():
    # deltas 1, 1 + 2^-52 and 1 + 2^-51 (exact: lt = 1, lr = 0, -2^-52, -2^-51
    # are fp32 values and their differences are doubles): the keys share their
    # first 62 bits, so every radix pass is needed, with heavy ties in each
    n = 300_000
    g = torch.Generator(device="cpu").manual_seed(5)
    u = torch.rand(n, generator=g)
    lr = torch.zeros(n, dtype=torch.float32)
    lr[u < 0.5] = -(2.0 ** -52)
    lr[u < 0.2] = -(2.0 ** -51)
    lt = torch.ones(n, dtype=torch.float32)
    d = lt.double() - lr.double()
    assert len(set(d.tolist())) == 3
    for q in ((0.01, 0.5, 0.999), (0.2, 0.5, 0.8)):
        got, _ = check(lt.to(DEV), lr.to(DEV), None, 1.0, rq=q, aq=(0.35,), label=f"near ties {q}")
    assert got["n_extreme"] == int((d > 1.0).sum())


def test_signed_zero_deltas_and_magnitudes_across_the_fp32_range():
    # several pass blocks (N > 8192).  First every delta is a zero, -0 on a
    # third of the tokens ((-0) - (+0)), +0 elsewhere: two keys for one
    # value, resolved to a zero either way, ratio 1 and |delta| 0.
    n = 300_000
    g = torch.Generator(device="cpu").manual_seed(11)
    lt = torch.zeros(n, dtype=torch.float32)
    lt[torch.rand(n, generator=g) < 1.0 / 3.0] = -0.0
    lr = torch.zeros(n, dtype=torch.float32)
    assert int(torch.signbit(lt.double() - lr.double()).sum()) > n // 4
    got, _ = check(lt.to(DEV), lr.to(DEV), None, 0.1, label="signed zeros")
    assert got["ratio_q"] == [1.0, 1.0, 1.0] and got["abs_q"] == [0.0]
    # then lt and lr drawn from magnitudes across the fp32 range with random
    # signs: rel_diff's divisor |lt| + 1e-8 runs from 1e-8 to 3.4e38 and its
    # numerator |delta| up to 6.8e38, the keys span every binade
    mags = torch.tensor([0.0, 1e-45, 1e-38, 1e-8, 0.5, 1.0, 3.0, 1e20, 3.4e38],
                        dtype=torch.float32)
    pick = lambda: mags[torch.randint(0, len(mags), (n,), generator=g)] * \
        torch.where(torch.rand(n, generator=g) < 0.5, -1.0, 1.0)
    lt, lr = pick(), pick()
    check(lt.to(DEV), lr.to(DEV), None, 1.0, label="fp32 range")
    check(lt.to(DEV), lr.to(DEV), None, 1.0, rq=(0.2, 0.8), aq=(0.1, 0.9),
          label="fp32 range, other quantiles")


def test_candidate_overflow_falls_back_to_the_inputs():
    # every delta in [1, 1.4): one first-pass bucket holds all keys, more than
    # the candidate regions take, so the later passes read the tokens again
    n = 400_000
    g = torch.Generator(device="cpu").manual_seed(8)
    lr = -torch.rand(n, generator=g) * 4
    lt = (lr.double() + 1.0 + 0.4 * torch.rand(n, generator=g, dtype=torch.float64)).float()
    check(lt.to(DEV), lr.to(DEV), None, 1.2, rq=(0.01, 0.5, 0.99), aq=(0.95,), label="overflow")
    # and the same law on a tenth of the tokens, inside regions of their own
    m = (torch.rand(n, generator=g) < 0.1).to(torch.uint8)
    check(lt.to(DEV), lr.to(DEV), m.to(DEV), 1.2, rq=(0.01, 0.5, 0.99), aq=(0.95,),
          label="masked to a tenth")


def test_sample_that_misleads_the_windows_falls_back_to_the_inputs():
    # the tokens the sample reads (the first 16 of every 1024) carry one
    # delta, the others a spread: every predicted window sits on the sampled
    # value's bin, misses the true order statistics, and pass 1 reads the
    # tokens again; the results are the oracle's all the same
    n = (1 << 25) + 12345                # the sample runs from 2^25 tokens
    g = torch.Generator(device="cpu").manual_seed(12)
    lr = -torch.rand(n, generator=g) * 3
    dl = torch.randn(n, generator=g, dtype=torch.float64) * 0.01
    sampled = (torch.arange(n) % 1024) < 16
    dl[sampled] = 0.3
    lt = (lr.double() + dl).float()
    m = (torch.rand(n, generator=g) < 0.9).to(torch.uint8)
    check(lt.to(DEV), lr.to(DEV), m.to(DEV), 0.1, label="misleading sample")
    check(lt.to(DEV), lr.to(DEV), None, 0.1, rq=(0.2, 0.7), aq=(0.5, 0.99),
          label="misleading sample, unmasked")


def test_extras_run_to_run_determinism():
    lt, lr, mask, _ = workloads.stats_scale(1 << 21, seed=10, device=DEV)
    outs = [tim.tim_mismatch_extras(lt, lr, mask, tok_tau=0.1) for _ in range(3)]
    small = [tim.tim_mismatch_extras(lt[:5000], lr[:5000], mask[:5000], tok_tau=0.1)
             for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int64), outs[0].view(torch.int64))
    for o in small[1:]:
        assert torch.equal(o.view(torch.int64), small[0].view(torch.int64))


def k3_margin(ref, bound):
    mk3 = ref["seq"]["mean_k3"]
    ok = ref["seq"]["n_valid"] > 0
    return np.abs(mk3 - bound)[ok].min() if ok.any() else math.inf


@pytest.mark.parametrize("name", ["small", "dsv3"])
def test_k3_sequence_rejection_parity(name):
    w = workloads.make(name, device=DEV)
    sp = w.spec
    mask_h = None if w.mask is None else w.mask.cpu()
    base = oracle.mismatch_stats(w.logp_sampler.cpu(), w.logp_rollout.cpu(), mask_h,
                                 w.cu_seqlens.cpu(), clip_c=sp.clip_c, seq_lo=sp.seq_lo,
                                 seq_hi=sp.seq_hi)
    # the workload's bound, and one half-way between the two middle sequence
    # means of k3 so that both flag values occur
    mk3 = np.sort(base["seq"]["mean_k3"][base["seq"]["n_valid"] > 0])
    mid = len(mk3) // 2
    for bound in (sp.seq_k3_hi, 0.5 * (mk3[mid - 1] + mk3[mid])):
        res = tim.tim_mismatch_stats(w.logp_sampler, w.logp_rollout, w.mask, w.cu_seqlens,
                                     tis_clip=sp.clip_c, seq_bounds=(sp.seq_lo, sp.seq_hi),
                                     seq_k3_max=bound)
        torch.cuda.synchronize()
        ref = oracle.mismatch_stats(w.logp_sampler.cpu(), w.logp_rollout.cpu(), mask_h,
                                    w.cu_seqlens.cpu(), clip_c=sp.clip_c, seq_lo=sp.seq_lo,
                                    seq_hi=sp.seq_hi, seq_k3_hi=bound)
        # a flag could only differ within summation rounding of the bound
        margin = k3_margin(ref, bound)
        say(f"{name}: bound {bound:.3e}, K3 flag margin {margin:.3e}, rejected "
            f"{int(ref['batch']['n_seq_rejected_k3'])}/{int(ref['batch']['n_seq_nonempty'])}")
        assert margin > 1e-12 * bound
        np.testing.assert_array_equal(res["seq"]["reject_k3"].cpu().numpy(),
                                      ref["seq"]["reject_k3"])
        got = tim.batch_dict(res["batch"])
        assert got["reject_k3_frac"] == ref["batch"]["reject_k3_frac"]
        assert got["n_seq_rejected_k3"] == ref["batch"]["n_seq_rejected_k3"]
    assert 0 < got["n_seq_rejected_k3"] < got["n_seq_nonempty"]


def test_k3_rejection_stress_and_default_off():
    lt, lr, mask, cu = workloads.stats_scale(1 << 18, seed=12, device=DEV)
    res = tim.tim_mismatch_stats(lt, lr, mask, cu, seq_k3_max=5e-5)
    off = tim.tim_mismatch_stats(lt, lr, mask, cu)
    torch.cuda.synchronize()
    ref = oracle.mismatch_stats(lt.cpu(), lr.cpu(), mask.cpu(), cu.cpu(), clip_c=2.0,
                                seq_lo=-0.01, seq_hi=0.01, seq_k3_hi=5e-5)
    assert k3_margin(ref, 5e-5) > 1e-17
    np.testing.assert_array_equal(res["seq"]["reject_k3"].cpu().numpy(), ref["seq"]["reject_k3"])
    assert not off["seq"]["reject_k3"].cpu().any()
    assert tim.batch_dict(off["batch"])["n_seq_rejected_k3"] == 0
