"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's formula: each expected value comes
from a value the pages print (``tests/golden``), a closed form, an invariant,
exact rational arithmetic, or a brute-force evaluation by a different route
(normalised probabilities in 50-digit decimal arithmetic).  The last test
plants mistakes in a copy of the oracle and checks that these pins catch them.
"""
import json
import math
import os
import re
import subprocess
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
getcontext().prec = 50


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def _exact_logits(h, w):
    """z[t, v] as exact rationals from float inputs."""
    hf = [[Fraction(float(x)) for x in row] for row in h]
    wf = [[Fraction(float(x)) for x in row] for row in w]
    return [[sum(a * b for a, b in zip(hr, wr)) for wr in wf] for hr in hf]


def _brute_logp(z_row, a):
    """log of the normalised probability p_a = e^{z_a} / sum_v e^{z_v}."""
    ez = [_dec(z).exp() for z in z_row]
    p = ez[a] / sum(ez)
    return float(p.ln())


# ---------------------------------------------------------------------------
# bf16 (the pages' rounding example)
# ---------------------------------------------------------------------------

def test_bf16_order_of_addition_example():
    g = json.load(open(os.path.join(GOLDEN, "bf16_rounding_order.json")))
    a, b, c = g["a"], g["b"], g["c"]

    def rnd(x):
        return float(oracle.bf16_decode(oracle.bf16_round_rne([x]))[0])

    assert rnd(1.0 + 2.0 ** -7) == g["next_above_one"]
    assert rnd(a + b) == 1.0                      # exact tie -> even -> 1
    left = rnd(rnd(a + b) + c)
    right = rnd(a + rnd(b + c))
    assert left == g["left_assoc_result"]
    assert right == g["right_assoc_result"]
    assert int(oracle.bf16_round_rne([left])[0]) == int(g["left_assoc_bits"], 16)
    assert int(oracle.bf16_round_rne([right])[0]) == int(g["right_assoc_bits"], 16)
    # torch's float32 -> bfloat16 conversion (used to make bf16 inputs) agrees
    t = lambda x: torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).float().item()
    assert t(t(a + b) + c) == left and t(a + t(b + c)) == right


def test_bf16_decode_known_patterns():
    pats = {0x3F80: 1.0, 0x3F81: 1.0 + 2 ** -7, 0xC000: -2.0, 0x0001: 2.0 ** -133,
            0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x0000: 0.0}
    got = oracle.bf16_decode(list(pats))
    assert list(got) == list(pats.values())
    inf = oracle.bf16_decode([0x7F80, 0xFF80, 0x7FC0])
    assert inf[0] == math.inf and inf[1] == -math.inf and math.isnan(inf[2])


def test_bf16_rne_matches_torch_conversion():
    """Round-to-nearest-even is also what torch implements for fp32 -> bf16;
    compare on random values, exact ties and subnormals."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3.0),
        # exact ties: bf16 value + half an ulp (low 16 bits = 0x8000)
        (rng.integers(0x3000, 0x4F00, 500, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([2.0 ** -130, 3 * 2.0 ** -134, -2.0 ** -127], np.float32),
    ])
    ours = oracle.bf16_round_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


# ---------------------------------------------------------------------------
# selected-token log-probability
# ---------------------------------------------------------------------------

def _lp(h, w, ids, dtype=oracle.F32, rows=None):
    logp, lse, zsel, _ = oracle.logprob(h, w, ids, dtype=dtype, rows=rows, nthreads=2)
    return logp, lse, zsel


def test_equal_logits_give_minus_log_v():
    rng = np.random.default_rng(1)
    v, d = 1024, 256
    h = rng.standard_normal((8, d)).astype(np.float32)
    ids = rng.integers(0, v, 8).astype(np.int32)
    logp, lse, _ = _lp(h, np.zeros((v, d), np.float32), ids)
    np.testing.assert_allclose(logp, -math.log(v), rtol=0, atol=1e-13)
    assert abs(-math.log(1024) - (-6.931471805599453)) < 1e-15
    w = rng.standard_normal((v, d)).astype(np.float32)
    logp, _, _ = _lp(np.zeros((8, d), np.float32), w, ids)
    np.testing.assert_allclose(logp, -math.log(v), rtol=0, atol=1e-13)
    # the Qwen3-8B vocabulary: -log 151936
    assert abs(-math.log(151936) - (-11.931215)) < 1e-6


def test_single_entry_vocabulary_is_certain():
    h = np.array([[0.5, -1.25]], np.float32)
    logp, lse, zsel = _lp(h, np.array([[2.0, 3.0]], np.float32), np.array([0], np.int32))
    assert logp[0] == 0.0 and lse[0] == zsel[0] == 0.5 * 2.0 - 1.25 * 3.0


def test_two_entry_vocabulary_closed_form_including_large_logits():
    # z_0 = 3 h, z_1 = -2 h: logp_0 = -log1p(exp(z_1 - z_0))
    for hv in (0.25, -1.5, 300.0, -400.0):
        h = np.array([[hv]] * 2, np.float32)
        w = np.array([[3.0], [-2.0]], np.float32)
        logp, lse, _ = _lp(np.repeat(h, 64, 1), np.repeat(w, 64, 1) / 64, np.array([0, 1], np.int32))
        z0, z1 = 3.0 * hv, -2.0 * hv
        np.testing.assert_allclose(logp[0], -math.log1p(math.exp(z1 - z0)) if z1 < z0
                                   else (z0 - z1) - math.log1p(math.exp(z0 - z1)), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(logp[1], -math.log1p(math.exp(z0 - z1)) if z0 < z1
                                   else (z1 - z0) - math.log1p(math.exp(z1 - z0)), rtol=1e-14, atol=1e-15)
        assert np.all(np.isfinite(lse))


def test_brute_force_against_exact_logits_and_decimal_softmax():
    rng = np.random.default_rng(2)
    n, d, v = 5, 3, 7                      # non-square: a transposed W fails
    h = rng.standard_normal((n, d)).astype(np.float32)
    w = (rng.standard_normal((v, d)) * 2).astype(np.float32)
    ids = rng.integers(0, v, n).astype(np.int32)
    logp, lse, zsel = _lp(h, w, ids)
    z = _exact_logits(h, w)
    for t in range(n):
        assert abs(zsel[t] - float(z[t][ids[t]])) <= 1e-15 * max(1.0, abs(float(z[t][ids[t]])))
        assert abs(logp[t] - _brute_logp(z[t], int(ids[t]))) < 1e-13
    # every id of one row: the probabilities sum to one
    ids_all = np.arange(v, dtype=np.int32)
    logp_all, lse_all, _ = _lp(np.repeat(h[:1], v, 0), w, ids_all)
    assert abs(np.exp(logp_all).sum() - 1.0) < 1e-14
    assert np.all(lse_all == lse_all[0])


def test_integer_exact_logits_bf16():
    """Inputs are small multiples of 2^-3 (exact in bf16): every logit is an
    exact rational, so zsel must equal the integer-arithmetic value."""
    rng = np.random.default_rng(3)
    n, d, v = 6, 128, 50
    hq = rng.integers(-16, 17, (n, d))
    wq = rng.integers(-16, 17, (v, d))
    h_bits = torch.from_numpy((hq / 8.0).astype(np.float32)).to(torch.bfloat16)
    w_bits = torch.from_numpy((wq / 8.0).astype(np.float32)).to(torch.bfloat16)
    ids = rng.integers(0, v, n).astype(np.int32)
    _, _, zsel = _lp(h_bits, w_bits, ids, dtype=oracle.BF16)
    exact = (hq * wq[ids]).sum(1) / 64.0
    np.testing.assert_array_equal(zsel, exact)
    # same values through the fp32 path give identical results
    a = _lp(h_bits.float().numpy(), w_bits.float().numpy(), ids, dtype=oracle.F32)
    b = _lp(h_bits, w_bits, ids, dtype=oracle.BF16)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_one_hot_rows_select_weight_entries():
    rng = np.random.default_rng(4)
    d, v = 64, 40
    w = rng.standard_normal((v, d)).astype(np.float32)
    ks = [0, 17, 63]
    h = np.zeros((3, d), np.float32)
    for r, k in enumerate(ks):
        h[r, k] = 1.0
    ids = np.array([5, 0, 39], np.int32)
    logp, lse, zsel = _lp(h, w, ids)
    for r, k in enumerate(ks):
        assert zsel[r] == float(w[ids[r], k])
        col = [Fraction(float(x)) for x in w[:, k]]
        ref = float((sum(_dec(c).exp() for c in col)).ln())
        assert abs(lse[r] - ref) < 1e-13


def test_out_of_range_ids_are_nan_and_rows_subset_matches():
    rng = np.random.default_rng(5)
    h = rng.standard_normal((10, 64)).astype(np.float32)
    w = rng.standard_normal((33, 64)).astype(np.float32)
    ids = rng.integers(0, 33, 10).astype(np.int32)
    ids[2], ids[7] = -100, 33               # ignore-index style and one past the end
    logp, lse, _ = _lp(h, w, ids)
    assert np.isnan(logp[2]) and np.isnan(logp[7]) and np.all(np.isfinite(lse))
    rows = np.array([9, 0, 4], np.int64)
    sub = _lp(h, w, ids, rows=rows)
    np.testing.assert_array_equal(sub[0], logp[rows])


# ---------------------------------------------------------------------------
# mismatch statistics
# ---------------------------------------------------------------------------

def _stats(lt, lr, cu, mask=None, c=2.0, lo=-0.01, hi=0.01):
    return oracle.mismatch_stats(np.asarray(lt, np.float32), np.asarray(lr, np.float32),
                                 mask, np.asarray(cu, np.int32), clip_c=c, seq_lo=lo, seq_hi=hi)


def test_vexact_table1_sign_and_derived_estimators():
    g = json.load(open(os.path.join(GOLDEN, "vexact_table1.json")))
    r = _stats(g["logp_train"], g["logp_rollout"], [0, 8])
    tol = 1.5 * 10.0 ** -g["printed_decimals"]    # three roundings of 5e-4
    np.testing.assert_allclose(r["token"]["delta"], g["delta"], rtol=0, atol=tol)
    # sign: the flipped token has delta = train - rollout < 0
    i = g["argmax_flip_index"]
    assert r["token"]["delta"][i] < -0.1
    d = Decimal(repr(float(np.float32(g["logp_train"][i])))) - \
        Decimal(repr(float(np.float32(g["logp_rollout"][i]))))
    assert abs(r["token"]["k1"][i] - float(-d)) < 1e-15
    assert abs(r["token"]["k2"][i] - float(d * d / 2)) < 1e-16
    assert abs(r["token"]["k3"][i] - float(d.exp() - 1 - d)) < 1e-16
    assert abs(r["token"]["k1"][i] - 0.133) < 1e-7
    assert abs(r["token"]["k2"][i] - 0.0088445) < 1e-7
    assert abs(r["token"]["k3"][i] - 0.0084651) < 1e-7
    # mean delta = -0.0175 -> geometric mean ratio 0.983 < 0.99 -> rejected
    assert r["seq"]["reject"][0] == 1
    r2 = _stats(g["logp_train"], g["logp_rollout"], [0, 8], lo=math.log(0.99), hi=math.log(1.01))
    assert r2["seq"]["reject"][0] == 1


def test_zero_mismatch_gives_zero_estimators():
    rng = np.random.default_rng(6)
    lt = -np.abs(rng.standard_normal(100)).astype(np.float32)
    r = _stats(lt, lt, [0, 30, 30, 100])
    t = r["token"]
    assert np.all(t["delta"] == 0) and np.all(t["k1"] == 0) and np.all(t["k2"] == 0)
    assert np.all(t["k3"] == 0) and np.all(t["ratio"] == 1) and np.all(t["tis_w"] == 1)
    assert not t["clipped"].any() and not r["seq"]["reject"].any()
    b = r["batch"]
    assert b["tok_mean_k3"] == 0 and b["clip_ratio"] == 0 and b["n_valid"] == 100
    assert b["n_seq_nonempty"] == 2 and b["tok_mean_tis_w"] == 1.0


def test_k3_nonnegative_and_matches_closed_form():
    deltas = np.concatenate([np.geomspace(1e-12, 20, 200), -np.geomspace(1e-12, 20, 200)])
    lr = np.full(deltas.size, -30.0, np.float32)
    lt = (lr.astype(np.float64) + deltas).astype(np.float32)
    r = _stats(lt, lr, [0, deltas.size])
    t = r["token"]
    assert np.all(t["k3"] >= 0)
    for i in range(0, deltas.size, 7):
        d = Decimal(float(t["delta"][i]))
        ref = d.exp() - 1 - d
        # (r - 1) - log r evaluated in fp64: each operand of the final
        # subtraction is within an ulp, so the error is bounded by a few ulps
        # of |delta| + |k3| (the cancellation of the definition itself)
        bound = Decimal(2) ** -51 * (abs(d) + abs(ref))
        assert abs(Decimal(float(t["k3"][i])) - ref) <= bound
        assert t["k2"][i] == float(t["delta"][i]) ** 2 / 2
        assert t["ratio"][i] == pytest.approx(float(d.exp()), rel=1e-15)


def test_constant_delta_means_are_exact():
    c = 2.0 ** -6
    lr = np.full(48, -1.0, np.float32)
    lt = lr + np.float32(c)
    r = _stats(lt, lr, [0, 16, 48])
    assert np.all(r["seq"]["mean_delta"] == c) and np.all(r["seq"]["mean_k1"] == -c)
    assert np.all(r["seq"]["mean_k2"] == c * c / 2)
    assert r["batch"]["tok_mean_delta"] == c and r["batch"]["seq_mean_delta"] == c
    assert r["seq"]["reject"].all()          # 2^-6 = 0.015625 > 0.01


def test_truncated_is_clips_above_log_c():
    lr = np.full(10, -2.0, np.float32)
    r = _stats(lr + np.float32(1.0), lr, [0, 10])          # delta 1 > log 2
    assert r["token"]["clipped"].all() and np.all(r["token"]["tis_w"] == 2.0)
    assert r["batch"]["clip_ratio"] == 1.0 and r["batch"]["tok_mean_tis_w"] == 2.0
    r = _stats(lr + np.float32(0.5), lr, [0, 10])          # delta 0.5 < log 2
    assert not r["token"]["clipped"].any()
    np.testing.assert_allclose(r["token"]["tis_w"], math.exp(0.5), rtol=1e-15)


def test_sequence_mean_then_batch_mean_differs_from_token_mean():
    # sequence A: two tokens with delta 1; sequence B: three tokens with delta 0
    lr = np.zeros(5, np.float32) - 1.0
    lt = lr.copy()
    lt[:2] = 0.0
    r = _stats(lt, lr, [0, 2, 5])
    assert r["batch"]["tok_mean_delta"] == 0.4
    assert r["batch"]["seq_mean_delta"] == 0.5
    assert r["batch"]["seq_mean_k2"] == 0.25 and r["batch"]["tok_mean_k2"] == 0.2
    assert list(r["seq"]["mean_delta"]) == [1.0, 0.0]
    assert list(r["seq"]["reject"]) == [1, 0]
    assert r["batch"]["reject_frac"] == 0.5


def test_mask_nan_and_empty_sequences():
    lt = np.array([-1, -1, -1, -1, -1, -1, -1], np.float32)
    lr = np.array([-1.5, np.nan, -1, -1, -1, -1, np.inf], np.float32)
    mask = np.array([1, 1, 0, 0, 1, 0, 1], np.uint8)
    cu = [0, 2, 2, 4, 7]                    # sequence 1 empty, sequence 2 all masked
    r = _stats(lt, lr, cu, mask=mask)
    s = r["seq"]
    assert list(s["n_valid"]) == [1, 0, 0, 1]
    assert list(s["n_nan"]) == [1, 0, 0, 1]
    assert list(s["reject"]) == [1, 0, 0, 0]
    assert s["mean_delta"][0] == 0.5 and s["mean_delta"][1] == 0 and s["mean_delta"][2] == 0
    b = r["batch"]
    assert b["n_valid"] == 2 and b["n_nan"] == 2 and b["nan_ratio"] == 2 / 4
    assert b["n_seq_nonempty"] == 2 and b["seq_mean_delta"] == 0.25
    t = r["token"]
    assert t["tis_w"][1] == 0 and t["ratio"][2] == 1 and t["tis_w"][2] == 0
    assert b["max_abs_delta"] == 0.5


def test_rejection_window_in_log_domain():
    lo, hi = math.log(0.99), math.log(1.01)
    base = np.full(4, -3.0, np.float32)
    cases = {lo - 1e-4: 1, lo + 1e-4: 0, 0.0: 0, hi - 1e-4: 0, hi + 1e-4: 1}
    for mean, want in cases.items():
        lt = (base.astype(np.float64) + mean).astype(np.float32)
        r = _stats(lt, base, [0, 4], lo=lo, hi=hi)
        m = r["seq"]["mean_delta"][0]
        gm = Decimal(float(m)).exp()            # geometric mean of the ratios
        assert (gm < Decimal("0.99") or gm > Decimal("1.01")) == bool(want)
        assert r["seq"]["reject"][0] == want


def test_k3_rejection_uses_mean_k3_not_k2():
    # constant delta c per sequence: mean k3 = e^c - 1 - c exactly as its own
    # closed form, mean k2 = c^2 / 2.  For c = +-0.3 the two k2 are equal
    # (0.045) while k3(+0.3) = 0.04986 > 0.0475 > k3(-0.3) = 0.04082, so only
    # a K3 test separates them.
    n = 8
    lr = np.full(3 * n, -2.0, np.float32)
    lt = lr.astype(np.float64).copy()
    lt[:n] += 0.3
    lt[n:2 * n] -= 0.3
    lt = lt.astype(np.float32)
    cu = [0, n, 2 * n, 2 * n, 3 * n]          # third sequence empty, fourth zero delta
    r = oracle.mismatch_stats(lt, lr, None, np.asarray(cu, np.int32), clip_c=2.0,
                              seq_lo=-1.0, seq_hi=1.0, seq_k3_hi=0.0475)
    d = r["token"]["delta"]
    for j, (a, b) in enumerate([(0, n), (n, 2 * n)]):
        c = Decimal(float(d[a]))
        assert np.all(d[a:b] == d[a])
        assert abs(Decimal(float(r["seq"]["mean_k3"][j])) - (c.exp() - 1 - c)) < Decimal(1e-15)
    assert list(r["seq"]["reject_k3"]) == [1, 0, 0, 0]
    assert list(r["seq"]["reject"]) == [0, 0, 0, 0]
    assert r["batch"]["n_seq_rejected_k3"] == 1 and r["batch"]["n_seq_nonempty"] == 3
    assert r["batch"]["reject_k3_frac"] == 1 / 3
    # strict bound: a bound equal to a sequence's mean k3 does not reject it
    r2 = oracle.mismatch_stats(lt, lr, None, np.asarray(cu, np.int32), clip_c=2.0,
                               seq_lo=-1.0, seq_hi=1.0, seq_k3_hi=float(r["seq"]["mean_k3"][1]))
    assert list(r2["seq"]["reject_k3"]) == [1, 0, 0, 0]
    # the default bound (+inf) never rejects
    r3 = oracle.mismatch_stats(lt, lr, None, np.asarray(cu, np.int32), clip_c=2.0,
                               seq_lo=-1.0, seq_hi=1.0)
    assert not r3["seq"]["reject_k3"].any() and r3["batch"]["reject_k3_frac"] == 0


# ---------------------------------------------------------------------------
# extra metrics: extreme-token rate, relative difference, quantiles
# ---------------------------------------------------------------------------

def _extras(lt, lr, mask=None, tau=0.1, rq=(), aq=()):
    return oracle.mismatch_extras(np.asarray(lt, np.float32), np.asarray(lr, np.float32),
                                  None if mask is None else np.asarray(mask, np.uint8),
                                  tok_tau=tau, ratio_q=rq, abs_q=aq)


def test_extreme_rate_is_strict_and_two_sided():
    lr = np.full(10, -4.0, np.float32)
    offs = np.array([0.25, -0.25, 0.125, -0.125, 0.5, -0.5, 0, 0, 1.0, -1.0])
    lt = (lr + offs).astype(np.float32)         # exact: dyadic offsets
    r = _extras(lt, lr, tau=0.25)
    assert r["n_extreme"] == 4                   # |delta| = 0.5, 0.5, 1, 1; 0.25 is not > 0.25
    assert r["extreme_frac"] == 0.4 and r["n_valid"] == 10
    mask = np.array([1] * 8 + [0, 0], np.uint8)  # masking drops the two |delta| = 1
    r = _extras(lt, lr, mask=mask, tau=0.25)
    assert r["n_extreme"] == 2 and r["n_valid"] == 8 and r["extreme_frac"] == 0.25
    r = _extras(lt, lr, tau=float("inf"))
    assert r["n_extreme"] == 0 and r["extreme_frac"] == 0


def test_rel_diff_equals_mean_abs_delta_when_train_logp_is_minus_one():
    # |lt| = 1 everywhere: the mean of |delta| / (1 + 1e-8) is the pinned
    # mean |delta| of the statistics pass, divided once by 1 + 1e-8
    rng = np.random.default_rng(11)
    n = 200
    lt = np.full(n, -1.0, np.float32)
    lr = (lt + rng.normal(0, 0.05, n)).astype(np.float32)
    mask = (rng.random(n) < 0.8).astype(np.uint8)
    lr[3] = np.nan                               # non-finite delta: left out of both
    mask[3] = 1
    r = _extras(lt, lr, mask=mask)
    st = oracle.mismatch_stats(lt, lr, mask, np.asarray([0, n], np.int32), clip_c=2.0,
                               seq_lo=-1.0, seq_hi=1.0)
    assert r["n_valid"] == st["batch"]["n_valid"]
    assert r["mean_rel_diff"] == pytest.approx(st["batch"]["mean_abs_delta"] / (1 + 1e-8),
                                               rel=1e-14)
    # the denominator is the trainer side: varying |lr| instead changes nothing
    # in this construction, while varying |lt| does
    lt2 = (lt * 2).astype(np.float32)            # |lt| = 2, same deltas after shifting lr
    lr2 = (lr.astype(np.float64) - 1.0).astype(np.float32)
    r2 = _extras(lt2, lr2, mask=mask)
    assert r2["mean_rel_diff"] == pytest.approx(r["mean_rel_diff"] / 2, rel=1e-6)


def test_rel_diff_zero_train_logp_and_scale_invariance():
    # lt = 0 exactly (a certain token): |delta| / 1e-8
    r = _extras([0.0], [-(2.0 ** -20)])
    assert r["mean_rel_diff"] == pytest.approx(95.367431640625, rel=1e-15)
    # scaling both log-probabilities by 2^k leaves |delta| / |lt| unchanged up
    # to the 1e-8 guard
    rng = np.random.default_rng(12)
    lt = -rng.uniform(0.5, 3.0, 64).astype(np.float32)
    lr = (lt + rng.normal(0, 0.01, 64)).astype(np.float32)
    a = _extras(lt, lr)["mean_rel_diff"]
    b = _extras(lt * np.float32(8), lr * np.float32(8))["mean_rel_diff"]
    assert b == pytest.approx(a, rel=1e-7) and a > 1e-4


def test_quantiles_match_numpy_linear_method():
    rng = np.random.default_rng(13)
    for n in (1, 2, 3, 7, 100, 1001):
        lr = -rng.uniform(0.0, 5.0, n).astype(np.float32)
        lt = (lr + rng.normal(0, 0.02, n)).astype(np.float32)
        mask = (rng.random(n) < 0.7).astype(np.uint8)
        mask[0] = 1
        qs = (0.01, 0.5, 0.99)
        r = _extras(lt, lr, mask=mask, rq=qs, aq=(0.95,))
        d = lt.astype(np.float64)[mask != 0] - lr.astype(np.float64)[mask != 0]
        want_r = np.quantile(np.exp(d), qs, method="linear")
        want_a = np.quantile(np.abs(d), 0.95, method="linear")
        np.testing.assert_allclose(r["ratio_q"], want_r, rtol=1e-14, atol=0)
        assert r["abs_q"][0] == pytest.approx(want_a, rel=1e-14, abs=1e-300)


def test_quantiles_of_many_tokens_match_numpy():
    """Above 2^20 valid tokens the oracle sorts in pieces on several threads
    and merges them; the quantiles must still be numpy's on the same data."""
    rng = np.random.default_rng(29)
    n = (1 << 21) + 12345
    lr = -rng.uniform(0.0, 5.0, n).astype(np.float32)
    lt = (lr + rng.normal(0, 0.02, n)).astype(np.float32)
    mask = (rng.random(n) < 0.9).astype(np.uint8)
    qs = (0.0, 0.01, 0.5, 0.99)
    r = _extras(lt, lr, mask=mask, rq=qs, aq=())
    d = lt.astype(np.float64)[mask != 0] - lr.astype(np.float64)[mask != 0]
    np.testing.assert_allclose(r["ratio_q"], np.quantile(np.exp(d), qs, method="linear"),
                               rtol=1e-14, atol=0)
    for aq in ((0.95, 1.0, 0.25, 0.5),):
        ra = _extras(lt, lr, mask=mask, rq=(), aq=aq)
        np.testing.assert_allclose(ra["abs_q"], np.quantile(np.abs(d), aq, method="linear"),
                                   rtol=1e-14, atol=0)


def test_quantile_order_statistics_and_edge_cases():
    lr = np.full(5, -1.0, np.float32)
    offs = np.array([0.5, -0.25, 0.0, 0.125, -1.0])
    lt = (lr + offs).astype(np.float32)
    r = _extras(lt, lr, rq=(0.0, 0.5, 1.0, 0.25), aq=(0.0, 1.0, 0.5, 0.375))
    # five values: q = 0.25 lands on the second order statistic exactly,
    # q = 0.375 half-way between the second and third
    assert r["ratio_q"] == [math.exp(-1.0), 1.0, math.exp(0.5), math.exp(-0.25)]
    assert r["abs_q"][:3] == [0.0, 1.0, 0.25]
    assert r["abs_q"][3] == 0.125 + (0.25 - 0.125) * 0.5
    # order of the tokens does not matter
    for perm in ([4, 3, 2, 1, 0], [2, 0, 4, 1, 3]):
        rp = _extras(lt[perm], lr[perm], rq=(0.0, 0.5, 1.0, 0.25), aq=(0.0, 1.0, 0.5, 0.375))
        assert rp["ratio_q"] == r["ratio_q"] and rp["abs_q"] == r["abs_q"]
    # one valid token: every quantile is its value; none: zeros
    m1 = np.array([0, 0, 0, 1, 0], np.uint8)
    r1 = _extras(lt, lr, mask=m1, rq=(0.01, 0.99), aq=(0.95,))
    assert r1["ratio_q"] == [math.exp(0.125)] * 2 and r1["abs_q"] == [0.125]
    r0 = _extras(lt, lr, mask=np.zeros(5, np.uint8), rq=(0.5,), aq=(0.95,))
    assert r0["ratio_q"] == [0.0] and r0["abs_q"] == [0.0] and r0["n_valid"] == 0
    assert r0["mean_rel_diff"] == 0 and r0["extreme_frac"] == 0
    # all deltas equal (zero mismatch): every quantile is that value
    rz = _extras(lr, lr, rq=(0.01, 0.5, 0.99), aq=(0.95,))
    assert rz["ratio_q"] == [1.0, 1.0, 1.0] and rz["abs_q"] == [0.0]
    with pytest.raises(ValueError):
        _extras(lt, lr, rq=(1.5,))
    with pytest.raises(ValueError):
        _extras(lt, lr, tau=float("nan"))


# ---------------------------------------------------------------------------
# backward of the selected-token log-probability
# ---------------------------------------------------------------------------

def _bw_case(seed=21, n=6, d=16, v=11):
    rng = np.random.default_rng(seed)
    # dyadic values: h +- 2^-12 and W +- 2^-12 are exact in fp32
    h = (np.round(rng.standard_normal((n, d)) * 64) / 64).astype(np.float32)
    w = (np.round(rng.standard_normal((v, d)) * 16) / 64).astype(np.float32)
    ids = rng.integers(0, v, n).astype(np.int32)
    g = rng.standard_normal(n)
    g[2] = 0.0                                   # a token that does not contribute
    return h, w, ids, g


def _objective(h, w, ids, g):
    """sum_t g_t logp_t with the (separately pinned) fp64 forward."""
    logp, _, _ = _lp(h, w, ids, dtype=oracle.F32)
    return float(np.dot(g, logp))


def test_backward_matches_central_differences_of_the_forward():
    h, w, ids, g = _bw_case()
    dh, dw = oracle.logprob_backward(h, w, ids, g, dtype=oracle.F32)
    eps = 2.0 ** -12
    rng = np.random.default_rng(3)
    for _ in range(12):
        t, k = int(rng.integers(0, h.shape[0])), int(rng.integers(0, h.shape[1]))
        hp, hm = h.copy(), h.copy()
        hp[t, k] += np.float32(eps)
        hm[t, k] -= np.float32(eps)
        fd = (_objective(hp, w, ids, g) - _objective(hm, w, ids, g)) / (2 * eps)
        assert abs(fd - dh[t, k]) <= 1e-6 * (1 + abs(dh[t, k])), (t, k, fd, dh[t, k])
    for _ in range(12):
        c, k = int(rng.integers(0, w.shape[0])), int(rng.integers(0, w.shape[1]))
        wp, wm = w.copy(), w.copy()
        wp[c, k] += np.float32(eps)
        wm[c, k] -= np.float32(eps)
        fd = (_objective(h, wp, ids, g) - _objective(h, wm, ids, g)) / (2 * eps)
        assert abs(fd - dw[c, k]) <= 1e-6 * (1 + abs(dw[c, k])), (c, k, fd, dw[c, k])


def test_backward_invariants_and_row_selection():
    h, w, ids, g = _bw_case(seed=22, n=9, d=8, v=13)
    dh, dw = oracle.logprob_backward(h, w, ids, g, dtype=oracle.F32)
    # the softmax derivative sums to zero over the vocabulary, so the rows
    # of dW sum to zero; a token with g = 0 has dh = 0
    assert np.abs(dw.sum(axis=0)).max() < 1e-12
    assert np.all(dh[2] == 0)
    # linear in g
    dh2, dw2 = oracle.logprob_backward(h, w, ids, 2 * g, dtype=oracle.F32)
    np.testing.assert_allclose(dh2, 2 * dh, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dw2, 2 * dw, rtol=1e-14, atol=1e-15)
    # selected rows are the same rows
    sdh, sdw = oracle.logprob_backward(h, w, ids, g, dtype=oracle.F32, dh_rows=[4, 0],
                                       dw_rows=[12, 3, 3])
    np.testing.assert_array_equal(sdh, dh[[4, 0]])
    np.testing.assert_array_equal(sdw, dw[[12, 3, 3]])


# ---------------------------------------------------------------------------
# PPO / GRPO clipped surrogate
# ---------------------------------------------------------------------------

def _ppo(lp, ot, orr, a, mask=None, lo=0.2, hi=0.28, bypass=False, c=0.0, scale=0.0):
    f = lambda x: np.asarray(x, np.float32)
    return oracle.ppo_loss(f(lp), f(ot), f(orr), f(a), mask, eps_lo=lo, eps_hi=hi,
                           bypass=bypass, tis_c=c, grad_scale=scale)


def test_ppo_clip_branches_closed_form():
    # ratios 1.5 (above 1 + 0.28) and 0.5 (below 1 - 0.2) with both signs of A
    old = np.zeros(4, np.float32) - 2.0
    d = np.array([math.log(1.5), math.log(1.5), math.log(0.5), math.log(0.5)])
    lp = (old.astype(np.float64) + d).astype(np.float32)
    a = [1.0, -1.0, 1.0, -1.0]
    r = _ppo(lp, old, old, a)
    rr = np.exp(lp.astype(np.float64) - old.astype(np.float64))
    # A > 0, r > 1 + eps: clipped at (1 + eps) A, no gradient
    assert r["loss"][0] == -1.28 and r["grad"][0] == 0 and r["clipped"][0] == 1
    # A < 0, r > 1 + eps: r A is the smaller term, gradient flows
    assert r["loss"][1] == rr[1] and r["clipped"][1] == 0
    assert r["grad"][1] == pytest.approx(rr[1] / 4, rel=1e-15)   # -(r A) / n with A = -1
    # A > 0, r < 1 - eps: r A is the smaller term, gradient flows
    assert r["loss"][2] == -rr[2] and r["clipped"][2] == 0
    # A < 0, r < 1 - eps: clipped at (1 - eps) A
    assert r["loss"][3] == pytest.approx(0.8, rel=1e-15) and r["grad"][3] == 0
    assert r["batch"]["clip_frac"] == 0.5 and r["batch"]["n_valid"] == 4


def test_ppo_gradient_matches_central_differences():
    rng = np.random.default_rng(31)
    n = 40
    ot = (-rng.uniform(0.5, 3, n)).astype(np.float32)
    orr = (ot + rng.normal(0, 0.05, n)).astype(np.float32)
    lp = (ot + rng.normal(0, 0.2, n)).astype(np.float32)
    a = rng.normal(0, 1, n).astype(np.float32)
    for bypass, c in ((False, 0.0), (False, 2.0), (True, 0.0)):
        base = _ppo(lp, ot, orr, a, bypass=bypass, c=c)
        eps = 2.0 ** -16
        for t in range(0, n, 3):
            r_t = base["ratio"][t]
            # skip tokens within reach of a clip boundary
            if min(abs(r_t - 1.28), abs(r_t - 0.8)) < 1e-3:
                continue
            lpp, lpm = lp.copy(), lp.copy()
            lpp[t] += np.float32(eps)
            lpm[t] -= np.float32(eps)
            fd = (_ppo(lpp, ot, orr, a, bypass=bypass, c=c)["batch"]["mean_loss"] -
                  _ppo(lpm, ot, orr, a, bypass=bypass, c=c)["batch"]["mean_loss"]) / (2 * eps)
            assert abs(fd - base["grad"][t]) < 1e-7, (bypass, c, t, fd, base["grad"][t])


def test_ppo_scaled_gradient_is_that_of_the_scaled_token_sum():
    # grad_scale > 0: the derivative of grad_scale * sum_t loss_t, by central
    # differences of the per-token losses (masked tokens included as zeros)
    rng = np.random.default_rng(35)
    n = 24
    ot = (-rng.uniform(0.5, 3, n)).astype(np.float32)
    orr = (ot + rng.normal(0, 0.05, n)).astype(np.float32)
    lp = (ot + rng.normal(0, 0.2, n)).astype(np.float32)
    a = rng.normal(0, 1, n).astype(np.float32)
    mask = (np.arange(n) % 5 != 0).astype(np.uint8)
    scale = 1.0 / 4096
    base = _ppo(lp, ot, orr, a, mask=mask, c=2.0, scale=scale)
    eps = 2.0 ** -16
    checked = 0
    for t in range(n):
        r_t = base["ratio"][t]
        if min(abs(r_t - 1.28), abs(r_t - 0.8)) < 1e-3:
            continue
        lpp, lpm = lp.copy(), lp.copy()
        lpp[t] += np.float32(eps)
        lpm[t] -= np.float32(eps)
        fd = scale * (_ppo(lpp, ot, orr, a, mask=mask, c=2.0)["loss"].sum() -
                      _ppo(lpm, ot, orr, a, mask=mask, c=2.0)["loss"].sum()) / (2 * eps)
        assert abs(fd - base["grad"][t]) < 1e-10, (t, fd, base["grad"][t])
        checked += 1
    assert checked >= 20 and base["grad"][0] == 0.0          # token 0 is masked
    # the mean's gradient is the scaled one at scale 1 / n_valid, and every
    # other output does not depend on the scale
    mean = _ppo(lp, ot, orr, a, mask=mask, c=2.0)
    nv = mean["batch"]["n_valid"]
    assert np.allclose(_ppo(lp, ot, orr, a, mask=mask, c=2.0, scale=1.0 / nv)["grad"],
                       mean["grad"], rtol=1e-15, atol=0)
    for k in ("loss", "ratio", "contrib", "clipped"):
        assert np.array_equal(base[k], mean[k])
    assert base["batch"] == mean["batch"]


def test_ppo_contribution_has_the_gradient_of_minus_r_a_and_tis_moves_the_ratio():
    rng = np.random.default_rng(32)
    n = 16
    ot = (-rng.uniform(0.5, 3, n)).astype(np.float32)
    orr = (ot + rng.normal(0, 0.02, n)).astype(np.float32)
    lp = (ot + rng.normal(0, 0.02, n)).astype(np.float32)
    a = rng.normal(0, 1, n).astype(np.float32)
    base = _ppo(lp, ot, orr, a)
    eps = 2.0 ** -16
    for t in range(n):
        lpp, lpm = lp.copy(), lp.copy()
        lpp[t] += np.float32(eps)
        lpm[t] -= np.float32(eps)
        fd = (_ppo(lpp, ot, orr, a)["contrib"][t] - _ppo(lpm, ot, orr, a)["contrib"][t]) / (2 * eps)
        assert fd == pytest.approx(-base["ratio"][t] * float(a[t]), rel=1e-6, abs=1e-9)
        assert base["contrib"][t] == pytest.approx(-(base["ratio"][t] - 1) * float(a[t]),
                                                   rel=1e-12, abs=1e-15)
    # an untruncated r_corr weight times the trainer-side ratio is the
    # rollout-side ratio: recompute + TIS equals bypass where nothing clips
    rec = _ppo(lp, ot, orr, a, c=100.0)
    byp = _ppo(lp, ot, orr, a, bypass=True)
    ok = (rec["clipped"] == 0) & (byp["clipped"] == 0)
    assert ok.sum() >= n - 2
    np.testing.assert_allclose(rec["loss"][ok], byp["loss"][ok], rtol=1e-14, atol=1e-16)
    # truncation: with C below every r_corr the weight is C
    low = _ppo(lp, ot, orr, a, c=1e-3)
    assert low["batch"]["mean_tis_w"] == pytest.approx(1e-3, rel=1e-15)


def test_ppo_mask_and_nan_tokens():
    lp = np.array([-1.0, -1.0, np.nan, -1.0], np.float32)
    ot = np.array([-1.1, -1.1, -1.1, -1.1], np.float32)
    a = np.array([1.0, 2.0, 1.0, 5.0], np.float32)
    mask = np.array([1, 1, 1, 0], np.uint8)
    r = _ppo(lp, ot, ot, a, mask=mask)
    b = r["batch"]
    assert b["n_valid"] == 2 and b["n_nan"] == 1
    assert r["loss"][2] == 0 and r["grad"][2] == 0 and r["loss"][3] == 0
    rr = math.exp(float(np.float32(-1.0)) - float(np.float32(-1.1)))
    assert b["mean_loss"] == pytest.approx(-(rr * 1 + rr * 2) / 2, rel=1e-15)


# ---------------------------------------------------------------------------
# temperature and entropy
# ---------------------------------------------------------------------------

def _lpx(h, w, ids, tau, dtype=oracle.F32):
    return oracle.logprob_ex(h, w, ids, dtype=dtype, temperature=tau, nthreads=2)


def _bf16_exact(rng, shape, scale):
    """float32 values that are exact bf16 numbers."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return oracle.bf16_decode(oracle.bf16_round_rne(x).ravel()).reshape(shape).astype(np.float32)


def test_temperature_divides_the_logits():
    # softmax(z / 2) from W is softmax(z') from W / 2: halving bf16 weights is
    # exact, so logp, lse and entropy agree to the bit; likewise tau = 1/2 and 2 W
    rng = np.random.default_rng(41)
    h = _bf16_exact(rng, (6, 64), 1.0)
    w = _bf16_exact(rng, (300, 64), 0.5)
    ids = rng.integers(0, 300, 6).astype(np.int32)
    for tau, wscaled in ((2.0, w / 2), (0.5, w * 2)):
        a = _lpx(h, w, ids, tau)
        b = _lpx(h, wscaled, ids, 1.0)
        for k in ("logp", "lse", "entropy", "zsel"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"tau={tau} {k}")
    # tau = 1 is the plain forward
    plain = _lp(h, w, ids)
    one = _lpx(h, w, ids, 1.0)
    np.testing.assert_array_equal(one["logp"], plain[0])
    np.testing.assert_array_equal(one["lse"], plain[1])


def test_entropy_closed_forms():
    rng = np.random.default_rng(42)
    # equal logits: uniform distribution, H = log V at any temperature
    for tau in (0.3, 1.0, 7.0):
        r = _lpx(rng.standard_normal((3, 32)).astype(np.float32), np.zeros((777, 32), np.float32),
                 np.array([0, 5, 776], np.int32), tau)
        np.testing.assert_allclose(r["entropy"], math.log(777), rtol=1e-12)   # 777 rounded terms
        np.testing.assert_allclose(r["logp"], -math.log(777), rtol=1e-14)
    # two entries: p = sigmoid(dz / tau), H = binary entropy
    for hv in (0.25, -1.5, 6.0):
        for tau in (0.5, 1.0, 3.0):
            h = np.full((1, 64), hv, np.float32)
            w = np.repeat(np.array([[3.0], [-2.0]], np.float32), 64, 1) / 64
            r = _lpx(h, w, np.array([1], np.int32), tau)
            x = 5.0 * hv / tau                      # (z0 - z1) / tau
            p1 = 1.0 / (1.0 + math.exp(x))
            hb = math.log1p(math.exp(-abs(x))) + abs(x) * (1.0 / (1.0 + math.exp(abs(x))))
            # lp = z - lse cancels to an absolute error of ~ulp(|z| / tau)
            np.testing.assert_allclose(r["entropy"][0], hb, rtol=1e-12, atol=1e-15 * (1 + abs(x)))
            lp1 = -math.log1p(math.exp(x)) if x < 0 else -x - math.log1p(math.exp(-x))
            np.testing.assert_allclose(r["logp"][0], lp1, rtol=1e-13, atol=1e-15 * (1 + abs(x)))
            assert abs(math.exp(lp1) - p1) < 1e-15
    # a dominant logit at a low temperature: H -> 0, logp of the winner -> 0
    h = np.ones((1, 16), np.float32)
    w = np.zeros((50, 16), np.float32)
    w[7] = 1.0 / 16
    r = _lpx(h, w, np.array([7], np.int32), 0.01)     # gap 1 / 0.01 = 100 nats
    # 49 losers, each p = e^-100 and -log p = 100: H ~ 49 * 101 e^-100 ~ 1.8e-40
    assert 0 <= r["entropy"][0] < 1e-39 and abs(r["logp"][0]) < 1e-40


def test_entropy_matches_scipy_on_exact_logits():
    import scipy.special
    import scipy.stats
    rng = np.random.default_rng(43)
    # integer-valued inputs: every logit is an exact small integer in fp64
    h = rng.integers(-3, 4, (5, 24)).astype(np.float32)
    w = rng.integers(-2, 3, (200, 24)).astype(np.float32)
    ids = rng.integers(0, 200, 5).astype(np.int32)
    z = h.astype(np.float64) @ w.astype(np.float64).T
    for tau in (0.7, 1.0, 2.5):
        r = _lpx(h, w, ids, tau)
        p = scipy.special.softmax(z / tau, axis=1)
        np.testing.assert_allclose(r["entropy"], scipy.stats.entropy(p, axis=1), rtol=1e-12)
        np.testing.assert_allclose(r["logp"], np.log(p[np.arange(5), ids]), rtol=1e-12)
        np.testing.assert_allclose(r["lse"], scipy.special.logsumexp(z / tau, axis=1), rtol=1e-14)


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def test_rmsnorm_constant_rows_give_the_gain():
    rng = np.random.default_rng(44)
    d = 96
    gamma = _bf16_exact(rng, (d,), 1.0)
    x = np.zeros((4, d), np.float32)
    x[0] = 3.0
    x[1] = -0.75
    x[2, ::2], x[2, 1::2] = 2.0, -2.0          # |x| constant: rms = 2
    y, rstd = oracle.rmsnorm(x, gamma, dtype=oracle.F32, eps=0.0)
    g = gamma.astype(np.float64)
    np.testing.assert_allclose(y[0], g, rtol=2e-16)
    np.testing.assert_allclose(y[1], -g, rtol=2e-16)
    np.testing.assert_allclose(y[2], np.where(np.arange(d) % 2 == 0, g, -g), rtol=2e-16)
    np.testing.assert_allclose(rstd[:3], [1 / 3, 4 / 3, 0.5], rtol=1e-16)
    # a zero row stays zero; its rstd is 1 / sqrt(eps)
    y, rstd = oracle.rmsnorm(x, gamma, dtype=oracle.F32, eps=1e-6)
    assert np.all(y[3] == 0) and rstd[3] == pytest.approx(1000.0, rel=1e-15)


def test_rmsnorm_unit_mean_square_scale_invariance_and_torch():
    rng = np.random.default_rng(45)
    n, d = 7, 256
    x = _bf16_exact(rng, (n, d), 3.0)
    x[2] *= 128                 # a loud row (stays bf16-exact)
    ones = np.ones(d, np.float32)
    # eps = 0 and unit gain: every row has mean square 1; with eps the mean
    # square is ms / (ms + eps) for the row's own mean square ms
    y, _ = oracle.rmsnorm(x, ones, dtype=oracle.F32, eps=0.0)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-14)
    eps = 0.5
    y, _ = oracle.rmsnorm(x, ones, dtype=oracle.F32, eps=eps)
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    np.testing.assert_allclose((y ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-13)
    # scaling a row by a power of two changes nothing (eps = 0), to the bit
    gamma = _bf16_exact(rng, (d,), 1.0)
    y1, _ = oracle.rmsnorm(x, gamma, dtype=oracle.F32, eps=0.0)
    y4, _ = oracle.rmsnorm(x * 4, gamma, dtype=oracle.F32, eps=0.0)
    np.testing.assert_array_equal(y1, y4)
    # the library routine in float64
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (d,),
                                       weight=torch.from_numpy(gamma.astype(np.float64)),
                                       eps=1e-6).numpy()
    y, _ = oracle.rmsnorm(x, gamma, dtype=oracle.F32, eps=1e-6)
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-300)
    # bf16 inputs decode exactly: the bf16 path equals the fp32 path on the same values
    xb = oracle.bf16_round_rne(x)
    gb = oracle.bf16_round_rne(gamma)
    yb, _ = oracle.rmsnorm(xb, gb, dtype=oracle.BF16, eps=1e-6)
    np.testing.assert_array_equal(yb, y)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

MUTATIONS = [
    ("no max subtraction", "s += exp(zr[c] - m);", "s += exp(zr[c]);",
     "test_two_entry_vocabulary_closed_form_including_large_logits"),
    ("gather off by one", "ok ? zr[a] - l : NAN", "ok ? zr[(a + 1) % v] - l : NAN",
     "test_brute_force_against_exact_logits_and_decimal_softmax"),
    ("transposed W", "wd[k] = load_elem(j->w, j->dtype, c * j->ldw + k);",
     "wd[k] = load_elem(j->w, j->dtype, k * j->ldw + c);",
     "test_brute_force_against_exact_logits_and_decimal_softmax"),
    ("delta sign", "                delta = (double)lt[t] - (double)lr[t];",
     "                delta = (double)lr[t] - (double)lt[t];",
     "test_vexact_table1_sign_and_derived_estimators"),
    ("extras delta sign", "double delta = (double)lt[t] - (double)lr[t];",
     "double delta = (double)lr[t] - (double)lt[t];",
     "test_quantile_order_statistics_and_edge_cases"),
    ("k3 without -delta", "k3 = expm1(delta) - delta;", "k3 = expm1(delta);",
     "test_k3_nonnegative_and_matches_closed_form"),
    ("k3 without -1", "k3 = expm1(delta) - delta;", "k3 = exp(delta) - delta;",
     "test_zero_mismatch_gives_zero_estimators"),
    ("token mean for sequence mean", "bs_delta += m_delta;", "bs_delta += q_delta;",
     "test_sequence_mean_then_batch_mean_differs_from_token_mean"),
    ("clip at C instead of log C", "clipped = delta > log_c;", "clipped = delta > clip_c;",
     "test_truncated_is_clips_above_log_c"),
    ("K3 rejection on k2", "int reject_k3 = q_valid > 0 && m_k3 > seq_k3_hi;",
     "int reject_k3 = q_valid > 0 && m_k2 > seq_k3_hi;",
     "test_k3_rejection_uses_mean_k3_not_k2"),
    ("K3 rejection not strict", "int reject_k3 = q_valid > 0 && m_k3 > seq_k3_hi;",
     "int reject_k3 = q_valid > 0 && m_k3 >= seq_k3_hi;",
     "test_k3_rejection_uses_mean_k3_not_k2"),
    ("extreme without abs", "if (fabs(delta) > tok_tau) n_ext++;",
     "if (delta > tok_tau) n_ext++;", "test_extreme_rate_is_strict_and_two_sided"),
    ("extreme not strict", "if (fabs(delta) > tok_tau) n_ext++;",
     "if (fabs(delta) >= tok_tau) n_ext++;", "test_extreme_rate_is_strict_and_two_sided"),
    ("rel diff over rollout", "rel_sum += fabs(delta) / (fabs((double)lt[t]) + 1e-8);",
     "rel_sum += fabs(delta) / (fabs((double)lr[t]) + 1e-8);",
     "test_rel_diff_equals_mean_abs_delta_when_train_logp_is_minus_one"),
    ("rel diff guard 1e-6", "rel_sum += fabs(delta) / (fabs((double)lt[t]) + 1e-8);",
     "rel_sum += fabs(delta) / (fabs((double)lt[t]) + 1e-6);",
     "test_rel_diff_zero_train_logp_and_scale_invariance"),
    ("quantile without interpolation", "return x[lo] + (x[hi] - x[lo]) * frac;",
     "return x[lo];", "test_quantile_order_statistics_and_edge_cases"),
    ("quantile of unsorted values",
     "if (sort_doubles(ratio, m, nsort) != 0 || sort_doubles(absd, m, nsort) != 0) {",
     "if (sort_doubles(absd, m, nsort) != 0) {", "test_quantile_order_statistics_and_edge_cases"),
    ("pieces merged by the largest head",
     "if (pos[i] < end[i] && (best < 0 || x[pos[i]] < x[pos[best]])) best = i;",
     "if (pos[i] < end[i] && (best < 0 || x[pos[i]] > x[pos[best]])) best = i;",
     "test_quantiles_of_many_tokens_match_numpy"),
    ("pieces merged unsorted", "    qsort(j->a, j->n, sizeof(double), cmp_double);\n    return NULL;",
     "    (void)j;\n    return NULL;", "test_quantiles_of_many_tokens_match_numpy"),
    ("quantile position over m", "double pos = q * (double)(m - 1);",
     "double pos = q * (double)m;", "test_quantiles_match_numpy_linear_method"),
    ("softmax derivative sign", "dz[c] = g * ((c == a ? 1.0 : 0.0) - p);",
     "dz[c] = g * (p - (c == a ? 1.0 : 0.0));",
     "test_backward_matches_central_differences_of_the_forward"),
    ("upstream gradient dropped", "dz[c] = g * ((c == a ? 1.0 : 0.0) - p);",
     "dz[c] = ((c == a ? 1.0 : 0.0) - p);", "test_backward_invariants_and_row_selection"),
    ("dW from W instead of h", "o[k] += f * load_elem(j->h, j->dtype, t * j->ldh + k);",
     "o[k] += f * load_elem(j->w, j->dtype, t * j->ldw + k);",
     "test_backward_matches_central_differences_of_the_forward"),
    ("ppo max instead of min", "const double sur = fmin(r * a, rc * a);",
     "const double sur = fmax(r * a, rc * a);", "test_ppo_clip_branches_closed_form"),
    ("ppo clip side", "const int active = (a > 0.0 && r > 1.0 + eps_hi) || (a < 0.0 && r < 1.0 - eps_lo);",
     "const int active = (a > 0.0 && r < 1.0 - eps_lo) || (a < 0.0 && r > 1.0 + eps_hi);",
     "test_ppo_clip_branches_closed_form"),
    ("ppo bypass ignored", "const double old = bypass ? (double)old_rollout[t] : (double)old_train[t];",
     "const double old = (double)old_train[t];",
     "test_ppo_contribution_has_the_gradient_of_minus_r_a_and_tis_moves_the_ratio"),
    ("tis weight untruncated", "? fmin(exp((double)old_train[t] - (double)old_rollout[t]), tis_c) : 1.0;",
     "? exp((double)old_train[t] - (double)old_rollout[t]) : 1.0;",
     "test_ppo_contribution_has_the_gradient_of_minus_r_a_and_tis_moves_the_ratio"),
    ("ppo gradient without weight", "g_t = active ? 0.0 : -w * r * a;", "g_t = active ? 0.0 : -r * a;",
     "test_ppo_gradient_matches_central_differences"),
    ("ppo gradient scale ignored", "for (int64_t t = 0; t < n; ++t) grad[t] *= grad_scale;",
     "for (int64_t t = 0; t < n; ++t) grad[t] *= 1.0;",
     "test_ppo_scaled_gradient_is_that_of_the_scaled_token_sum"),
    ("temperature multiplies", "zr[c] = zr[c] / j->tau;", "zr[c] = zr[c] * j->tau;",
     "test_temperature_divides_the_logits"),
    ("entropy sign", "hsum += -exp(lp) * lp;", "hsum += exp(lp) * lp;",
     "test_entropy_closed_forms"),
    ("entropy unnormalised", "const double lp = zr[c] - l;", "const double lp = zr[c] - m;",
     "test_entropy_matches_scipy_on_exact_logits"),
    ("rms of the sum", "const double r = 1.0 / sqrt(ss / (double)d + eps);",
     "const double r = 1.0 / sqrt(ss + eps);", "test_rmsnorm_constant_rows_give_the_gain"),
    ("eps outside the root", "const double r = 1.0 / sqrt(ss / (double)d + eps);",
     "const double r = 1.0 / (sqrt(ss / (double)d) + eps);",
     "test_rmsnorm_unit_mean_square_scale_invariance_and_torch"),
    ("gain not applied", "y[t * d + k] = load_elem(gamma, dtype, k) * load_elem(x, dtype, t * ldx + k) * r;",
     "y[t * d + k] = load_elem(x, dtype, t * ldx + k) * r;",
     "test_rmsnorm_constant_rows_give_the_gain"),
]


@pytest.mark.parametrize("label,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, label, old, new, pin):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, label
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-pthread", "-o", str(so), str(mutated), "-lm"], check=True)
    good = oracle._load()
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "build", lambda force=True: str(so))
    # the transposed-W mutant reads W[k, c]; keep its reads in bounds
    fn = globals()[pin]
    with pytest.raises(AssertionError):
        fn()
    monkeypatch.setattr(oracle, "_lib", good)
