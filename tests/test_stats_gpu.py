"""GPU parity of tim_mismatch_stats against the fp64 oracle on identical
inputs: flags and counts bit-exact, aggregates within 1e-3 relative; plus
per-sequence invariance under batch recomposition and run-to-run determinism.
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
REL = 1e-3


def say(msg):
    print(f"[stats-gpu] {msg}", flush=True)
    sys.stdout.flush()


def run_both(lt, lr, mask, cu, c, lo, hi, token_outputs=True):
    res = tim.tim_mismatch_stats(lt, lr, mask, cu, tis_clip=c, seq_bounds=(lo, hi),
                                 token_outputs=token_outputs)
    torch.cuda.synchronize()
    ref = oracle.mismatch_stats(lt.cpu(), lr.cpu(), None if mask is None else mask.cpu(),
                                cu.cpu(), clip_c=c, seq_lo=lo, seq_hi=hi)
    return res, ref


def flag_margin(ref, lo, hi, cu):
    """Smallest distance of a non-empty sequence's mean delta to a bound, and
    the fp64 summation error bound it has to beat."""
    md = ref["seq"]["mean_delta"]
    nv = ref["seq"]["n_valid"]
    ok = nv > 0
    if not ok.any():
        return math.inf, 0.0
    margin = np.minimum(np.abs(md - lo), np.abs(md - hi))[ok].min()
    # |sum error| <= n * eps * sum|delta| (any summation order); divide by n
    lens = np.diff(cu.cpu().numpy())[ok]
    bound = (lens * 2.0 ** -52 * np.maximum(np.abs(md[ok]), 1.0)).max() * 4
    return margin, bound


def compare(res, ref, lo, hi, cu, label, token=True):
    s = res["seq"]
    r = ref["seq"]
    margin, bound = flag_margin(ref, lo, hi, cu)
    say(f"{label}: flag margin {margin:.3e} (fp64 order bound {bound:.1e})")
    assert margin > bound, "a sequence sits within rounding of a bound"
    for k in ("n_valid", "n_clipped", "n_nan", "reject"):
        np.testing.assert_array_equal(s[k].cpu().numpy(), r[k], err_msg=f"{label} seq {k}")
    for k in ("mean_delta", "mean_k1", "mean_k2", "mean_k3", "mean_tis_w"):
        np.testing.assert_allclose(s[k].cpu().numpy(), r[k], rtol=REL, atol=1e-12,
                                   err_msg=f"{label} seq {k}")
    got = tim.batch_dict(res["batch"])
    for k_ours, k_ref in zip(tim.BATCH_FIELDS, oracle.BATCH_FIELDS):
        a, b = got[k_ours], ref["batch"][k_ref]
        if k_ours.startswith("n_") or k_ours in ("is_clip_ratio", "is_nan_ratio", "reject_frac"):
            assert a == b, f"{label} batch {k_ours}: {a} vs {b}"      # counts: exact
        elif k_ours == "max_abs_delta":
            assert a == b, f"{label} batch {k_ours}: {a} vs {b}"      # a max of exact deltas
        else:
            assert abs(a - b) <= REL * abs(b) + 1e-12, f"{label} batch {k_ours}: {a} vs {b}"
    if token:
        t = res["token"]
        rt = ref["token"]
        np.testing.assert_array_equal(t["clipped"].cpu().numpy(), rt["clipped"])
        d = rt["delta"]
        for k in ("delta", "ratio", "k1", "k2", "k3", "tis_w"):
            g = t[k].cpu().double().numpy()
            e = rt[k]
            fin = np.isfinite(e)
            assert np.array_equal(np.isfinite(g), fin), f"{label} token {k} finiteness"
            # fp32 outputs: a few fp32 ulps; k3 also carries the oracle's own
            # cancellation error (e^d - 1) - d, a few fp64 ulps of |d|
            tol = 2e-6 * np.abs(e[fin]) + (2.0 ** -50 * np.abs(d[fin]) if k == "k3" else 0)
            err = np.abs(g[fin] - e[fin])
            assert np.all(err <= tol), f"{label} token {k}: worst {err.max()}"
    return got


@pytest.mark.parametrize("name", ["tiny", "small", "qwen3_8b", "dsv3"])
def test_workload_stats_parity(name):
    say(f"workload {name}")
    # the sampler's record plays the trainer side here: identical inputs to both
    w = workloads.make(name, device=DEV)
    sp = w.spec
    res, ref = run_both(w.logp_sampler, w.logp_rollout, w.mask, w.cu_seqlens,
                        sp.clip_c, sp.seq_lo, sp.seq_hi)
    got = compare(res, ref, sp.seq_lo, sp.seq_hi, w.cu_seqlens, name)
    say(f"{name}: is_approx_k3_kl {got['is_approx_k3_kl']:.3e}, "
        f"reject_frac {got['reject_frac']:.3f}, clip {got['is_clip_ratio']:.4f}")


def _stress(n, seed):
    lt, lr, mask, cu = workloads.stats_scale(n, seed=seed, device=DEV)
    # add empty sequences (index 2 and the last two) and an all-masked one (4)
    cu_h = cu.cpu().numpy().tolist()
    cu_h = cu_h[:3] + [cu_h[2]] + cu_h[3:] + [cu_h[-1], cu_h[-1]]
    cu2 = torch.tensor(cu_h, dtype=torch.int32, device=DEV)
    mask = mask.clone()
    mask[cu_h[4]:cu_h[5]] = 0
    return lt, lr, mask, cu2


def test_stress_input_parity():
    lt, lr, mask, cu = _stress(1 << 16, 21)
    lo, hi = math.log(0.99), math.log(1.01)
    say("stress 2^16")
    res, ref = run_both(lt, lr, mask, cu, 2.0, lo, hi)
    got = compare(res, ref, lo, hi, cu, "stress")
    assert got["n_nan"] > 0 and got["n_clipped"] > 0 and got["n_seq_rejected"] > 0
    nv = res["seq"]["n_valid"].cpu()
    assert nv[2].item() == 0            # the inserted empty sequence [c2, c2)
    assert nv[4].item() == 0            # the all-masked sequence


@pytest.mark.parametrize("with_mask", [True, False])
@pytest.mark.parametrize("token_outputs", [False, True])
def test_clip_bound_inside_the_series_range(with_mask, token_outputs):
    # C = 1.01: log C < 1/32, so the kernel tests the clip on every token
    # instead of leaving it to the rare branch (|delta| > 1/32); ~half the
    # tokens of this input are clipped
    lt, lr, mask, cu = _stress(1 << 16, 23)
    lo, hi = math.log(0.99), math.log(1.01)
    say(f"clip 1.01, mask {with_mask}, token outputs {token_outputs}")
    res, ref = run_both(lt, lr, mask if with_mask else None, cu, 1.01, lo, hi,
                        token_outputs=token_outputs)
    got = compare(res, ref, lo, hi, cu, "clip 1.01", token=token_outputs)
    assert got["n_clipped"] > 0


def test_large_stats_parity_without_token_outputs():
    n = 1 << 24
    lt, lr, mask, cu = workloads.stats_scale(n, seed=5, device=DEV)
    lo, hi = math.log(0.99), math.log(1.01)
    say("stats 2^24 tokens")
    res, ref = run_both(lt, lr, mask, cu, 2.0, lo, hi, token_outputs=False)
    compare(res, ref, lo, hi, cu, "stats 2^24", token=False)


def test_long_sequences_span_many_subchunks():
    # sequences far longer than a sub-chunk, ragged, plus one-token sequences
    lens = [1, 5000, 1, 1023, 1024, 1025, 77777, 2, 3000]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    n = int(cu[-1])
    g = torch.Generator(device=DEV).manual_seed(4)
    lt = -torch.rand(n, generator=g, device=DEV) * 5
    lr = lt + torch.randn(n, generator=g, device=DEV) * 0.01
    say("long sequences")
    res, ref = run_both(lt, lr, None, cu, 1.5, -0.002, 0.002)
    compare(res, ref, -0.002, 0.002, cu, "long sequences")


def test_zero_mismatch_exact():
    w = workloads.make("tiny", device=DEV)
    res = tim.tim_mismatch_stats(w.logp_sampler, w.logp_sampler, None, w.cu_seqlens,
                                 token_outputs=True)
    b = tim.batch_dict(res["batch"])
    assert b["tok_mean_delta"] == 0 and b["is_approx_k3_kl"] == 0 and b["tok_mean_k2"] == 0
    assert b["is_clip_ratio"] == 0 and b["reject_frac"] == 0 and b["tok_mean_tis_w"] == 1.0
    assert torch.all(res["token"]["ratio"] == 1) and torch.all(res["token"]["k3"] == 0)


def test_per_sequence_results_do_not_depend_on_the_batch():
    lt, lr, mask, cu = workloads.stats_scale(1 << 18, seed=8, device=DEV)
    lo, hi = -0.01, 0.01
    say("per-sequence invariance")
    full = tim.tim_mismatch_stats(lt, lr, mask, cu, seq_bounds=(lo, hi))
    cu_h = cu.cpu().numpy()
    # the sequences 10..40 scored alone, as a batch of their own
    a, b = int(cu_h[10]), int(cu_h[41])
    sub_cu = torch.tensor(cu_h[10:42] - a, dtype=torch.int32, device=DEV)
    part = tim.tim_mismatch_stats(lt[a:b].contiguous(), lr[a:b].contiguous(),
                                  mask[a:b].contiguous(), sub_cu, seq_bounds=(lo, hi))
    torch.cuda.synchronize()
    for k in ("mean_delta", "mean_k1", "mean_k2", "mean_k3", "mean_tis_w"):
        x = full["seq"][k][10:41].cpu().view(torch.int64)
        y = part["seq"][k].cpu().view(torch.int64)
        assert torch.equal(x, y), k


def test_stats_run_to_run_determinism():
    lt, lr, mask, cu = workloads.stats_scale(1 << 20, seed=9, device=DEV)
    outs = [tim.tim_mismatch_stats(lt, lr, mask, cu, token_outputs=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o["batch"].view(torch.int64), outs[0]["batch"].view(torch.int64))
        for k in ("mean_delta", "mean_k3"):
            assert torch.equal(o["seq"][k].view(torch.int64), outs[0]["seq"][k].view(torch.int64))


def test_end_to_end_small_against_oracle():
    """GPU logprob -> GPU stats versus oracle logprob -> oracle stats."""
    w = workloads.make("small", device=DEV)
    sp = w.spec
    say("end to end: small")
    lt = tim.tim_logprob_forward(w.h, w.w, w.ids)
    res = tim.tim_mismatch_stats(lt, w.logp_rollout, w.mask, w.cu_seqlens,
                                 tis_clip=sp.clip_c, seq_bounds=(sp.seq_lo, sp.seq_hi))
    torch.cuda.synchronize()
    lt_ref, _, _, _ = oracle.logprob(w.h.cpu(), w.w.cpu(), w.ids.cpu(), dtype=oracle.BF16)
    ref = oracle.mismatch_stats(lt_ref.astype(np.float32), w.logp_rollout.cpu(), w.mask.cpu(),
                                w.cu_seqlens.cpu(), clip_c=sp.clip_c, seq_lo=sp.seq_lo,
                                seq_hi=sp.seq_hi)
    got = tim.batch_dict(res["batch"])
    # logp differ by <= 2e-4 per token; k means move by at most that much
    for k_ours, k_ref in zip(tim.BATCH_FIELDS, oracle.BATCH_FIELDS):
        a, b = got[k_ours], ref["batch"][k_ref]
        if k_ours.startswith("n_") or k_ours in ("is_nan_ratio",):
            assert a == b, k_ours
        else:
            assert abs(a - b) <= 2e-4 + REL * abs(b), f"{k_ours}: {a} vs {b}"
    # a flag may differ only where the oracle's mean delta is within 2e-4 of a bound
    md = ref["seq"]["mean_delta"]
    close = np.minimum(np.abs(md - sp.seq_lo), np.abs(md - sp.seq_hi)) < 2e-4
    diff = res["seq"]["reject"].cpu().numpy() != ref["seq"]["reject"]
    assert not np.any(diff & ~close)


def _partition(name):
    """Sequence lengths that put sequence, sub-chunk (1024 tokens) and
    streaming-range (512 tokens at these sizes) boundaries in awkward places."""
    rng = np.random.default_rng(31)
    if name == "one_sequence":
        return [300001]
    if name == "all_one_token":
        return [1] * 5000
    if name == "empties_everywhere":
        lens = []
        for i in range(300):
            lens += [0] * int(rng.integers(0, 3)) + [int(rng.integers(1, 3000))]
        return [0, 0] + lens + [0, 0, 0]
    if name == "aligned":
        return [512] * 40 + [1024] * 20 + [2048] * 10 + [513, 511, 1023, 1025]
    if name == "all_empty":
        return [0] * 7
    raise KeyError(name)


@pytest.mark.parametrize("name", ["one_sequence", "all_one_token", "empties_everywhere",
                                  "aligned", "all_empty"])
def test_partition_edges_against_oracle(name):
    lens = _partition(name)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    n = int(cu[-1])
    g = torch.Generator(device=DEV).manual_seed(77)
    lt = -torch.rand(n, generator=g, device=DEV) * 5
    lr = lt + torch.randn(n, generator=g, device=DEV) * 0.004
    mask = (torch.rand(n, generator=g, device=DEV) > 0.1).to(torch.uint8)
    lo, hi = -0.0015, 0.0015
    say(f"partition {name}: n {n}, s {len(lens)}")
    res, ref = run_both(lt, lr, mask, cu, 1.5, lo, hi)
    compare(res, ref, lo, hi, cu, f"partition {name}")
    # each sequence alone gives the bits it has in the batch
    cu_h = cu.cpu().numpy()
    for j in [0, len(lens) // 2, len(lens) - 1]:
        a, b = int(cu_h[j]), int(cu_h[j + 1])
        one = tim.tim_mismatch_stats(lt[a:b].contiguous(), lr[a:b].contiguous(),
                                     mask[a:b].contiguous(),
                                     torch.tensor([0, b - a], dtype=torch.int32, device=DEV),
                                     tis_clip=1.5, seq_bounds=(lo, hi))
        torch.cuda.synchronize()
        for k in ("mean_delta", "mean_k3", "mean_tis_w", "n_valid"):
            x = res["seq"][k][j:j + 1].cpu()
            y = one["seq"][k].cpu()
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{name} seq {j} {k}"
