"""GPU parity of tim_logprob_backward and tim_ppo_loss against the fp64 oracle.

Backward tolerances follow from the arithmetic: dz is rounded to bf16 once
(relative error <= 2^-9 per element) and the fp32 logits carry ~1e-5 of
absolute error into the softmax, so |dh - dh_ref|[t, k] <= 2^-7 * 2 |g_t| *
max_v |W[v, k]| (sum_v |dz[t, v]| <= 2 |g_t|) and |dW - dW_ref|[v, k] <=
2^-7 * sum_t |dz[t, v]| |h[t, k]| + 1e-6 * max |g| max |h|, both with a 4x
margin over the rounding bound.  Invariance and determinism are bit-exact.
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


def say(msg):
    print(f"[backward-gpu] {msg}", flush=True)
    sys.stdout.flush()


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _case(n, d, v, seed, zero_frac=0.2):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn(n, d, generator=g).to(torch.bfloat16)
    w = (torch.randn(v, d, generator=g) * 0.05).to(torch.bfloat16)
    ids = torch.randint(0, v, (n,), generator=g, dtype=torch.int32)
    gr = torch.randn(n, generator=g, dtype=torch.float32)
    gr[torch.rand(n, generator=g) < zero_frac] = 0.0
    return h.to(DEV), w.to(DEV), ids.to(DEV), gr.to(DEV)


def _dz_abs(h, w, ids, gr, rows_v):
    """|dz[:, rows_v]| in fp64 from the oracle's lse (for the dW bound)."""
    hd = h.float().double().cpu().numpy()
    wd = w.float().double().cpu().numpy()[rows_v]
    _, lse, _, _ = oracle.logprob(h.cpu(), w.cpu(), ids.cpu(), dtype=oracle.BF16)
    z = hd @ wd.T
    p = np.exp(z - lse[:, None])
    onehot = (ids.cpu().numpy()[:, None] == np.asarray(rows_v)[None, :]).astype(np.float64)
    return np.abs(gr.double().cpu().numpy()[:, None] * (onehot - p))


def check_dh(dh, dh_ref, gr, w, rows, label):
    wmax = w.float().abs().amax(dim=0).double().cpu().numpy()          # max_v |W[v, k]|
    g = np.abs(gr.double().cpu().numpy()[rows])
    tol = 2.0 ** -7 * 2 * g[:, None] * wmax[None, :] + 1e-7
    err = np.abs(dh - dh_ref)
    say(f"{label}: dh worst err {err.max():.3e}, worst err/tol {(err / tol).max():.3f}")
    assert np.all(err <= tol), f"{label}: dh"


def check_dw(dw, dw_ref, dzabs, h, gr, label):
    ha = h.float().abs().double().cpu().numpy()
    tol = 2.0 ** -7 * (dzabs.T @ ha) + 1e-6 * float(gr.abs().max()) * float(ha.max())
    err = np.abs(dw - dw_ref)
    say(f"{label}: dW worst err {err.max():.3e}, worst err/tol {(err / tol).max():.3f}")
    assert np.all(err <= tol), f"{label}: dW"


def test_backward_parity_ragged_sizes():
    # N, V not multiples of 64 or 256; one id out of range (contributes nothing)
    n, d, v = 300, 256, 2000
    h, w, ids, gr = _case(n, d, v, seed=1)
    ids[17] = v + 5
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    torch.cuda.synchronize()
    dh_ref, dw_ref = oracle.logprob_backward(bf16_bits(h), bf16_bits(w), ids.cpu(), gr.cpu(),
                                             dtype=oracle.BF16)
    check_dh(dh.double().cpu().numpy(), dh_ref, gr, w, np.arange(n), "ragged")
    gr_eff = gr.clone()
    gr_eff[17] = 0.0                                  # the out-of-range id's row
    ids_c = ids.clone()
    ids_c[17] = 0
    dzabs = _dz_abs(h, w, ids_c, gr_eff, np.arange(v))
    check_dw(dw.double().cpu().numpy(), dw_ref, dzabs, h, gr_eff, "ragged")
    assert torch.all(dh[17] == 0)


@pytest.mark.parametrize("n,d,v", [(1, 64, 5), (3, 64, 257), (65, 128, 64), (256, 64, 1)])
def test_backward_parity_edge_sizes(n, d, v):
    # one token, a vocabulary smaller than one MFMA block, one K stage
    # (D = 64), N just past a 64-token stage, V = 1 (p = 1: dz = 0)
    h, w, ids, gr = _case(n, d, v, seed=n + v, zero_frac=0.0)
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    torch.cuda.synchronize()
    dh_ref, dw_ref = oracle.logprob_backward(bf16_bits(h), bf16_bits(w), ids.cpu(), gr.cpu(),
                                             dtype=oracle.BF16)
    check_dh(dh.double().cpu().numpy(), dh_ref, gr, w, np.arange(n), f"n={n} d={d} v={v}")
    dzabs = _dz_abs(h, w, ids, gr, np.arange(v))
    check_dw(dw.double().cpu().numpy(), dw_ref, dzabs, h, gr, f"n={n} d={d} v={v}")
    if v == 1:
        assert torch.all(dh == 0) and torch.all(dw == 0)


def test_backward_zero_gradient_gives_zeros():
    n, d, v = 100, 128, 700
    h, w, ids, _ = _case(n, d, v, seed=8)
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dw = torch.full((v, d), 7.0, device=DEV)
    dh, _ = tim.tim_logprob_backward(h, w, ids, lse, torch.zeros(n, device=DEV), dw=dw)
    torch.cuda.synchronize()
    assert torch.all(dh == 0) and torch.all(dw == 0)


def test_backward_full_size_sparse_gradient():
    # the Qwen3-8B-shaped head at its full size, with an upstream gradient on
    # 16 tokens so that the oracle computes only those rows
    w8 = workloads.make("qwen3_8b", device=DEV)
    h, w, ids = w8.h, w8.w, w8.ids
    n, v = h.shape[0], w.shape[0]
    rng = np.random.default_rng(5)
    tok = np.sort(rng.choice(n, 16, replace=False))
    gr = torch.zeros(n, dtype=torch.float32, device=DEV)
    gr[torch.as_tensor(tok, device=DEV)] = torch.as_tensor(rng.normal(0, 1, 16), dtype=torch.float32,
                                                          device=DEV)
    say("full size: forward + backward")
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    torch.cuda.synchronize()
    rows_v = np.unique(np.concatenate([ids.cpu().numpy()[tok], rng.choice(v, 16, replace=False),
                                       [v - 1]]))
    zero_tok = np.setdiff1d(np.arange(n), tok)[:4]
    dh_rows = np.concatenate([tok, zero_tok])
    say("full size: oracle rows")
    dh_ref, dw_ref = oracle.logprob_backward(bf16_bits(h), bf16_bits(w), ids.cpu(), gr.cpu(),
                                             dtype=oracle.BF16, dh_rows=dh_rows, dw_rows=rows_v)
    check_dh(dh[torch.as_tensor(dh_rows, device=DEV)].double().cpu().numpy(), dh_ref, gr, w,
             dh_rows, "full size")
    hs = h[torch.as_tensor(tok, device=DEV)]
    dzabs = _dz_abs(hs, w, ids[torch.as_tensor(tok, device=DEV)], gr[torch.as_tensor(tok, device=DEV)],
                    rows_v)
    check_dw(dw[torch.as_tensor(rows_v, device=DEV)].double().cpu().numpy(), dw_ref, dzabs, hs,
             gr[torch.as_tensor(tok, device=DEV)], "full size")


def test_dh_rows_do_not_depend_on_the_batch_and_runs_repeat():
    n, d, v = 512, 256, 3000
    h, w, ids, gr = _case(n, d, v, seed=2)
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    dh2, dw2 = tim.tim_logprob_backward(h, w, ids, lse, gr)
    a, b = 64, 197
    _, lse_s, _ = tim.tim_logprob_forward(h[a:b].contiguous(), w, ids[a:b].contiguous(),
                                          return_lse=True)
    dh_s, _ = tim.tim_logprob_backward(h[a:b].contiguous(), w, ids[a:b].contiguous(), lse_s,
                                       gr[a:b].contiguous(), want_dw=False)
    torch.cuda.synchronize()
    assert torch.equal(lse_s.view(torch.int32), lse[a:b].view(torch.int32))
    assert torch.equal(dh_s.view(torch.int32), dh[a:b].view(torch.int32))
    assert torch.equal(dh.view(torch.int32), dh2.view(torch.int32))
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))


def test_dw_accumulated_over_micro_batches_is_bitwise_one_batch():
    n, d, v = 640, 256, 1500
    h, w, ids, gr = _case(n, d, v, seed=3)
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    _, dw_full = tim.tim_logprob_backward(h, w, ids, lse, gr, want_dh=False)
    dw = torch.zeros(v, d, dtype=torch.float32, device=DEV)
    for a, b in ((0, 256), (256, 448), (448, 640)):     # multiples of 64 tokens
        tim.tim_logprob_backward(h[a:b].contiguous(), w, ids[a:b].contiguous(),
                                 lse[a:b].contiguous(), gr[a:b].contiguous(), want_dh=False,
                                 dw=dw, accumulate_dw=True)
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw_full.view(torch.int32))
    # an output that is not 16-byte aligned is refused, and left untouched
    buf = torch.zeros(v * d + 1, dtype=torch.float32, device=DEV)
    dw_u = buf[1:].view(v, d)
    with pytest.raises(tim.TimError):
        tim.tim_logprob_backward(h, w, ids, lse, gr, want_dh=False, dw=dw_u)
    torch.cuda.synchronize()
    assert torch.all(buf == 0)


# ---------------------------------------------------------------------------
# surrogate
# ---------------------------------------------------------------------------

def _ppo_inputs(n, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    ot = -torch.rand(n, generator=g) * 4
    orr = ot + torch.randn(n, generator=g) * 0.05
    lp = ot + torch.randn(n, generator=g) * 0.3
    adv = torch.randn(n, generator=g)
    mask = (torch.rand(n, generator=g) < 0.85).to(torch.uint8)
    lp[5] = float("nan")
    mask[5] = 1
    return [x.to(DEV) for x in (lp, ot, orr, adv, mask)]


@pytest.mark.parametrize("n", [1, 1000, 100_003])
@pytest.mark.parametrize("mode", ["recompute", "recompute+tis", "bypass"])
def test_ppo_parity(n, mode):
    lp, ot, orr, adv, mask = _ppo_inputs(max(n, 6), seed=n)
    lp, ot, orr, adv, mask = (x[:n].contiguous() for x in (lp, ot, orr, adv, mask))
    kw = dict(eps_low=0.2, eps_high=0.28, bypass=mode == "bypass",
              tis_c=2.0 if mode == "recompute+tis" else 0.0)
    res = tim.tim_ppo_loss(lp, ot, orr, adv, mask, **kw)
    torch.cuda.synchronize()
    ref = oracle.ppo_loss(lp.cpu(), ot.cpu(), orr.cpu(), adv.cpu(), mask.cpu(),
                          eps_lo=kw["eps_low"], eps_hi=kw["eps_high"], bypass=kw["bypass"],
                          tis_c=kw["tis_c"])
    t = res["token"]
    np.testing.assert_array_equal(t["clipped"].cpu().numpy(), ref["clipped"])
    for k in ("loss", "grad", "ratio", "contrib"):
        np.testing.assert_allclose(t[k].double().cpu().numpy(), ref[k], rtol=1e-6, atol=1e-30,
                                   err_msg=f"{mode} {k}")
    got = dict(zip(tim.PPO_FIELDS, res["batch"].cpu().tolist()))
    for k in tim.PPO_FIELDS:
        if k.startswith("n_") or k == "clip_frac":
            assert got[k] == ref["batch"][k], k
        else:
            m = max(got["n_valid"], 1)
            assert got[k] == pytest.approx(ref["batch"][k], rel=2 * m * 2.0 ** -53 + 1e-15,
                                           abs=1e-300), k
    say(f"ppo {mode} n={n}: loss {got['mean_loss']:.4e}, clip {got['clip_frac']:.3f}")


@pytest.mark.parametrize("n", [1, 1003, 100_003])
def test_ppo_scaled_gradient_one_pass(n):
    lp, ot, orr, adv, mask = _ppo_inputs(max(n, 6), seed=n + 7)
    lp, ot, orr, adv, mask = (x[:n].contiguous() for x in (lp, ot, orr, adv, mask))
    scale = 1.0 / 3000.0
    kw = dict(eps_low=0.2, eps_high=0.28, tis_c=2.0)
    res = tim.tim_ppo_loss(lp, ot, orr, adv, mask, grad_scale=scale, **kw)
    mean = tim.tim_ppo_loss(lp, ot, orr, adv, mask, **kw)
    torch.cuda.synchronize()
    ref = oracle.ppo_loss(lp.cpu(), ot.cpu(), orr.cpu(), adv.cpu(), mask.cpu(), eps_lo=0.2,
                          eps_hi=0.28, tis_c=2.0, grad_scale=scale)
    np.testing.assert_allclose(res["token"]["grad"].double().cpu().numpy(), ref["grad"],
                               rtol=1e-6, atol=1e-30)
    # everything else has the bits of the mean-gradient call
    for k in ("loss", "ratio", "contrib", "clipped"):
        assert torch.equal(res["token"][k], mean["token"][k]), k
    assert torch.equal(res["batch"], mean["batch"])


def test_ppo_unaligned_inputs_give_the_aligned_bits():
    # a view one element in takes the element-wise variant; the same values in
    # fresh (16-byte aligned) storage take the 16-byte one: same assignment
    # of tokens to threads, same bits
    n = 50_001
    lp, ot, orr, adv, mask = _ppo_inputs(n + 1, seed=11)
    views = [x[1:] for x in (lp, ot, orr, adv, mask)]
    assert views[0].data_ptr() % 16 != 0
    fresh = [x.clone() for x in views]
    assert fresh[0].data_ptr() % 16 == 0
    for scale in (0.0, 1e-4):
        a = tim.tim_ppo_loss(*views, eps_low=0.2, eps_high=0.28, tis_c=2.0, grad_scale=scale)
        b = tim.tim_ppo_loss(*fresh, eps_low=0.2, eps_high=0.28, tis_c=2.0, grad_scale=scale)
        for k in ("loss", "grad", "ratio", "contrib", "clipped"):
            assert torch.equal(a["token"][k], b["token"][k]), (scale, k)
        assert torch.equal(a["batch"], b["batch"])


# ---------------------------------------------------------------------------
# fp32 head ("Train-Inference Consistency", section 3: the output layer's
# weights and compute stay in FP32).  dz is not rounded; the error comes
# from fp32 arithmetic alone.  With u = 2^-24, S_t = max_v sum_k |h_tk w_vk|:
# the logits and lse carry at most D u S_t each, so p_tv is off by at most
# p_tv (2 D u S_t + 5 u) (the exponential's own few ulps included), and the
# fp32 chains over V (dh) or N (dW) add at most V u or N u of the sum of
# their absolute terms.  The bounds below take M_tv = |g_t| (p_tv + [v = a_t])
# >= |dz_tv| for those sums, with a 4x margin.
# ---------------------------------------------------------------------------

U32 = 2.0 ** -24


def _case32(n, d, v, seed, zero_frac=0.2):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn(n, d, generator=g)
    w = torch.randn(v, d, generator=g) * 0.05
    ids = torch.randint(0, v, (n,), generator=g, dtype=torch.int32)
    gr = torch.randn(n, generator=g, dtype=torch.float32)
    gr[torch.rand(n, generator=g) < zero_frac] = 0.0
    return h.to(DEV), w.to(DEV), ids.to(DEV), gr.to(DEV)


def _bounds32(h, w, ids, gr, rows_t, rows_v):
    """(per-token relative error of p, M[rows_t, rows_v]) in fp64."""
    hd = h.double().cpu().numpy()[rows_t]
    wd = w.double().cpu().numpy()
    _, lse, _, _ = oracle.logprob(h.cpu()[rows_t], w.cpu(), ids.cpu()[rows_t], dtype=oracle.F32)
    s = (np.abs(hd) @ np.abs(wd).T).max(axis=1)                       # S_t
    rel = U32 * (2 * hd.shape[1] * s + 5)
    z = hd @ wd[rows_v].T
    p = np.exp(z - lse[:, None])
    onehot = (ids.cpu().numpy()[rows_t][:, None] == np.asarray(rows_v)[None, :])
    m = np.abs(gr.double().cpu().numpy()[rows_t])[:, None] * (p + onehot)
    return rel, m


def check_dh32(dh, dh_ref, h, w, ids, gr, rows, label):
    v = w.shape[0]
    rel, m = _bounds32(h, w, ids, gr, rows, np.arange(v))
    wa = w.abs().double().cpu().numpy()
    tol = 4 * ((m * rel[:, None]) @ wa + v * U32 * (m @ wa)) + 1e-12
    err = np.abs(dh - dh_ref)
    say(f"{label}: dh worst err {err.max():.3e}, worst err/tol {(err / tol).max():.3f}")
    assert np.all(err <= tol), f"{label}: dh"


def check_dw32(dw, dw_ref, h, w, ids, gr, rows_t, rows_v, label):
    rel, m = _bounds32(h, w, ids, gr, rows_t, rows_v)
    ha = h.abs().double().cpu().numpy()[rows_t]
    n = h.shape[0]
    tol = 4 * ((m * rel[:, None]).T @ ha + n * U32 * (m.T @ ha)) + 1e-12
    err = np.abs(dw - dw_ref)
    say(f"{label}: dW worst err {err.max():.3e}, worst err/tol {(err / tol).max():.3f}")
    assert np.all(err <= tol), f"{label}: dW"


@pytest.mark.parametrize("n,d,v", [(300, 256, 2000), (1, 64, 5), (3, 64, 257), (65, 128, 64),
                                   (256, 64, 1)])
def test_fp32_backward_parity(n, d, v):
    h, w, ids, gr = _case32(n, d, v, seed=n * 7 + v)
    if n > 20:
        ids[17] = v + 5                              # out of range: contributes nothing
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    torch.cuda.synchronize()
    dh_ref, dw_ref = oracle.logprob_backward(h.cpu(), w.cpu(), ids.cpu(), gr.cpu(),
                                             dtype=oracle.F32)
    gr_eff, ids_c = gr.clone(), ids.clone()
    if n > 20:
        gr_eff[17], ids_c[17] = 0.0, 0
        assert torch.all(dh[17] == 0)
    label = f"fp32 n={n} d={d} v={v}"
    check_dh32(dh.double().cpu().numpy(), dh_ref, h, w, ids_c, gr_eff, np.arange(n), label)
    check_dw32(dw.double().cpu().numpy(), dw_ref, h, w, ids_c, gr_eff, np.arange(n),
               np.arange(v), label)
    if v == 1:
        assert torch.all(dh == 0) and torch.all(dw == 0)


def test_fp32_backward_invariance_repeat_and_accumulation():
    n, d, v = 640, 256, 1500
    h, w, ids, gr = _case32(n, d, v, seed=4)
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    dh2, dw2 = tim.tim_logprob_backward(h, w, ids, lse, gr)
    a, b = 64, 197
    dh_s, _ = tim.tim_logprob_backward(h[a:b].contiguous(), w, ids[a:b].contiguous(),
                                       lse[a:b].contiguous(), gr[a:b].contiguous(), want_dw=False)
    acc = torch.zeros(v, d, dtype=torch.float32, device=DEV)
    for a2, b2 in ((0, 256), (256, 448), (448, 640)):     # multiples of 64 tokens
        tim.tim_logprob_backward(h[a2:b2].contiguous(), w, ids[a2:b2].contiguous(),
                                 lse[a2:b2].contiguous(), gr[a2:b2].contiguous(), want_dh=False,
                                 dw=acc, accumulate_dw=True)
    torch.cuda.synchronize()
    assert torch.equal(dh.view(torch.int32), dh2.view(torch.int32))
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))
    assert torch.equal(dh_s.view(torch.int32), dh[a:b].view(torch.int32))
    assert torch.equal(acc.view(torch.int32), dw.view(torch.int32))


def test_fp32_backward_full_size_sparse_gradient():
    # the FP32 head at its full size (N = 4096, D = 4096, V = 151936), an
    # upstream gradient on 8 tokens so that the oracle computes only those
    wl = workloads.make("fp32_head", device=DEV)
    h, w, ids = wl.h, wl.w, wl.ids
    n, v = h.shape[0], w.shape[0]
    rng = np.random.default_rng(6)
    tok = np.sort(rng.choice(n, 8, replace=False))
    gr = torch.zeros(n, dtype=torch.float32, device=DEV)
    gr[torch.as_tensor(tok, device=DEV)] = torch.as_tensor(rng.normal(0, 1, 8), dtype=torch.float32,
                                                          device=DEV)
    say("fp32 full size: forward + backward")
    _, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    dh, dw = tim.tim_logprob_backward(h, w, ids, lse, gr)
    torch.cuda.synchronize()
    rows_v = np.unique(np.concatenate([ids.cpu().numpy()[tok], rng.choice(v, 8, replace=False),
                                       [v - 1]]))
    dh_rows = np.concatenate([tok, np.setdiff1d(np.arange(n), tok)[:3]])
    say("fp32 full size: oracle rows")
    dh_ref, dw_ref = oracle.logprob_backward(h.cpu(), w.cpu(), ids.cpu(), gr.cpu(),
                                             dtype=oracle.F32, dh_rows=dh_rows, dw_rows=rows_v)
    tt = torch.as_tensor(tok, device=DEV)
    check_dh32(dh[torch.as_tensor(dh_rows, device=DEV)].double().cpu().numpy(), dh_ref, h, w, ids,
               gr, dh_rows, "fp32 full size")
    # dW rows see only the 8 tokens with a gradient
    check_dw32(dw[torch.as_tensor(rows_v, device=DEV)].double().cpu().numpy(), dw_ref, h[tt], w,
               ids[tt], gr[tt], np.arange(len(tok)), rows_v, "fp32 full size")
