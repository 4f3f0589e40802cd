"""GPU parity, batch invariance and determinism of tim_logprob_forward.

Every value here comes from the HIP library through its C ABI and is compared
with the fp64 oracle on the same seeded inputs (|delta logp| <= 2e-4), or with
itself across batch splits and repeats (bit-exact).
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

TOL_LOGP = 2e-4
DEV = "cuda"


def say(msg):
    print(f"[logprob-gpu] {msg}", flush=True)
    sys.stdout.flush()


_cache = {}


def wl(name):
    if name not in _cache:
        say(f"generating workload {name}")
        _cache[name] = workloads.make(name, device=DEV)
        torch.cuda.synchronize()
    return _cache[name]


_host = {}


def host(name, key):
    k = (name, key)
    if k not in _host:
        _host[k] = getattr(wl(name), key).cpu()
    return _host[k]


def odtype(t):
    return oracle.BF16 if t.dtype == torch.bfloat16 else oracle.F32


def check_rows(h, w, ids, logp_gpu, rows, label, h_host=None, w_host=None, lse_gpu=None):
    rows = np.asarray(sorted(set(int(r) for r in rows)), np.int64)
    hh = h.cpu() if h_host is None else h_host
    ww = w.cpu() if w_host is None else w_host
    ref, ref_lse, _, used = oracle.logprob(hh, ww, ids.cpu(), dtype=odtype(h), rows=rows)
    got = logp_gpu.cpu().double().numpy()[rows]
    err = np.abs(got - ref)
    say(f"{label}: {rows.size} rows, oracle threads {used}, max|dlogp| {err.max():.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= TOL_LOGP, f"{label}: max |dlogp| {err.max()} at row {rows[err.argmax()]}"
    if lse_gpu is not None:
        el = np.abs(lse_gpu.cpu().double().numpy()[rows] - ref_lse)
        assert el.max() <= TOL_LOGP
    return err.max()


def spread_rows(n, k, seed, extra=()):
    rng = np.random.default_rng(seed)
    base = {0, n - 1, min(n - 1, 255), min(n - 1, 256)}
    base.update(int(x) for x in extra)
    base.update(int(x) for x in rng.integers(0, n, k))
    return sorted(r for r in base if 0 <= r < n)


# ---------------------------------------------------------------------------
# parity against the oracle
# ---------------------------------------------------------------------------

def test_tiny_fp32_all_rows():
    w = wl("tiny")
    say("tiny fp32 forward")
    logp, lse, nbad = tim.tim_logprob_forward(w.h, w.w, w.ids, return_lse=True)
    torch.cuda.synchronize()
    check_rows(w.h, w.w, w.ids, logp, range(w.n), "tiny fp32", lse_gpu=lse)
    assert int(nbad.item()) == 0


def test_tiny_bf16_all_rows():
    w = wl("tiny")
    h, ww = w.h.to(torch.bfloat16), w.w.to(torch.bfloat16)
    say("tiny bf16 forward")
    logp = tim.tim_logprob_forward(h, ww, w.ids)
    torch.cuda.synchronize()
    check_rows(h, ww, w.ids, logp, range(w.n), "tiny bf16")


def test_small_bf16_rows_across_all_tiles():
    w = wl("small")
    say("small bf16 forward")
    logp = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    rows = spread_rows(w.n, 160, 1, extra=range(0, w.n, 97))
    check_rows(w.h, w.w, w.ids, logp, rows, "small bf16",
               h_host=host("small", "h"), w_host=host("small", "w"))


@pytest.mark.parametrize("n,d,v,dtype", [
    (300, 128, 1000, torch.bfloat16),     # ragged N and V, last chunk partial
    (257, 64, 700, torch.float32),        # one row past a token tile; 1-tile last chunk
    (1, 192, 257, torch.bfloat16),        # a single row; V one past a tile
    (5, 64, 1, torch.float32),            # V = 1: logp = 0
    (513, 256, 2, torch.bfloat16),        # V = 2
])
def test_ragged_shapes(n, d, v, dtype):
    g = torch.Generator(device="cpu").manual_seed(n * 7 + v)
    h = torch.randn(n, d, generator=g).to(dtype).to(DEV)
    w = (torch.randn(v, d, generator=g) * 0.1).to(dtype).to(DEV)
    ids = torch.randint(0, v, (n,), generator=g, dtype=torch.int32).to(DEV)
    say(f"ragged n={n} d={d} v={v} {dtype}")
    logp = tim.tim_logprob_forward(h, w, ids)
    torch.cuda.synchronize()
    check_rows(h, w, ids, logp, range(n), f"ragged {n}x{d}x{v}")
    if v == 1:
        assert torch.all(logp == 0)


def test_qwen3_8b_shape_sampled_rows():
    w = wl("qwen3_8b")
    say("qwen3_8b forward")
    logp = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    rows = spread_rows(w.n, 20, 2, extra=[511, 512, 4095, 4096, 8191])
    check_rows(w.h, w.w, w.ids, logp, rows, "qwen3_8b",
               h_host=host("qwen3_8b", "h"), w_host=host("qwen3_8b", "w"))


def test_dsv3_shape_sampled_rows():
    w = wl("dsv3")
    say("dsv3 forward")
    logp = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    cu = w.cu_seqlens.cpu().numpy()
    ends = [cu[j] for j in range(0, 64, 8)] + [cu[j + 1] - 1 for j in range(3, 64, 8)]
    rows = spread_rows(w.n, 6, 3, extra=ends)
    check_rows(w.h, w.w, w.ids, logp, rows, "dsv3",
               h_host=host("dsv3", "h"), w_host=host("dsv3", "w"))
    assert torch.all(torch.isfinite(logp))


def test_fp32_head_sampled_rows_and_bf16_rerun():
    w = wl("fp32_head")
    say("fp32_head forward (fp32 MFMA)")
    logp32 = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    rows = spread_rows(w.n, 12, 4, extra=[4095])
    check_rows(w.h, w.w, w.ids, logp32, rows, "fp32_head",
               h_host=host("fp32_head", "h"), w_host=host("fp32_head", "w"))
    say("fp32_head rows rounded to bf16")
    hb, wb = w.h.to(torch.bfloat16), w.w.to(torch.bfloat16)
    logp16 = tim.tim_logprob_forward(hb, wb, w.ids)
    torch.cuda.synchronize()
    dd = (logp16.double() - logp32.double()).abs().cpu().numpy()
    say(f"|logp_bf16 - logp_fp32|: mean {dd.mean():.3e} p99 {np.quantile(dd, 0.99):.3e} "
        f"max {dd.max():.3e}")
    # bf16 rounding of inputs moves logits by O(sqrt(D) * 2^-9 * |h||w|) ~ 1e-2
    assert dd.max() < 0.1 and dd.mean() > 0


# ---------------------------------------------------------------------------
# closed forms on the GPU path
# ---------------------------------------------------------------------------

def test_equal_logits_and_bad_ids():
    n, d, v = 70, 128, 151936
    h = torch.randn(n, d, device=DEV).to(torch.bfloat16)
    w = torch.zeros(v, d, device=DEV, dtype=torch.bfloat16)
    ids = torch.randint(0, v, (n,), device=DEV, dtype=torch.int32)
    ids[3] = -100
    ids[10] = v
    say("equal logits")
    logp, lse, nbad = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    torch.cuda.synchronize()
    good = torch.ones(n, dtype=torch.bool)
    good[[3, 10]] = False
    lp = logp.cpu()
    assert torch.isnan(lp[3]) and torch.isnan(lp[10]) and int(nbad.item()) == 2
    assert torch.all((lp[good].double() + math.log(v)).abs() < 2e-5)
    assert torch.all(torch.isfinite(lse))


def test_integer_exact_logits():
    """Inputs that are multiples of 1/8 with |z| < 2^10: the fp32 accumulation
    is exact, so only the exp/log evaluation separates GPU and oracle."""
    g = torch.Generator().manual_seed(5)
    n, d, v = 96, 256, 3000
    h = (torch.randint(-4, 5, (n, d), generator=g).float() / 8).to(torch.bfloat16).to(DEV)
    w = (torch.randint(-4, 5, (v, d), generator=g).float() / 8).to(torch.bfloat16).to(DEV)
    ids = torch.randint(0, v, (n,), generator=g, dtype=torch.int32).to(DEV)
    say("integer-exact logits")
    logp, lse, _ = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse, zsel, _ = oracle.logprob(h.cpu(), w.cpu(), ids.cpu(), dtype=oracle.BF16)
    assert np.all(zsel == np.round(zsel * 64) / 64)          # exact rationals
    got_z = (logp.double() + lse.double()).cpu().numpy()
    assert np.abs(got_z - zsel).max() <= 1e-4 * np.abs(zsel).max() + 1e-4
    assert np.abs(logp.cpu().double().numpy() - ref).max() <= 2e-5


def test_completeness_over_all_ids_and_identical_lse():
    w = wl("tiny")
    row = 5
    v = w.spec.v
    h = w.h[row:row + 1].expand(v, -1).contiguous()
    ids = torch.arange(v, dtype=torch.int32, device=DEV)
    say("one row replicated over every id")
    logp, lse, _ = tim.tim_logprob_forward(h, w.w, ids, return_lse=True)
    torch.cuda.synchronize()
    assert torch.unique(lse.cpu().view(torch.int32)).numel() == 1     # identical bits
    total = torch.exp(logp.double()).sum().item()
    assert abs(total - 1.0) < 1e-5, total


# ---------------------------------------------------------------------------
# batch invariance and determinism (bit-exact)
# ---------------------------------------------------------------------------

def _sliced(h, w, ids, slices):
    out = torch.empty(h.shape[0], dtype=torch.float32, device=DEV)
    for s, e in slices:
        out[s:e] = tim.tim_logprob_forward(h[s:e], w, ids[s:e])
    torch.cuda.synchronize()
    return out


def test_qwen3_8b_batch_invariance_sweep():
    w = wl("qwen3_8b")
    say("qwen3_8b full batch (reference bits)")
    full = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    full_bits = full.view(torch.int32).cpu()
    for b in (1, 7, 64, 1000, 8192):
        say(f"qwen3_8b sliced in batches of {b}")
        got = _sliced(w.h, w.w, w.ids, workloads.sweep_slices(w.n, b))
        diff = int((got.view(torch.int32).cpu() != full_bits).sum())
        assert diff == 0, f"batch {b}: {diff} rows differ"
    say("qwen3_8b random partition")
    got = _sliced(w.h, w.w, w.ids, workloads.random_slices(w.n, 17))
    assert torch.equal(got.view(torch.int32).cpu(), full_bits)


def test_same_row_in_different_tile_slots_and_shuffled_order():
    w = wl("small")
    n = w.n
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).to(DEV)
    say("small: shuffled rows")
    a = tim.tim_logprob_forward(w.h, w.w, w.ids)
    b = tim.tim_logprob_forward(w.h[perm].contiguous(), w.w, w.ids[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a[perm].view(torch.int32), b.view(torch.int32))
    # one row replicated 300 times (two token tiles, ragged) with varying ids
    rep = w.h[7:8].expand(300, -1).contiguous()
    ids = torch.randint(0, w.spec.v, (300,), device=DEV, dtype=torch.int32)
    ids[0] = w.ids[7]
    logp, lse, _ = tim.tim_logprob_forward(rep, w.w, ids, return_lse=True)
    torch.cuda.synchronize()
    assert torch.unique(lse.view(torch.int32).cpu()).numel() == 1
    assert logp[0].view(torch.int32).item() == a[7].view(torch.int32).item()


def test_fp32_batch_invariance_and_strided_rows():
    w = wl("tiny")
    full = tim.tim_logprob_forward(w.h, w.w, w.ids)
    for b in (1, 3, 64):
        say(f"tiny fp32 batches of {b}")
        got = _sliced(w.h, w.w, w.ids, workloads.sweep_slices(w.n, b))
        assert torch.equal(got.view(torch.int32), full.view(torch.int32))
    # leading dimension > D: a column slice of a wider matrix
    wide = torch.zeros(w.n, w.spec.d + 64, device=DEV)
    wide[:, 32:32 + w.spec.d] = w.h
    say("tiny fp32 with ldh > d")
    strided = tim.tim_logprob_forward(wide[:, 32:32 + w.spec.d], w.w, w.ids)
    torch.cuda.synchronize()
    assert torch.equal(strided.view(torch.int32), full.view(torch.int32))


def test_run_to_run_determinism():
    for name in ("small", "qwen3_8b"):
        w = wl(name)
        say(f"{name}: three repeats")
        outs = [tim.tim_logprob_forward(w.h, w.w, w.ids) for _ in range(3)]
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_free_schedule_matches_oracle_and_is_deterministic():
    w = wl("small")
    say("small: free schedule")
    a = tim.tim_logprob_forward(w.h, w.w, w.ids, schedule="free")
    b = tim.tim_logprob_forward(w.h, w.w, w.ids, schedule="free")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    check_rows(w.h, w.w, w.ids, a, spread_rows(w.n, 40, 9), "small free schedule",
               h_host=host("small", "h"), w_host=host("small", "w"))


def test_empty_batch():
    w = wl("tiny")
    out = tim.tim_logprob_forward(w.h[:0], w.w, w.ids[:0])
    assert out.numel() == 0
