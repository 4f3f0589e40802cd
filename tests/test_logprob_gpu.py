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


def tile_slot_rows(n, k, seed):
    """About k rows of [0, n): every slot of the 256-token tile once (in a
    seeded random tile), the first and last row of every tile, then seeded
    random rows up to k."""
    rng = np.random.default_rng(seed)
    tiles = (n + 255) // 256
    rows = {int(rng.integers(0, tiles)) * 256 + s for s in range(256)}
    rows.update(t * 256 for t in range(tiles))
    rows.update(min(n - 1, t * 256 + 255) for t in range(tiles))
    rows = {r for r in rows if r < n}
    while len(rows) < k:
        rows.add(int(rng.integers(0, n)))
    return sorted(rows)


def test_qwen3_8b_shape_512_oracle_rows():
    w = wl("qwen3_8b")
    say("qwen3_8b forward")
    logp = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    rows = tile_slot_rows(w.n, 512, 2)
    assert len(rows) >= 512 and {r % 256 for r in rows} == set(range(256))
    check_rows(w.h, w.w, w.ids, logp, rows, "qwen3_8b",
               h_host=host("qwen3_8b", "h"), w_host=host("qwen3_8b", "w"))


def test_dsv3_shape_256_oracle_rows_with_every_sequence_boundary():
    w = wl("dsv3")
    say("dsv3 forward")
    logp = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    cu = w.cu_seqlens.cpu().numpy()
    ends = [int(cu[j]) for j in range(64)] + [int(cu[j + 1]) - 1 for j in range(64)]
    rng = np.random.default_rng(3)
    rows = set(ends)
    while len(rows) < 256:
        rows.add(int(rng.integers(0, w.n)))
    check_rows(w.h, w.w, w.ids, logp, sorted(rows), "dsv3",
               h_host=host("dsv3", "h"), w_host=host("dsv3", "w"))
    assert torch.all(torch.isfinite(logp))


def test_fp32_head_128_oracle_rows_and_bf16_rerun():
    w = wl("fp32_head")
    say("fp32_head forward (fp32 MFMA)")
    logp32 = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    rows = tile_slot_rows(w.n, 128, 4)[::3][:96] + spread_rows(w.n, 40, 4, extra=[4095])
    rows = sorted(set(rows))
    assert len(rows) >= 128
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

@pytest.mark.parametrize("n", [70, 20, 3])      # 256-token kernel; small-batch kernel, 2 and 1 blocks
def test_equal_logits_and_bad_ids(n):
    d, v = 128, 151936
    h = torch.randn(n, d, device=DEV).to(torch.bfloat16)
    w = torch.zeros(v, d, device=DEV, dtype=torch.bfloat16)
    ids = torch.randint(0, v, (n,), device=DEV, dtype=torch.int32)
    bad = [1, 2] if n < 10 else [3, 10]
    ids[bad[0]] = -100
    ids[bad[1]] = v
    say(f"equal logits, n={n}")
    logp, lse, nbad = tim.tim_logprob_forward(h, w, ids, return_lse=True)
    torch.cuda.synchronize()
    good = torch.ones(n, dtype=torch.bool)
    good[bad] = False
    lp = logp.cpu()
    assert torch.isnan(lp[bad[0]]) and torch.isnan(lp[bad[1]]) and int(nbad.item()) == 2
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


def test_qwen3_8b_small_batches_through_every_narrow_width():
    """Batches of 16 and fewer tokens take one token block per wave of the
    small-batch kernel, 17..32 two, 33..64 four; each must give the full
    batch's bits, and 65 the 256-token kernel's."""
    w = wl("qwen3_8b")
    full = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    full_bits = full.view(torch.int32).cpu()
    for b in (16, 17, 31, 32, 33, 48, 63, 64, 65):
        say(f"qwen3_8b sliced in batches of {b} (first 2048 rows)")
        got = _sliced(w.h[:2048], w.w, w.ids[:2048], workloads.sweep_slices(2048, b))
        diff = int((got.view(torch.int32).cpu() != full_bits[:2048]).sum())
        assert diff == 0, f"batch {b}: {diff} rows differ"


@pytest.mark.parametrize("d,v", [(64, 5), (256, 129), (128, 1000), (64, 32001)])
def test_small_batch_kernel_at_ragged_vocabularies(d, v):
    """Batches of at most 64 tokens take the small-batch kernel, whose last
    half-chunk of a vocabulary that is not a multiple of 128 reads its
    missing rows as zeros: the oracle's values, and the bits the 256-token
    kernel gives the same rows inside a batch of 300."""
    g = torch.Generator(device="cpu").manual_seed(d + v)
    h = torch.randn(300, d, generator=g).to(torch.bfloat16)
    w = (torch.randn(v, d, generator=g) * 0.05).to(torch.bfloat16)
    ids = torch.randint(0, v, (300,), generator=g, dtype=torch.int32)
    hd, wd, idd = h.to("cuda"), w.to("cuda"), ids.to("cuda")
    big = tim.tim_logprob_forward(hd, wd, idd)
    for b in (1, 5, 17, 32, 33, 64):
        say(f"d={d} v={v}: batch of {b}")
        got = tim.tim_logprob_forward(hd[:b].contiguous(), wd, idd[:b].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), big[:b].view(torch.int32)), b
        check_rows(hd[:b], wd, idd[:b], got, range(b), f"d={d} v={v} b={b}")


@pytest.mark.parametrize("name,sizes", [("dsv3", (1, 7, 64, 1000, 32768)),
                                        ("small", (1, 7, 17, 64, 1000, 2048))])
def test_batch_invariance_sweep_other_shapes(name, sizes):
    w = wl(name)
    say(f"{name} full batch (reference bits)")
    full = tim.tim_logprob_forward(w.h, w.w, w.ids)
    torch.cuda.synchronize()
    full_bits = full.view(torch.int32).cpu()
    for b in sizes:
        say(f"{name} sliced in batches of {b}")
        got = _sliced(w.h, w.w, w.ids, workloads.sweep_slices(w.n, b))
        diff = int((got.view(torch.int32).cpu() != full_bits).sum())
        assert diff == 0, f"{name} batch {b}: {diff} rows differ"
    say(f"{name} random partition")
    got = _sliced(w.h, w.w, w.ids, workloads.random_slices(w.n, 23))
    assert torch.equal(got.view(torch.int32).cpu(), full_bits)


def test_side_stream_gives_the_default_stream_bits():
    """Calls on a caller's side stream: inputs written on the current stream
    are waited for, and outputs equal the default-stream call bit for bit."""
    w = wl("small")
    ref = tim.tim_logprob_forward(w.h, w.w, w.ids)
    ref_st = tim.tim_mismatch_stats(ref, w.logp_rollout, w.mask, w.cu_seqlens,
                                    tis_clip=w.spec.clip_c, seq_bounds=(w.spec.seq_lo, w.spec.seq_hi))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    h2 = w.h * 1                                  # written on the current stream just before
    got = tim.tim_logprob_forward(h2, w.w, w.ids, stream=side)
    got_st = tim.tim_mismatch_stats(got, w.logp_rollout, w.mask, w.cu_seqlens,
                                    tis_clip=w.spec.clip_c,
                                    seq_bounds=(w.spec.seq_lo, w.spec.seq_hi), stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    assert torch.equal(got_st["batch"], ref_st["batch"])
    for k in ref_st["seq"]:
        assert torch.equal(got_st["seq"][k], ref_st["seq"][k]), k


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


@pytest.mark.parametrize("n", [2048, 256, 200, 64, 33, 7])
@pytest.mark.parametrize("schedule", ["free", "split_k"])
def test_other_schedules_match_oracle_and_are_deterministic(n, schedule):
    """The free and K-split schedules need not be batch invariant (the K
    split is not at 33..256 tokens), but their results must still match the
    oracle and repeat."""
    w = wl("small")
    h, ids = w.h[:n], w.ids[:n]
    say(f"small: {schedule} schedule, n={n}")
    a = tim.tim_logprob_forward(h, w.w, ids, schedule=schedule)
    b = tim.tim_logprob_forward(h, w.w, ids, schedule=schedule)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    rows = spread_rows(n, 40, 9) if n > 64 else range(n)
    check_rows(h, w.w, ids, a, rows, f"small {schedule} schedule n={n}",
               h_host=host("small", "h")[:n], w_host=host("small", "w"))


@pytest.mark.parametrize("n", [64, 300])
def test_fp32_free_schedule_is_the_invariant_one(n):
    """At the fp32 head's vocabulary and a few hundred tokens the free
    schedule is the invariant one (one tile per chunk in every schedule):
    the same bits, and the oracle's values."""
    w = wl("fp32_head")
    h, ids = w.h[:n], w.ids[:n]
    say(f"fp32_head: free schedule, n={n}")
    a = tim.tim_logprob_forward(h, w.w, ids, schedule="free")
    inv = tim.tim_logprob_forward(h, w.w, ids)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), inv.view(torch.int32))
    check_rows(h, w.w, ids, a, spread_rows(n, 24, 5, extra=(0, n - 1)),
               f"fp32_head free n={n}", h_host=host("fp32_head", "h")[:n],
               w_host=host("fp32_head", "w"))


def test_split_k_schedule_at_the_qwen3_shape():
    w = wl("qwen3_8b")
    n = 100
    say("qwen3_8b: K-split schedule, 100 tokens")
    a = tim.tim_logprob_forward(w.h[:n], w.w, w.ids[:n], schedule="split_k")
    inv = tim.tim_logprob_forward(w.h[:n], w.w, w.ids[:n])
    torch.cuda.synchronize()
    check_rows(w.h[:n], w.w, w.ids[:n], a, range(0, n, 3), "qwen3_8b free n=100",
               h_host=host("qwen3_8b", "h")[:n], w_host=host("qwen3_8b", "w"))
    # the two schedules agree to rounding (the K halves are summed separately)
    assert (a.double() - inv.double()).abs().max().item() < 1e-4


def test_empty_batch():
    w = wl("tiny")
    out = tim.tim_logprob_forward(w.h[:0], w.w, w.ids[:0])
    assert out.numel() == 0
