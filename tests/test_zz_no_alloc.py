"""tim_logprob_forward_noalloc (static per-device scratch, no workspace)
against tim_logprob_forward (caller's workspace), both through the C ABI.

Two calls in a row on one device, the second on a smaller batch taken from
other rows, so that anything the second call read from the first call's
scratch contents would show.  The bar is bit equality with the workspace
entry point on the same inputs (same kernels, same schedule), which is
stricter than the oracle tolerance those results are held to elsewhere.
"""
import sys

import pytest
import torch

import invariant_logprobs_amd as tim
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _forward_ws(lib, h, w, ids):
    n, d = h.shape
    v = w.shape[0]
    dt = tim.TIM_BF16 if h.dtype == torch.bfloat16 else tim.TIM_F32
    need = lib.tim_logprob_workspace_bytes(n, d, v, dt, tim.TIM_SCHED_INVARIANT)
    ws = torch.empty(max(int(need), 256), dtype=torch.uint8, device=DEV)
    logp = torch.empty(n, dtype=torch.float32, device=DEV)
    lse = torch.empty(n, dtype=torch.float32, device=DEV)
    nbad = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    st = lib.tim_logprob_forward(h.data_ptr(), h.stride(0), w.data_ptr(), w.stride(0),
                                 ids.data_ptr(), n, d, v, dt, tim.TIM_SCHED_INVARIANT,
                                 logp.data_ptr(), lse.data_ptr(), nbad.data_ptr(),
                                 ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == tim.TIM_OK, tim.status_string(st)
    return logp, lse, nbad


def _forward_noalloc(lib, h, w, ids):
    n, d = h.shape
    v = w.shape[0]
    dt = tim.TIM_BF16 if h.dtype == torch.bfloat16 else tim.TIM_F32
    # outputs start as NaN / -7 so that an unwritten entry cannot pass
    logp = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    nbad = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    st = lib.tim_logprob_forward_noalloc(h.data_ptr(), h.stride(0), w.data_ptr(), w.stride(0),
                                         ids.data_ptr(), n, d, v, dt, tim.TIM_SCHED_INVARIANT,
                                         logp.data_ptr(), lse.data_ptr(), nbad.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
    assert st == tim.TIM_OK, tim.status_string(st)
    return logp, lse, nbad


def _same_bits(a, b):
    return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))


# (workload, rows of the first call, first row and rows of the second call):
# bf16 through the 256-token kernel and then the small-batch kernel, the
# Qwen3-8B-shaped head at its full 8192 rows (39 MB of scratch) and then a
# ragged 300-row batch, and the fp32 head.
CASES = [("small", 2048, 1500, 20), ("qwen3_8b", 8192, 4000, 300), ("tiny", 64, 40, 5)]


@pytest.mark.parametrize("name,n1,off2,n2", CASES)
def test_noalloc_matches_workspace_entry_on_two_calls(name, n1, off2, n2):
    lib = tim.load_library()
    say(f"{name}: generating inputs")
    wl = workloads.make(name, device=DEV)
    h, w = wl.h, wl.w
    v = w.shape[0]
    dt = tim.TIM_BF16 if h.dtype == torch.bfloat16 else tim.TIM_F32
    need = lib.tim_logprob_workspace_bytes(n1, h.shape[1], v, dt, tim.TIM_SCHED_INVARIANT)
    assert 0 < need <= tim.NOALLOC_SCRATCH_BYTES
    h1, ids1 = h[:n1], wl.ids[:n1].contiguous()
    h2 = h[off2:off2 + n2]
    ids2 = wl.ids[off2:off2 + n2].clone()
    ids2[1] = v + 5            # one out-of-range id: NaN and a count of 1
    torch.cuda.synchronize()

    say(f"{name}: first call, {n1} rows")
    got1 = _forward_noalloc(lib, h1, w, ids1)
    say(f"{name}: second call, {n2} rows from row {off2}")
    got2 = _forward_noalloc(lib, h2, w, ids2)
    ref1 = _forward_ws(lib, h1, w, ids1)
    ref2 = _forward_ws(lib, h2, w, ids2)
    torch.cuda.synchronize()

    for k, (g, r) in enumerate(zip(got1, ref1)):
        assert _same_bits(g, r), f"{name} first call, output {k}"
    for k, (g, r) in enumerate(zip(got2, ref2)):
        assert _same_bits(g, r), f"{name} second call, output {k}"
    assert int(got1[2].item()) == int(ref1[2].item())
    assert int(got2[2].item()) == 1
    assert torch.isnan(got2[0][1]) and torch.isfinite(got2[0][torch.arange(n2, device=DEV) != 1]).all()
    assert torch.isfinite(got1[0]).all() == torch.isfinite(ref1[0]).all()

    say(f"{name}: the first input again after the second")
    again = _forward_noalloc(lib, h1, w, ids1)
    torch.cuda.synchronize()
    for g, r in zip(again, ref1):
        assert _same_bits(g, r)
    del wl, h, w
    torch.cuda.empty_cache()


def test_noalloc_refuses_requests_beyond_its_scratch():
    lib = tim.load_library()
    d, v = 4096, 151936
    n = 1
    while lib.tim_logprob_workspace_bytes(n, d, v, tim.TIM_BF16, 0) <= tim.NOALLOC_SCRATCH_BYTES:
        n *= 2
    # buffers of the full sizes, so that even a launch would stay in bounds
    h = torch.zeros(n, d, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(v, d, dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(n, dtype=torch.int32, device=DEV)
    logp = torch.full((n,), 3.0, dtype=torch.float32, device=DEV)
    st = lib.tim_logprob_forward_noalloc(h.data_ptr(), d, w.data_ptr(), d, ids.data_ptr(), n, d,
                                         v, tim.TIM_BF16, 0, logp.data_ptr(), None, None,
                                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == tim.TIM_ESCRATCH
    assert bool((logp == 3.0).all())      # refused before any launch
    say(f"refused {n} rows: {tim.status_string(st)}")
