"""Host-side checks of libtim.so: it loads, exports every symbol the header
declares, sizes workspaces as documented, and rejects bad arguments before any
launch.  No call here reaches the GPU (every checked path returns during host
validation), so these run without one."""
import ctypes
import os
import re

import pytest
import torch

import invariant_logprobs_amd as tim

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tim.h")
FAKE = 0x10000           # non-null, 256-byte aligned host value; never dereferenced


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tim_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return tim.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert declared == sorted(tim.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.tim_abi_version() == tim.ABI_VERSION == 5


def test_status_strings(lib):
    for st in range(6):
        assert tim.status_string(st).startswith("TIM_")
    assert "TIM_NOALLOC_SCRATCH_BYTES" in tim.status_string(tim.TIM_ESCRATCH)
    assert "unknown" in tim.status_string(99)


def test_logprob_workspace_layout(lib):
    # invariant schedule: 256-entry vocabulary chunks, (max, sum) fp32 pairs
    n, d, v = 8192, 4096, 151936
    chunks = -(-v // 256)
    assert chunks == 594
    want = -(-(chunks * n * 8) // 256) * 256 + -(-(n * 4) // 256) * 256
    assert lib.tim_logprob_workspace_bytes(n, d, v, tim.TIM_BF16, tim.TIM_SCHED_INVARIANT) == want
    # the invariant layout does not depend on dtype; it scales with n only linearly
    assert lib.tim_logprob_workspace_bytes(n, d, v, tim.TIM_F32, 0) == want
    assert lib.tim_logprob_workspace_bytes(-1, d, v, 0, 0) == 0
    assert lib.tim_logprob_workspace_bytes(n, d, v, 7, 0) == 0
    assert lib.tim_logprob_workspace_bytes(n, d, v, 0, 5) == 0
    # the K-split schedule keeps two partial-logit copies at 33..256 tokens
    # (at 64 tokens the invariant schedule takes the small-batch kernel,
    # whose partials are per half chunk; the K split, asked for, takes the
    # 256-token tile's chunk partials plus the two copies)
    small = lib.tim_logprob_workspace_bytes(64, d, v, tim.TIM_BF16, tim.TIM_SCHED_INVARIANT)
    split = lib.tim_logprob_workspace_bytes(64, d, v, tim.TIM_BF16, tim.TIM_SCHED_SPLIT_K)
    assert small == -(-(2 * chunks * 64 * 8) // 256) * 256 + 256
    assert split >= -(-(chunks * 64 * 8) // 256) * 256 + 256 + 2 * v * 64 * 4
    assert lib.tim_logprob_workspace_bytes(64, d, v, tim.TIM_BF16, tim.TIM_SCHED_FREE) == small
    assert lib.tim_stats_workspace_bytes(1 << 20, 1000) > 0
    assert lib.tim_stats_workspace_bytes(-1, 3) == 0


def _fwd(lib, **kw):
    a = dict(h=FAKE, ldh=64, w=FAKE, ldw=64, ids=FAKE, n=4, d=64, v=100, dtype=0, flags=0,
             logp=FAKE, lse=None, nbad=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.tim_logprob_forward(a["h"], a["ldh"], a["w"], a["ldw"], a["ids"], a["n"], a["d"],
                                   a["v"], a["dtype"], a["flags"], a["logp"], a["lse"],
                                   a["nbad"], a["ws"], a["wsb"], a["stream"])


def test_logprob_argument_errors(lib):
    assert _fwd(lib, n=-1) == tim.TIM_EINVAL
    assert _fwd(lib, d=0) == tim.TIM_EINVAL
    assert _fwd(lib, v=0) == tim.TIM_EINVAL
    assert _fwd(lib, v=1 << 31) == tim.TIM_EINVAL
    assert _fwd(lib, dtype=2) == tim.TIM_EINVAL
    assert _fwd(lib, flags=3) == tim.TIM_EINVAL
    assert _fwd(lib, ldh=32) == tim.TIM_EINVAL
    assert _fwd(lib, ldw=63) == tim.TIM_EINVAL
    assert _fwd(lib, h=None) == tim.TIM_EINVAL
    assert _fwd(lib, ids=None) == tim.TIM_EINVAL
    assert _fwd(lib, logp=None) == tim.TIM_EINVAL
    assert _fwd(lib, d=96, ldh=96, ldw=96) == tim.TIM_EUNSUPPORTED      # d % 64
    assert _fwd(lib, ldh=68) == tim.TIM_EUNSUPPORTED                     # 136 B rows
    assert _fwd(lib, dtype=1, ldh=66, ldw=64) == tim.TIM_EUNSUPPORTED    # fp32, 264 B rows
    assert _fwd(lib, h=FAKE + 8) == tim.TIM_EUNSUPPORTED                 # 16-byte alignment
    assert _fwd(lib, ws=None) == tim.TIM_EWORKSPACE
    assert _fwd(lib, wsb=16) == tim.TIM_EWORKSPACE
    assert _fwd(lib, ws=FAKE + 16) == tim.TIM_EUNSUPPORTED               # 256-byte alignment
    # n == 0: success with no launch and no pointer needed
    assert _fwd(lib, n=0, h=None, w=None, ids=None, logp=None, ws=None) == tim.TIM_OK


def _stats(lib, n=10, s=2, c=2.0, lo=-0.01, hi=0.01, lt=FAKE, lr=FAKE, cu=FAKE, ws=FAKE,
           wsb=1 << 30, params=True, k3=float("inf")):
    p = tim._StatsParams(c, lo, hi, k3)
    return lib.tim_mismatch_stats(lt, lr, None, cu, n, s, ctypes.byref(p) if params else None,
                                  None, None, None, ws, wsb, None)


def test_stats_argument_errors(lib):
    assert _stats(lib, n=-1) == tim.TIM_EINVAL
    assert _stats(lib, s=-1) == tim.TIM_EINVAL
    assert _stats(lib, s=0) == tim.TIM_EINVAL
    assert _stats(lib, params=False) == tim.TIM_EINVAL
    assert _stats(lib, c=0.0) == tim.TIM_EINVAL
    assert _stats(lib, c=-2.0) == tim.TIM_EINVAL
    assert _stats(lib, c=float("inf")) == tim.TIM_EINVAL
    assert _stats(lib, c=float("nan")) == tim.TIM_EINVAL
    assert _stats(lib, lo=0.1, hi=0.0) == tim.TIM_EINVAL
    assert _stats(lib, lo=float("nan")) == tim.TIM_EINVAL
    assert _stats(lib, k3=float("nan")) == tim.TIM_EINVAL
    assert _stats(lib, lt=None) == tim.TIM_EINVAL
    assert _stats(lib, cu=None) == tim.TIM_EINVAL
    assert _stats(lib, ws=None) == tim.TIM_EWORKSPACE
    assert _stats(lib, wsb=8) == tim.TIM_EWORKSPACE
    assert _stats(lib, ws=FAKE + 64) == tim.TIM_EUNSUPPORTED
    assert _stats(lib, n=1 << 31, s=2) == tim.TIM_EUNSUPPORTED
    assert _stats(lib, n=0, s=0, lt=None, lr=None, cu=None, ws=None) == tim.TIM_OK


def test_binding_refuses_host_tensors():
    import torch
    h = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        tim.tim_logprob_forward(h, h, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError):
        tim.tim_mismatch_stats(torch.zeros(4), torch.zeros(4), None,
                               torch.tensor([0, 4], dtype=torch.int32))


def _extras(lib, n=10, tau=0.1, rq=(0.5,), aq=(0.95,), lt=FAKE, lr=FAKE, ws=FAKE, wsb=1 << 30,
            params=True, nrq=None, naq=None):
    q = lambda v: (ctypes.c_double * tim.X_MAX_Q)(*(list(v) + [0.0] * (tim.X_MAX_Q - len(v))))
    p = tim._ExtrasParams(tau, len(rq) if nrq is None else nrq, len(aq) if naq is None else naq,
                          q(rq), q(aq))
    return lib.tim_mismatch_extras(lt, lr, None, n, ctypes.byref(p) if params else None, None,
                                   ws, wsb, None)


def test_extras_workspace_and_argument_errors(lib):
    # the workspace depends on n only: none is used up to 8192 tokens (one
    # block keeps everything in LDS); above, it is dominated by the candidate
    # regions, a quarter of the keys (2 bytes per token) plus a margin
    small, big = lib.tim_extras_workspace_bytes(8192), lib.tim_extras_workspace_bytes(1 << 28)
    assert 0 < small <= 256
    assert 2 * (1 << 28) < big < 3 * (1 << 28)
    assert lib.tim_extras_workspace_bytes(8193) > small
    assert lib.tim_extras_workspace_bytes(0) > 0
    assert lib.tim_extras_workspace_bytes(-1) == 0
    assert lib.tim_extras_workspace_bytes(1 << 31) == 0
    assert _extras(lib, n=-1) == tim.TIM_EINVAL
    assert _extras(lib, params=False) == tim.TIM_EINVAL
    assert _extras(lib, tau=float("nan")) == tim.TIM_EINVAL
    assert _extras(lib, rq=(1.5,)) == tim.TIM_EINVAL
    assert _extras(lib, aq=(-0.1,)) == tim.TIM_EINVAL
    assert _extras(lib, rq=(float("nan"),)) == tim.TIM_EINVAL
    assert _extras(lib, rq=(0.1, 0.2, 0.3), aq=(0.4, 0.5)) == tim.TIM_EINVAL   # 5 > 4
    assert _extras(lib, nrq=-1) == tim.TIM_EINVAL
    assert _extras(lib, lt=None) == tim.TIM_EINVAL
    assert _extras(lib, ws=None) == tim.TIM_EWORKSPACE
    assert _extras(lib, wsb=8) == tim.TIM_EWORKSPACE
    assert _extras(lib, ws=FAKE + 64) == tim.TIM_EUNSUPPORTED
    assert _extras(lib, n=1 << 31) == tim.TIM_EUNSUPPORTED


def test_binding_extras_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        tim.tim_mismatch_extras(torch.zeros(4), torch.zeros(4), None, tok_tau=0.1)


def test_backward_and_ppo_argument_errors(lib):
    fwd = lambda **kw: lib.tim_logprob_backward(
        kw.get("h", FAKE), kw.get("ldh", 64), kw.get("w", FAKE), kw.get("ldw", 64),
        kw.get("ids", FAKE), kw.get("lse", FAKE), kw.get("g", FAKE), kw.get("n", 4),
        kw.get("d", 64), kw.get("v", 100), kw.get("dtype", 0), kw.get("flags", 0),
        kw.get("dh", FAKE), kw.get("dw", FAKE), kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)
    assert fwd(n=-1) == tim.TIM_EINVAL
    assert fwd(flags=2) == tim.TIM_EINVAL
    assert fwd(dtype=2) == tim.TIM_EINVAL
    assert fwd(dtype=1, ldh=66, ldw=64) == tim.TIM_EUNSUPPORTED     # fp32, 264 B rows
    assert fwd(lse=None) == tim.TIM_EINVAL
    assert fwd(g=None) == tim.TIM_EINVAL
    assert fwd(d=96, ldh=96, ldw=96) == tim.TIM_EUNSUPPORTED
    assert fwd(ws=None) == tim.TIM_EWORKSPACE
    assert fwd(ws=FAKE + 16) == tim.TIM_EUNSUPPORTED
    assert fwd(dh=FAKE + 4) == tim.TIM_EUNSUPPORTED                 # 16-byte aligned outputs
    assert fwd(dw=FAKE + 8) == tim.TIM_EUNSUPPORTED
    assert fwd(n=0, dw=FAKE + 8) == tim.TIM_EUNSUPPORTED
    assert lib.tim_logprob_backward_workspace_bytes(8192, 4096, 151936, 2) == 0
    # fp32: W^T, h^T and dz in both layouts, fp32
    b32 = lib.tim_logprob_backward_workspace_bytes(4096, 4096, 151936, 1)
    assert 4 * (4096 * 151936 + 4096 * 4096 + 2 * 151936 * 4096) <= b32 \
        <= 4 * (4096 * 151936 + 4096 * 4096 + 2 * 151936 * 4096) + 1024
    b = lib.tim_logprob_backward_workspace_bytes(8192, 4096, 151936, 0)
    # h^T and dz (once), bf16, vocabulary padded to 151936 (a multiple of
    # 64 already); W and dz are read K-major, so neither W^T nor dz^T
    assert 2 * (4096 * 8192 + 151936 * 8192) <= b <= 2 * (4096 * 8192 + 151936 * 8192) + 1024
    p = tim._PpoParams(0.2, 0.28, 0, 2.0)
    ppo = lambda **kw: lib.tim_ppo_loss(FAKE, FAKE, FAKE, FAKE, None, kw.get("n", 10),
                                        ctypes.byref(kw.get("p", p)) if kw.get("params", True)
                                        else None, None, None, kw.get("ws", FAKE),
                                        kw.get("wsb", 1 << 24), None)
    assert ppo(n=-1) == tim.TIM_EINVAL
    assert ppo(params=False) == tim.TIM_EINVAL
    assert ppo(p=tim._PpoParams(-0.1, 0.28, 0, 0.0)) == tim.TIM_EINVAL
    assert ppo(p=tim._PpoParams(0.2, float("nan"), 0, 0.0)) == tim.TIM_EINVAL
    assert ppo(p=tim._PpoParams(0.2, 0.28, 2, 0.0)) == tim.TIM_EINVAL
    assert ppo(p=tim._PpoParams(0.2, 0.28, 0, float("nan"))) == tim.TIM_EINVAL
    for bad in (-1.0, float("nan"), float("inf")):
        assert ppo(p=tim._PpoParams(0.2, 0.28, 0, 2.0, bad)) == tim.TIM_EINVAL
    assert ppo(ws=None) == tim.TIM_EWORKSPACE
    assert ppo(wsb=8) == tim.TIM_EWORKSPACE
    assert ppo(ws=FAKE + 8) == tim.TIM_EUNSUPPORTED


def _fp(temperature=1.0, gamma=None, eps=1e-6):
    return ctypes.byref(tim._ForwardParams(temperature, gamma, eps))


def test_forward_ex_workspace_layout(lib):
    n, d, v = 8192, 4096, 151936
    chunks = -(-v // 256)
    up = lambda x: -(-x // 256) * 256
    plain = up(chunks * n * 8) + up(n * 4)
    ws = lambda **kw: lib.tim_logprob_ex_workspace_bytes(
        n, d, v, kw.get("dtype", 0), 0, _fp(kw.get("tau", 1.0), kw.get("g"), kw.get("eps", 1e-6)),
        kw.get("ent", 0))
    assert ws() == plain == lib.tim_logprob_workspace_bytes(n, d, v, 0, 0)
    assert ws(tau=0.7) == plain
    assert ws(ent=1) == plain + up(chunks * n * 4)                  # the entropy partials
    assert ws(g=FAKE) == plain + up(n * d * 2)                      # normalised bf16 rows
    assert ws(g=FAKE, dtype=1, ent=1) == plain + up(chunks * n * 4) + up(n * d * 4)
    assert ws(tau=0.0) == 0 and ws(tau=-1.0) == 0 and ws(tau=float("inf")) == 0
    assert ws(tau=float("nan")) == 0
    assert ws(g=FAKE, eps=-1.0) == 0 and ws(g=FAKE, eps=float("nan")) == 0
    assert lib.tim_logprob_ex_workspace_bytes(n, d, v, 0, 0, None, 0) == 0


def _fwdx(lib, **kw):
    a = dict(h=FAKE, ldh=64, w=FAKE, ldw=64, ids=FAKE, n=4, d=64, v=100, dtype=0, flags=0,
             prm=_fp(), logp=FAKE, lse=None, ent=None, nbad=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.tim_logprob_forward_ex(a["h"], a["ldh"], a["w"], a["ldw"], a["ids"], a["n"], a["d"],
                                      a["v"], a["dtype"], a["flags"], a["prm"], a["logp"],
                                      a["lse"], a["ent"], a["nbad"], a["ws"], a["wsb"], a["stream"])


def test_forward_ex_and_rmsnorm_argument_errors(lib):
    assert _fwdx(lib, prm=None) == tim.TIM_EINVAL
    assert _fwdx(lib, prm=_fp(0.0)) == tim.TIM_EINVAL
    assert _fwdx(lib, prm=_fp(float("nan"))) == tim.TIM_EINVAL
    assert _fwdx(lib, prm=_fp(1.0, FAKE, -1.0)) == tim.TIM_EINVAL
    assert _fwdx(lib, n=-1) == tim.TIM_EINVAL
    assert _fwdx(lib, ldh=32) == tim.TIM_EINVAL
    assert _fwdx(lib, logp=None) == tim.TIM_EINVAL
    assert _fwdx(lib, d=96, ldh=96, ldw=96) == tim.TIM_EUNSUPPORTED
    assert _fwdx(lib, h=FAKE + 2) == tim.TIM_EUNSUPPORTED            # unaligned rows ...
    assert _fwdx(lib, h=FAKE + 2, prm=_fp(1.0, FAKE), ws=None) == tim.TIM_EWORKSPACE  # ... fine with a norm
    assert _fwdx(lib, ws=None) == tim.TIM_EWORKSPACE
    assert _fwdx(lib, ent=FAKE, wsb=lib.tim_logprob_workspace_bytes(4, 64, 100, 0, 0)) == \
        tim.TIM_EWORKSPACE                                             # entropy needs more
    assert _fwdx(lib, ws=FAKE + 8) == tim.TIM_EUNSUPPORTED
    assert _fwdx(lib, n=0, logp=None) == tim.TIM_OK                  # nothing to do
    norm = lambda **kw: lib.tim_rmsnorm(kw.get("x", FAKE), kw.get("ldx", 64), kw.get("g", FAKE),
                                        kw.get("n", 4), kw.get("d", 64), kw.get("dtype", 0),
                                        kw.get("eps", 1e-6), kw.get("y", FAKE), kw.get("ldy", 64),
                                        None, None)
    assert norm(n=-1) == tim.TIM_EINVAL
    assert norm(d=0) == tim.TIM_EINVAL
    assert norm(dtype=5) == tim.TIM_EINVAL
    assert norm(eps=-1e-6) == tim.TIM_EINVAL
    assert norm(eps=float("inf")) == tim.TIM_EINVAL
    assert norm(ldx=63) == tim.TIM_EINVAL
    assert norm(ldy=10) == tim.TIM_EINVAL
    assert norm(x=None) == tim.TIM_EINVAL
    assert norm(g=None) == tim.TIM_EINVAL
    assert norm(y=None) == tim.TIM_EINVAL
    assert norm(n=0, x=None, g=None, y=None) == tim.TIM_OK


def test_binding_norm_and_ex_refuse_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tim.tim_rmsnorm(x, torch.ones(64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        tim.tim_logprob_forward_ex(x, torch.zeros(10, 64, dtype=torch.bfloat16),
                                   torch.zeros(4, dtype=torch.int32), temperature=0.7)


def test_buffer_extent_limits_are_refused_before_any_launch(lib):
    """A 256-row operand tile is addressed through a buffer descriptor with
    a 32-bit extent and 32-bit per-lane offsets: sizes whose tile would
    reach 2^31 bytes are refused on the host."""
    big_ld = (1 << 31) // 255 // 2 + 64            # bf16 elements: 255 rows past 2^31
    big_ld -= big_ld % 64
    assert 255 * big_ld * 2 + 64 * 2 >= 1 << 31
    assert _fwd(lib, ldh=big_ld) == tim.TIM_EUNSUPPORTED
    assert _fwd(lib, ldw=big_ld) == tim.TIM_EUNSUPPORTED
    ok_ld = big_ld - 1024                           # just below: accepted by the check
    assert 255 * ok_ld * 2 + 64 * 2 < 1 << 31
    assert _fwd(lib, ldh=ok_ld, wsb=16) == tim.TIM_EWORKSPACE     # gets past it
    assert _fwdx(lib, ldw=big_ld) == tim.TIM_EUNSUPPORTED
    bwd = lambda **kw: lib.tim_logprob_backward(
        FAKE, kw.get("ldh", 64), FAKE, kw.get("ldw", 64), FAKE, FAKE, FAKE, kw.get("n", 4),
        64, kw.get("v", 100), 0, 0, FAKE, FAKE, FAKE, 1 << 62, None)
    # dW = dz^T h has K = tokens (rows of Np bf16), dh = dz W has K = vocabulary
    assert bwd(n=(1 << 22)) == tim.TIM_EUNSUPPORTED               # 512 Np >= 2^31
    assert bwd(v=(1 << 22)) == tim.TIM_EUNSUPPORTED
    assert bwd(ldh=big_ld) == tim.TIM_EUNSUPPORTED


def _fwd_noalloc(lib, **kw):
    a = dict(h=FAKE, ldh=64, w=FAKE, ldw=64, ids=FAKE, n=4, d=64, v=100, dtype=0, flags=0,
             logp=FAKE, lse=None, nbad=None, stream=None)
    a.update(kw)
    return lib.tim_logprob_forward_noalloc(a["h"], a["ldh"], a["w"], a["ldw"], a["ids"], a["n"],
                                           a["d"], a["v"], a["dtype"], a["flags"], a["logp"],
                                           a["lse"], a["nbad"], a["stream"])


def test_noalloc_checks_and_scratch_limit_before_any_device_call(lib):
    """The no-allocation forward shares the workspace entry point's host
    checks, and refuses a request whose workspace would exceed its static
    scratch (TIM_NOALLOC_SCRATCH_BYTES) before touching the device."""
    assert tim.NOALLOC_SCRATCH_BYTES == 64 << 20
    hdr = open(HEADER).read()
    assert "#define TIM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in hdr
    assert _fwd_noalloc(lib, n=0) == tim.TIM_OK
    assert _fwd_noalloc(lib, n=-1) == tim.TIM_EINVAL
    assert _fwd_noalloc(lib, d=32) == tim.TIM_EUNSUPPORTED
    assert _fwd_noalloc(lib, flags=3) == tim.TIM_EINVAL
    assert _fwd_noalloc(lib, logp=None) == tim.TIM_EINVAL
    assert _fwd_noalloc(lib, h=FAKE + 8) == tim.TIM_EUNSUPPORTED
    d, v = 4096, 151936
    fits = big = 0
    for n in (1, 64, 1000, 8192, 12000, 14000, 14100, 16384, 65536):
        need = lib.tim_logprob_workspace_bytes(n, d, v, 0, 0)
        if need > tim.NOALLOC_SCRATCH_BYTES:
            big += 1
            assert _fwd_noalloc(lib, n=n, d=d, v=v, ldh=d, ldw=d) == tim.TIM_ESCRATCH
        else:
            fits = n
    assert big >= 2 and 12000 <= fits < 16384      # the headline 8192-row head fits
    # the K-split schedule's partial logits at 256 tokens: 2 x 151936 x 256 fp32
    assert lib.tim_logprob_workspace_bytes(256, d, v, 0, tim.TIM_SCHED_SPLIT_K) > (64 << 20)
    assert _fwd_noalloc(lib, n=256, d=d, v=v, ldh=d, ldw=d,
                        flags=tim.TIM_SCHED_SPLIT_K) == tim.TIM_ESCRATCH


def test_cu_seqlens_debug_check():
    ok = torch.tensor([0, 3, 3, 10], dtype=torch.int32)
    tim._check_cu_seqlens(ok, 10)
    for bad, n in (([1, 3, 10], 10), ([0, 3, 9], 10), ([0, 5, 4, 10], 10), ([], 0)):
        with pytest.raises(ValueError):
            tim._check_cu_seqlens(torch.tensor(bad, dtype=torch.int32), n)
