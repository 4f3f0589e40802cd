"""Host checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

import workloads as W


def test_tiny_is_seeded_and_reproducible():
    a = W.make("tiny", device="cpu")
    b = W.make("tiny", device="cpu")
    for x, y in [(a.h, b.h), (a.w, b.w), (a.ids, b.ids), (a.logp_rollout, b.logp_rollout)]:
        assert torch.equal(x, y)
    assert a.h.dtype == torch.float32 and a.h.shape == (64, 256) and a.w.shape == (1024, 256)
    assert a.ids.dtype == torch.int32 and int(a.ids.min()) >= 0 and int(a.ids.max()) < 1024
    assert a.cu_seqlens.tolist() == [0, 16, 32, 48, 64] and a.mask is None
    # rollout record = sampler's logp + N(0, 1e-3^2)
    d = (a.logp_rollout - a.logp_sampler).double()
    assert 3e-4 < float(d.std()) < 3e-3 and float(d.abs().max()) < 6e-3
    # sampled ids have the softmax's typical log-probability, not uniform's
    assert -9 < float(a.logp_sampler.mean()) < -4


def test_small_has_prompt_mask_and_spikes():
    w = W.make("small", device="cpu")
    assert w.h.dtype == torch.bfloat16 and w.w.shape == (32000, 2048)
    m = w.mask.numpy()
    assert m.sum() == 2048 - 8 * 26
    for j in range(8):
        assert not m[256 * j: 256 * j + 26].any() and m[256 * j + 26: 256 * (j + 1)].all()
    d = (w.logp_rollout - w.logp_sampler).abs()
    assert int((d > 0.4).sum()) == 20          # round(0.01 * 2048) spikes of 0.5


def test_lognormal_lengths_and_stats_scale():
    lens = W.lognormal_lengths(32768, 64, 123)
    assert lens.sum() == 32768 and lens.min() >= 128 and lens.max() <= 4096
    lt, lr, mask, cu = W.stats_scale(1 << 15, device="cpu")
    assert int(cu[-1]) == 1 << 15 and int(cu[0]) == 0
    assert bool(torch.all(cu[1:] >= cu[:-1]))
    delta = (lt.double() - lr.double())
    assert int(torch.isnan(delta).sum()) >= 1
    assert int((delta > 0.9).sum()) >= 20
    assert 0.85 < float(mask.float().mean()) < 0.95


def test_sweep_partitions_cover_rows():
    for b in (1, 7, 64, 1000, 8192):
        sl = W.sweep_slices(8192, b)
        assert sl[0][0] == 0 and sl[-1][1] == 8192
        assert all(x[1] == y[0] for x, y in zip(sl, sl[1:]))
    rs = W.random_slices(8192, 11)
    assert rs[-1][1] == 8192 and all(1 <= e - s <= 1000 for s, e in rs)
