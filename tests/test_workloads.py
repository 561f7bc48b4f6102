"""Seeded synthetic workloads: segment tables, value statistics, determinism."""

import numpy as np
import torch

import workloads as W


def test_segment_tables():
    expect = {1: (4, 332_776), 2: (161, 25_557_032), 3: (391, 335_141_888),
              4: (199, 109_482_240)}
    for cfg, (nseg, n) in expect.items():
        off = W.config_offsets(cfg)
        assert off.size - 1 == nseg and off[-1] == n and off[0] == 0
        assert np.all(np.diff(off) > 0)
    off5 = W.config_offsets(5)
    lengths = np.diff(off5)
    assert off5.size - 1 == 20000
    assert lengths.min() >= 1 and lengths.max() < 1_000_000
    # E[exp(U ln 1e6)] = (1e6 - 1) / ln 1e6 ~ 72382 per segment
    assert abs(off5[-1] / 20000 / 72382.0 - 1) < 0.05
    assert (lengths < 256).mean() > 0.35


def test_resnet_lengths_shape_list():
    lengths = W.resnet50_lengths()
    assert lengths[:3] == [9408, 64, 64]
    assert lengths[-2:] == [2_048_000, 1000]
    assert max(lengths) == 2_359_296  # 3x3 conv 512->512


def test_small_config_values():
    wl = W.make_workload(1)
    assert wl.K == 2 and all(g.dtype == torch.float32 for g in wl.grads)
    x = wl.grads[0].double()
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1) < 0.01
    again = W.make_workload(1)
    assert all(torch.equal(a, b) for a, b in zip(wl.grads, again.grads))
    other = W.make_workload(1, seed=7)
    assert not torch.equal(wl.grads[0], other.grads[0])


def test_stress_subset_statistics():
    full = W.segment_params(5, 5, 20000, 32)
    all_flagged = full["zero"].any(axis=0)
    assert 0.04 < all_flagged.mean() < 0.06
    lengths = np.diff(W.config_offsets(5))
    small_flagged = np.flatnonzero(all_flagged & (lengths < 5000))[:12]
    big = np.flatnonzero(~all_flagged & (lengths > 200_000) & (lengths < 300_000))[:4]
    segs = np.concatenate([small_flagged, big])
    wl = W.make_workload(5, segments=segs)
    assert wl.K == 32 and wl.grads[0].dtype == torch.bfloat16
    zero = wl.notes["params"]["zero"]
    flagged = zero.any(axis=0)
    assert flagged[:len(small_flagged)].all() and not flagged[len(small_flagged):].any()
    off = wl.seg_offsets
    for s in np.flatnonzero(flagged)[:20]:
        lo, hi = int(off[s]), int(off[s + 1])
        for k in range(wl.K):
            seg = wl.grads[k][lo:hi]
            assert bool((seg == 0).all()) == bool(zero[k, s])
    # the per-segment cosine with the shared direction shows up in pairwise dots
    cos = wl.notes["params"]["cosine"]
    big = [s for s in range(len(segs)) if off[s + 1] - off[s] > 200_000 and not flagged[s]][:5]
    for s in big:
        lo, hi = int(off[s]), int(off[s + 1])
        a, b = wl.grads[0][lo:hi].double(), wl.grads[1][lo:hi].double()
        c = float(a @ b / (a.norm() * b.norm()))
        assert abs(c - cos[s] ** 2) < 0.02


def test_fp16_scaled_values_keep_subnormals():
    wl = W.random_case(4, [5000] * 12, dtype="f16", seed=3, kind="scaled")
    g = wl.grads[0]
    sub = (g != 0) & (g.abs() < 6.1e-5)
    assert int(sub.sum()) > 0


def test_random_case_zero_workers():
    wl = W.random_case(3, [7, 0, 9], seed=1, zero_workers=(1,))
    assert wl.N == 16 and wl.nseg == 3
    assert bool((wl.grads[1] == 0).all()) and not bool((wl.grads[0] == 0).all())


def test_resnet_shared_component_cosine():
    # g_k = s + n_k with s, n_k ~ N(0,1): pairwise cosine 1/2 (checked on a few large layers)
    off = W.config_offsets(2)
    lengths = np.diff(off)
    segs = np.argsort(lengths)[-3:]
    wl = W.make_workload(2, segments=segs)
    a, b = wl.grads[0].double(), wl.grads[5].double()
    c = float(a @ b / (a.norm() * b.norm()))
    assert abs(c - 0.5) < 0.01
