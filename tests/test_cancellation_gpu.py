"""GPU parity under deep cancellation: worker pairs that nearly cancel.

In the operator's properties, parallel gradients are averaged, so an exactly
anti-parallel pair of equal norms gives zero.  Next to that point a node is
far smaller than the operands under it, and every merge above it works on a
near-cancellation.  The inputs here are ``workloads.cancelling_pairs``:
g_{2m+1} = -(1 + eps) g_{2m} + eps n, so each level-1 node is about eps times
its operands and the level-2 merges see eps^2 in squared norm.
"""

import numpy as np
import pytest

import workloads as W
from parity import evaluate, passes, say

pytestmark = pytest.mark.gpu


def sweep_shape(case):
    """The shape that seeded sweep case ``case`` draws (K log-uniform in
    [1, 300), dtype, schedule, value family, 1-6 segments of 0 to 300,000
    rows, eps log-uniform in [1e-7, 1e-1] for the cancelling family)."""
    rng = np.random.default_rng(55000 + case)
    K = int(np.exp(rng.uniform(0, np.log(300))))
    dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
    schedule = "chain" if rng.random() < 0.4 else "tree"
    family = ["normal", "shared", "scaled", "cancel", "tiny", "huge"][int(rng.integers(0, 6))]
    lengths = []
    for _ in range(int(rng.integers(1, 7))):
        u = rng.random()
        if u < 0.05:
            lengths.append(0)
        elif u < 0.25:
            lengths.append(int(rng.integers(1, 9)))
        elif u < 0.45:
            lengths.append(int(rng.integers(9, 300)))
        elif u < 0.70:
            lengths.append(int(rng.integers(300, 20000)))
        else:
            lengths.append(int(rng.integers(20000, 300000)))
    while K * max(sum(lengths), 1) > 3e7:
        lengths = [n // 2 for n in lengths]
    eps = float(np.exp(rng.uniform(np.log(1e-7), np.log(1e-1)))) if family == "cancel" else None
    return K, dtype, schedule, family, lengths, eps


# The sweep cases (of 1,500) whose shapes missed a gate: twelve fp32 shapes
# whose output missed the 1e-5 relative L2 gate by up to 1.1e-2, and a bf16
# chain (K = 177) whose third-stage coefficient was off by 3.0e-6.
FAILED_SWEEP_CASES = [100, 127, 146, 277, 435, 500, 742, 786, 867, 931, 1315, 1427, 1441]


def test_failed_sweep_shapes(gpu):
    bad = []
    for case in FAILED_SWEEP_CASES:
        K, dtype, schedule, family, lengths, eps = sweep_shape(case)
        assert family == "cancel"
        wl = W.cancelling_pairs(K, lengths, eps, dtype=dtype, seed=55000 + case)
        wl.grads = [g.to(gpu) for g in wl.grads]
        ev = evaluate(wl, schedule)
        ok = passes(ev, dtype)
        say(f"sweep case {case}: K={K} {dtype} {schedule} eps={eps:.3g} lengths={lengths}: relative L2 "
            f"{ev['rel_l2']:.3g}, worst segment {ev['seg_worst']} at {ev['seg_ratio']:.3g} of its budget, "
            f"coefficient error {ev['coeff_err']:.3g}, {ev['exempt']} exempt{'' if ok else '  FAIL'}")
        if not ok:
            bad.append(case)
    assert not bad, f"cases {bad} miss a gate"


@pytest.mark.parametrize("K,schedule", [(4, "tree"), (16, "tree"), (20, "tree"), (16, "chain"), (40, "chain")])
@pytest.mark.parametrize("eps2", [1e-10, 1e-12])
def test_planted_cancellations_are_gated(gpu, K, schedule, eps2):
    """fp32 pairs cancelling to eps^2 = 1e-10 and 1e-12 in squared norm,
    over segments of many tiles, one tile and a few rows, in one block and
    across stages (K = 20, chains of 16 and 40).  The oracle resolves these
    merges (its rounding floor is near 1e-16), so every coefficient above
    them is gated, and the GPU must meet it: the walk flags those merges and
    recomputes their Gram entries exactly."""
    lengths = [70000, 3000, 7]
    wl = W.cancelling_pairs(K, lengths, np.sqrt(eps2), dtype="f32", seed=700 + K)
    wl.grads = [g.to(gpu) for g in wl.grads]
    ev = evaluate(wl, schedule)
    say(f"planted eps^2={eps2:g} K={K} {schedule}: relative L2 {ev['rel_l2']:.3g}, worst segment "
        f"{ev['seg_worst']} at {ev['seg_ratio']:.3g} of its budget, coefficient error {ev['coeff_err']:.3g}, "
        f"{ev['exempt']} exempt")
    assert ev["exempt"] == 0
    assert passes(ev, "f32")


def nearly_parallel_case(case):
    """The shape and inputs seeded sweep case ``case`` of nearly parallel
    workers draws: g_k = s_k (v + eta n_k), with per-worker scales s_k
    log-uniform over e^-8..1 (e^-3..1 for fp16) and random signs, eta
    log-uniform in [1e-6, 1e-1], 1-5 segments up to 200,000 rows."""
    import torch
    rng = np.random.default_rng(case)
    dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
    K = int(np.exp(rng.uniform(np.log(2), np.log(100))))
    schedule = "chain" if rng.random() < 0.5 else "tree"
    lengths = [int(np.exp(rng.uniform(0, np.log(200000)))) for _ in range(int(rng.integers(1, 6)))]
    while K * sum(lengths) > 2e7:
        lengths = [max(1, n // 2) for n in lengths]
    N = sum(lengths)
    eta = float(np.exp(rng.uniform(np.log(1e-6), np.log(1e-1))))
    span = 3.0 if dtype == "f16" else 8.0
    s = np.exp(rng.uniform(-span, 0, size=K)) * rng.choice([-1.0, 1.0], size=K)
    g = torch.Generator().manual_seed(case)
    v = torch.randn(N, generator=g, dtype=torch.float64)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    grads = [(float(s[k]) * (v + eta * torch.randn(N, generator=g, dtype=torch.float64))).to(tdt) for k in range(K)]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return W.Workload(K=K, dtype=dtype, seg_offsets=off, grads=grads, seed=case), schedule


@pytest.mark.parametrize("case", [511121, 520000, 520001, 520002])
def test_nearly_parallel_workers_with_random_scales(gpu, case):
    """Nearly parallel workers of random sign and scale: the chain's running
    result cancels against the next worker again and again, and each
    coefficient's error moves the result every later merge builds on.  In
    case 511121 (K = 98 fp32 chain) coefficients within 2.5e-7 of their own
    nodes, the old refinement bound, ended 1.85e-6 off at node 84.  Blocks
    over fp64 sums now refine below 1e-10."""
    wl, schedule = nearly_parallel_case(case)
    wl.grads = [g.to(gpu) for g in wl.grads]
    ev = evaluate(wl, schedule)
    say(f"nearly parallel case {case} K={wl.K} {wl.dtype} {schedule}: relative L2 {ev['rel_l2']:.3g}, "
        f"coefficient error {ev['coeff_err']:.3g}, {ev['exempt']} exempt")
    assert passes(ev, wl.dtype)


@pytest.mark.parametrize("K,schedule", [(12, "tree"), (20, "tree"), (16, "chain")])
def test_planted_cancellations_in_grouped_segments(gpu, K, schedule):
    """The same fp32 pairs cancelling to eps^2 = 1e-12, over a segment of 147
    tiles, whose walk first reads sums of groups of 16 tiles.  The flagged
    pairs' partials are then recomputed exactly for every tile and walked
    again tile by tile in double-double, as in short segments."""
    lengths = [300_000, 3000, 7]
    wl = W.cancelling_pairs(K, lengths, np.sqrt(1e-12), dtype="f32", seed=750 + K)
    wl.grads = [g.to(gpu) for g in wl.grads]
    ev = evaluate(wl, schedule)
    say(f"planted grouped K={K} {schedule}: relative L2 {ev['rel_l2']:.3g}, worst segment "
        f"{ev['seg_worst']} at {ev['seg_ratio']:.3g} of its budget, coefficient error {ev['coeff_err']:.3g}, "
        f"{ev['exempt']} exempt")
    assert ev["exempt"] == 0
    assert passes(ev, "f32")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("K", [4, 32])
def test_planted_cancellations_16bit(gpu, dtype, K):
    """16-bit pairs g_{2m+1} = -g_{2m} except for a few elements moved by one
    ulp: each level-1 node is exactly 3/2 of those few differences, about
    1e-11 (fp16) or 1e-9 (bf16) of its operands in squared norm, and the
    merges above it take their statistics from the matrix cores' 32-row fp32
    sums unless the walk flags them for exact recomputation."""
    import torch
    lengths = [70000, 4096, 300]
    base = W.random_case(K, lengths, dtype=dtype, seed=800 + K, kind="normal")
    rng = np.random.default_rng(800 + K)
    grads = []
    for k in range(K):
        g = base.grads[k]
        if k % 2 == 1:
            g = -grads[k - 1].clone()
            idx = torch.as_tensor(rng.choice(g.numel(), size=7, replace=False))
            bits = g.view(torch.int16)
            bits[idx] += 1  # one ulp away from zero, in magnitude
        grads.append(g)
    wl = W.Workload(K=K, dtype=dtype, seg_offsets=base.seg_offsets, grads=[g.to(gpu) for g in grads], seed=800 + K)
    ev = evaluate(wl, "tree")
    say(f"planted 16-bit {dtype} K={K}: relative L2 {ev['rel_l2']:.3g}, worst segment {ev['seg_worst']} at "
        f"{ev['seg_ratio']:.3g} of its budget, coefficient error {ev['coeff_err']:.3g}, {ev['exempt']} exempt")
    assert passes(ev, dtype)


@pytest.mark.parametrize("K,schedule", [(4, "tree"), (16, "chain")])
def test_small_combine_recomputes_flagged_pairs(gpu, K, schedule):
    """A small one-block combine takes two launches: the Gram pass, then the
    walk and weighted sum in one (each workgroup walks its own segment).  A
    merge flagged there, here above fp32 pairs cancelling to eps^2 = 1e-12,
    is recomputed exactly inside that launch: the Gram pass's rounding
    (about 2^-44 of the entries' terms) would otherwise move the
    coefficients above those pairs by about 2^-44 / 1e-12, far beyond the
    1e-6 gate."""
    from distributed_sgd_gradient_amd import _native
    lengths = [5000, 300, 3]
    wl = W.cancelling_pairs(K, lengths, np.sqrt(1e-12), dtype="f32", seed=900 + K)
    wl.grads = [g.to(gpu) for g in wl.grads]
    _native.profile_begin()
    try:
        ev = evaluate(wl, schedule)
    finally:
        kinds = _native.profile_end()
    launches = {k: v["launches"] for k, v in kinds.items()}
    say(f"small combine K={K} {schedule}: launches {launches}, relative L2 {ev['rel_l2']:.3g}, worst segment "
        f"{ev['seg_worst']} at {ev['seg_ratio']:.3g} of its budget, coefficient error {ev['coeff_err']:.3g}")
    assert launches == {"gram": 1, "wsum": 1}, launches
    assert ev["exempt"] == 0
    assert passes(ev, "f32")
