"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

The gates are those of ``parity`` (tests/parity.py): relative L2 of the whole
output and of every segment against its own norm (one output ulp per element
allowed), every coefficient away from the zero discontinuity within 1e-6, and
the statistics within 1e-5.  Inputs come from the seeded generators in
``workloads``; the oracle sees the same tensors copied to the host.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import TOL, check_coeffs, evaluate, full_check, passes, rel_l2, run_gpu, sampled_check, say

pytestmark = pytest.mark.gpu


def _A():
    import distributed_sgd_gradient_amd as A
    return A


# ---------------------------------------------------------------- workloads

def test_config1_full(gpu):
    wl = W.make_workload(1, device=gpu)
    _, _, err = full_check(wl, "config1")
    say("config1 relative L2", err)


def test_config2_full(gpu):
    wl = W.make_workload(2, device=gpu)
    full_check(wl, "config2")


def _spread(nseg, rng, extra=()):
    pick = set(range(min(3, nseg))) | set(range(max(0, nseg - 3), nseg)) | set(extra)
    pick |= set(rng.choice(nseg, size=min(8, nseg), replace=False).tolist())
    return sorted(pick)


@pytest.mark.parametrize("schedule", ["tree", "chain"])
def test_config3_sampled_full_size(gpu, schedule):
    # the BERT-Large workload at full size, as the benchmark runs it (and as a chain)
    wl = W.make_workload(3, device=gpu)
    lengths = np.diff(wl.seg_offsets)
    segs = _spread(wl.nseg, np.random.default_rng(3), extra=[int(np.argmax(lengths)), 10, 11, 15, 16])
    sampled_check(wl, segs, f"config3 {schedule}", schedule=schedule)


def test_config4_sampled_full_size(gpu):
    wl = W.make_workload(4, device=gpu)
    segs = _spread(wl.nseg, np.random.default_rng(4), extra=[0, 9, 13])
    sampled_check(wl, segs, "config4")


def test_config4_sampled_full_size_chain(gpu):
    # 64 fp16 inputs as a left-to-right chain: a block of the first 16, then stages of the running
    # result (fp64) and up to 15 more inputs
    wl = W.make_workload(4, device=gpu)
    segs = _spread(wl.nseg, np.random.default_rng(41), extra=[0, 9, 13])
    sampled_check(wl, segs, "config4 chain", schedule="chain")


@pytest.mark.parametrize("schedule", ["tree", "chain"])
def test_config5_sampled_full_size(gpu, schedule):
    wl = W.make_workload(5, device=gpu)
    lengths = np.diff(wl.seg_offsets)
    zero = wl.notes["params"]["zero"]
    flagged = np.flatnonzero(zero.any(axis=0))
    all_zero = np.flatnonzero(zero.all(axis=0))
    rng = np.random.default_rng(5)
    extra = list(flagged[:12]) + list(all_zero[:2]) + [int(np.argmin(lengths)), int(np.argmax(lengths))]
    extra += list(np.flatnonzero(lengths == 1)[:5])
    segs = _spread(wl.nseg, rng, extra=extra)
    sampled_check(wl, [int(s) for s in segs], f"config5 {schedule}", schedule=schedule)


@pytest.mark.parametrize("K,dtype,schedule", [(32, "bf16", "tree"), (32, "f16", "tree"), (16, "bf16", "tree"),
                                              (16, "f16", "tree"), (16, "f32", "tree"), (32, "bf16", "chain"),
                                              (16, "f32", "chain"), (48, "bf16", "tree"), (64, "f16", "tree"),
                                              (40, "bf16", "chain")])
def test_short_random_segments(gpu, K, dtype, schedule):
    """Hundreds of segments of 1..8 i.i.d. N(0,1) elements, plus tiles on
    both sides of the short-tile limit (256 rows): a short random vector is
    where two operands nearly cancel by chance, so coefficients of nodes far
    smaller than their parts are compared here, every (node, segment) of
    them, for the tree and for the chain (whose weights multiply up to K - 1
    coefficients).  16-bit tiles of at most 256 rows take the exact Gram
    sum."""
    rng = np.random.default_rng(4000 + K)
    lengths = [int(x) for x in rng.integers(1, 9, size=600)] + [255, 256, 257, 300, 1000]
    wl = W.random_case(K, lengths, dtype=dtype, seed=K + 7, kind="normal")
    grads = [g.to(gpu) for g in wl.grads]
    wl.grads = grads
    full_check(wl, f"short K={K} {dtype} {schedule}", schedule)


@pytest.mark.parametrize("K,dtype", [(4, "bf16"), (4, "f16"), (32, "bf16"), (32, "f16"), (64, "bf16"), (48, "f16")])
def test_long_near_cancelling_pairs_16bit(gpu, K, dtype):
    """Long segments (tens of thousands of elements, many matrix-core tiles)
    where every odd worker nearly cancels its even neighbour:
    g_{2m+1} = -g_{2m} + 0.01 n.  Each level-1 node is then about 1/100 of
    its operands, and the level-2 merge sees a 1e-4 cancellation: the fp32
    rounding of the matrix cores' 32-row sums alone would move its
    coefficients by about 1e-3.  The walk must flag those pairs, have their
    Gram matrices recomputed exactly, and meet the coefficient gate."""
    lengths = [70000, 33000, 300, 5]
    base = W.random_case(K, lengths, dtype="f32", seed=90 + K, kind="normal")
    grads = []
    for k in range(K):
        g = base.grads[k].double()
        if k % 2 == 1:
            g = -base.grads[k - 1].double() + 0.01 * g
        grads.append(g.float().to({"bf16": torch.bfloat16, "f16": torch.float16}[dtype]).to(gpu))
    wl = W.Workload(K=K, dtype=dtype, seg_offsets=base.seg_offsets, grads=grads, seed=base.seed)
    full_check(wl, f"near-cancelling K={K} {dtype}")


# ---------------------------------------------------------------- edge cases

RAGGED = [1, 3, 8, 9, 0, 8191, 8192, 8193, 20000, 5, 16, 17]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16])
def test_small_K_ragged_segments(gpu, K, dtype):
    wl = W.random_case(K, RAGGED, dtype=dtype, seed=K, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"ragged K={K} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K", [17, 20, 31, 32, 33, 48, 63, 64, 65, 70, 130, 257, 300])
def test_multistage_K(gpu, K, dtype):
    # more than 16 operands: one block of 32 or 64 (at most 32 or 64 16-bit
    # inputs), else blocks of 16 with fp64 block results and carried inputs; K = 130 has
    # stage positions beyond 127; K = 257 and 300 take three stages (blocks
    # of lower blocks' results)
    wl = W.random_case(K, [1, 300, 9, 40000, 8], dtype=dtype, seed=100 + K, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"multistage K={K} {dtype}")


@pytest.mark.parametrize("K,dtype,schedule", [(40, "f16", "tree"), (64, "bf16", "tree"), (33, "bf16", "chain")])
def test_wide_block_many_tiles(gpu, K, dtype, schedule):
    """33 to 64 16-bit inputs: one 64-operand block in the tree (a chain of
    33 takes blocks of 16 in three stages).  A segment of about
    980 tiles (the walk reads its partials in groups of 16 tiles), segments
    of exactly 16, 17 and 33 tiles (group boundaries), a short tile and a
    few rows."""
    lengths = [2_000_000, 16 * 2048, 17 * 2048, 33 * 2048 + 5, 300, 3]
    wl = W.random_case(K, lengths, dtype=dtype, seed=300 + K, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"wide K={K} {dtype} {schedule}", schedule)


@pytest.mark.parametrize("K,dtype,schedule", [(16, "f32", "tree"), (16, "f32", "chain"), (40, "f32", "tree"),
                                              (32, "bf16", "tree"), (12, "f16", "chain"), (9, "f32", "tree")])
def test_long_segment_tile_groups(gpu, K, dtype, schedule):
    """Blocks of up to 32 operands over a segment of 147 tiles: the walk
    reads the sums of groups of 16 tiles, formed by a launch of their own
    (a segment that long, summed by one workgroup tile by tile, would make
    the walk the slowest step of a mid-sized call).  Segments of exactly
    16 and of 18 tiles (group boundaries), a short tile and a few rows; one
    and two stages; both schedules."""
    lengths = [300_000, 16 * 2048, 17 * 2048 + 3, 300, 3]
    wl = W.random_case(K, lengths, dtype=dtype, seed=350 + K, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"tile groups K={K} {dtype} {schedule}", schedule)


@pytest.mark.parametrize("K", [8, 29, 50])
def test_fp16_subnormal_scales(gpu, K):
    wl = W.random_case(K, [3000] * 16 + [7, 1], dtype="f16", seed=11, kind="scaled")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"fp16 scaled K={K}")


@pytest.mark.parametrize("K", [8, 24, 48])
def test_bf16_exponent_extremes(gpu, K):
    """bf16 segments at magnitudes near and past the limits of fp32 products.

    Per-segment scales 2^-120 (bf16 subnormals), 2^-57 and 2^61 (values on
    both sides of the range whose pairwise products are exact in fp32),
    2^-40, 1 and 2^100, plus one segment that mixes 2^-100 and 2^90 values.
    K = 24 runs the 32-operand Gram pass, K = 48 the 64-operand one.
    """
    lengths = [5000, 5000, 5000, 5000, 5000, 5000, 3001]
    scales = [2.0 ** -120, 2.0 ** -57, 2.0 ** -40, 1.0, 2.0 ** 61, 2.0 ** 100]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    grads = []
    for k in range(K):
        g = torch.Generator().manual_seed(900 + k)
        parts = [torch.randn(n, generator=g, dtype=torch.float64) * sc for n, sc in zip(lengths, scales)]
        mixed = torch.randn(lengths[-1], generator=g, dtype=torch.float64)
        mixed[::2] *= 2.0 ** -100
        mixed[1::2] *= 2.0 ** 90
        parts.append(mixed)
        grads.append(torch.cat(parts).to(torch.bfloat16))
    wl = W.Workload(K=K, dtype="bf16", seg_offsets=off, grads=[x.to(gpu) for x in grads], seed=900)
    got, ref, _ = full_check(wl, f"bf16 exponent extremes K={K}")
    for s in range(len(lengths)):
        lo, hi = off[s], off[s + 1]
        err = rel_l2(got[lo:hi], ref["out_rounded"][lo:hi])
        assert err <= TOL["bf16"], f"segment {s}: relative L2 {err:.3g}"


def test_zero_workers(gpu):
    wl = W.random_case(8, [100, 1, 9000, 33], dtype="bf16", seed=12, zero_workers=(0, 3, 4, 5))
    wl.grads = [g.to(gpu) for g in wl.grads]
    got, ref, _ = full_check(wl, "zero workers")
    allzero = W.random_case(4, [50, 7], seed=13, zero_workers=(0, 1, 2, 3))
    allzero.grads = [g.to(gpu) for g in allzero.grads]
    out, coeffs, stats = run_gpu(allzero)
    assert torch.count_nonzero(out) == 0
    assert torch.all(coeffs == 1.0) and torch.all(stats == 0.0)


def test_antiparallel_pair_is_exactly_zero(gpu):
    A = _A()
    g = torch.randn(10000, generator=torch.Generator().manual_seed(5)).to(gpu)
    out, coeffs = A.combine([g, -g], [0, 10000], return_coeffs=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    assert torch.all(coeffs == 1.5)


def test_orthogonal_supports_give_exact_sum(gpu):
    A = _A()
    n = 4096
    gs = []
    for k in range(4):
        x = torch.zeros(n)
        x[k * 1000:(k + 1) * 1000] = torch.randn(1000, generator=torch.Generator().manual_seed(k))
        gs.append(x.to(gpu))
    out = A.combine(gs, [0, n])
    torch.cuda.synchronize()
    assert torch.equal(out, gs[0] + gs[1] + gs[2] + gs[3])


@pytest.mark.parametrize("K", [2, 5, 16])
def test_identical_inputs_return_input_exactly(gpu, K):
    A = _A()
    g = torch.randn(12345, generator=torch.Generator().manual_seed(K)).to(gpu)
    out = A.combine([g] * K, [0, 100, 12345])
    torch.cuda.synchronize()
    assert torch.equal(out, g)


def test_no_segments_and_empty_segments(gpu):
    A = _A()
    e = torch.empty(0, device=gpu)
    out = A.combine([e, e, e], [0])
    assert out.numel() == 0
    out, coeffs, stats = A.combine([e, e, e], [0, 0, 0], return_coeffs=True, return_stats=True)
    torch.cuda.synchronize()
    assert coeffs.shape == (2, 2, 2) and torch.all(coeffs == 1.0) and torch.all(stats == 0.0)


def test_deterministic_across_runs_and_streams(gpu):
    A = _A()
    wl = W.random_case(16, [70000, 12345, 3, 200000], dtype="f32", seed=21, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    first = A.combine(grads, wl.seg_offsets, return_coeffs=True)
    second = A.combine(grads, wl.seg_offsets, return_coeffs=True)
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        third = A.combine(grads, wl.seg_offsets, return_coeffs=True)
    torch.cuda.synchronize()
    for x, y in ((first, second), (first, third)):
        assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])
    cached = A.combine_cached(grads, wl.seg_offsets)
    torch.cuda.synchronize()
    assert torch.equal(cached, first[0])


def test_stacked_tensor_input_and_out_argument(gpu):
    A = _A()
    wl = W.random_case(4, [1000, 24], dtype="f32", seed=31)
    stacked = torch.stack(wl.grads).to(gpu)  # rows of 1024 fp32: 16-byte aligned
    out = torch.empty(1024, device=gpu)
    res = A.combine(stacked, wl.seg_offsets, out=out)
    torch.cuda.synchronize()
    assert res.data_ptr() == out.data_ptr()
    ref = A.combine([g.to(gpu) for g in wl.grads], wl.seg_offsets)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


# ---------------------------------------------------------------- chain, orthogonality, plain sum

@pytest.mark.parametrize("K,dtype,lengths,seed", [
    (214, "bf16", [21541, 1, 1349, 55375, 15491, 231, 7], 77066),
    (361, "f16", [1, 2468, 43085, 4142, 88], 77209),
])
def test_long_chain_one_element_segments(gpu, K, dtype, lengths, seed):
    """In a one-element segment every merge is of parallel operands, so the
    chain's running value wanders towards zero now and then; a stage's
    quadratic forms then cancel by the square of that ratio, and Gram entries
    rounded to fp64 once moved coefficients by up to 5e-6 (found by a seeded
    random sweep).  Short tiles keep their entries in double-double."""
    wl = W.random_case(K, lengths, dtype=dtype, seed=seed, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"long chain K={K} {dtype}", "chain")


@pytest.mark.parametrize("K,dtype,schedule,seed", [
    (62, "bf16", "chain", 310050), (64, "f16", "chain", 310051), (48, "bf16", "chain", 310052),
    (64, "bf16", "tree", 310050), (32, "f16", "chain", 310053),
])
def test_chain_of_widely_scaled_scalars(gpu, K, dtype, schedule, seed):
    """One-element segments of 16-bit inputs: i.i.d. normal values, each
    segment scaled by its own factor in [1e-6, 1].  Each merge averages two
    parallel values, and where the new input is much smaller than the
    running result, the update of the result's squared norm cancels about
    three quarters of its terms.  A 62-input chain walked as one 64-operand
    block amplified its double-double rounding to a 1.1e-4 coefficient error
    at the last merge (case 310050 of a seeded sweep), and 32-operand chains
    reached 4e-2 on other seeds.  Chains now take blocks of 16 operands
    whatever the dtype.  The tree's six levels are checked alongside."""
    wl = W.random_case(K, [9, 1, 5, 1, 2], dtype=dtype, seed=seed, kind="scaled")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"scaled scalars K={K} {dtype} {schedule}", schedule)


def scalar_chain_case(case):
    """The shape seeded sweep case ``case`` of chains over short segments
    draws: dtype, K (2..64 for 16-bit inputs, 2..39 for fp32), schedule
    (chain three times in four) and 50-300 segments of 1-4 i.i.d. N(0,1)
    values."""
    rng = np.random.default_rng(case)
    dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
    K = int(rng.integers(2, 65)) if dtype != "f32" else int(rng.integers(2, 40))
    schedule = "chain" if rng.random() < 0.75 else "tree"
    lengths = [int(x) for x in rng.integers(1, 5, size=int(rng.integers(50, 300)))]
    return K, dtype, schedule, lengths


# sweep cases whose chains missed the coefficient gate (1.2e-4, 1.6e-3, 4.2e-2) in blocks of 32 or 64,
# and 40 more seeds of the same sweep
@pytest.mark.parametrize("case", [400022, 400045, 400249] + list(range(420000, 420040)))
def test_chains_over_short_random_segments(gpu, case):
    K, dtype, schedule, lengths = scalar_chain_case(case)
    wl = W.random_case(K, lengths, dtype=dtype, seed=case, kind="normal")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"short-segment chain case {case} K={K} {dtype} {schedule}", schedule)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K", [2, 3, 5, 16, 17, 32, 33, 40, 100, 300])
def test_chain_schedule(gpu, K, dtype):
    # K = 300: twenty stages, each the running result (an fp32 slot) and 15 more inputs
    wl = W.random_case(K, [1, 300, 9, 20000, 8], dtype=dtype, seed=300 + K, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"chain K={K} {dtype}", "chain")


def test_chain_worked_example(gpu):
    # hand-derived linear-chain value (tests/golden/worked_examples.json)
    A = _A()
    g = [torch.tensor(v, dtype=torch.float32, device=gpu) for v in ([1, 0], [1, 1], [0, 2], [-1, 1])]
    out = A.combine(g, [0, 2], schedule="chain")
    torch.cuda.synchronize()
    expect = np.array([94141 / 3023008, 7606071 / 3023008])
    np.testing.assert_allclose(out.double().cpu().numpy(), expect, rtol=1e-6)


@pytest.mark.parametrize("K", [1, 2, 5, 16, 33, 64])
def test_orthogonality_ratio(gpu, K):
    A = _A()
    wl = W.random_case(K, [1, 500, 0, 9000, 7], dtype="f32", seed=400 + K, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    say(f"orthogonality K={K}")
    out, ortho = A.combine(grads, wl.seg_offsets, return_ortho=True)
    torch.cuda.synchronize()
    ref = oracle.orthogonality([g.double().numpy() for g in wl.grads], wl.seg_offsets)
    got = ortho.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))  # the empty segment is NaN
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(got[ok], ref[ok], rtol=1e-5)


def test_orthogonality_closed_forms(gpu):
    A = _A()
    n = 4096
    g = torch.randn(n, generator=torch.Generator().manual_seed(1)).to(gpu)
    _, ortho = A.combine([g] * 64, [0, n], return_ortho=True)   # 64 equal gradients: 1/64
    gs = []
    for k in range(8):                                            # disjoint supports: 1
        x = torch.zeros(n)
        x[k * 512:(k + 1) * 512] = torch.randn(512, generator=torch.Generator().manual_seed(k))
        gs.append(x.to(gpu))
    _, ortho2 = A.combine(gs, [0, n], return_ortho=True)
    z = torch.zeros(n, device=gpu)
    _, ortho3 = A.combine([z, z, z], [0, n], return_ortho=True)  # all zero: undefined
    torch.cuda.synchronize()
    assert abs(float(ortho[0]) - 1 / 64) <= 1e-12
    assert abs(float(ortho2[0]) - 1.0) <= 1e-12
    assert np.isnan(float(ortho3[0]))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 7, 64, 65, 130])
def test_plain_sum_bit_exact(gpu, K, dtype):
    A = _A()
    wl = W.random_case(K, [5, 20001], dtype=dtype, seed=500 + K, kind="scaled")
    grads = [g.to(gpu) for g in wl.grads]
    say(f"plain sum K={K} {dtype}")
    out = A.plain_sum(grads)
    torch.cuda.synchronize()
    ref = oracle.plain_sum([g.double().numpy() for g in wl.grads], out_format=dtype)["out_rounded"]
    got = out.double().cpu().numpy()
    assert np.array_equal(got, ref), f"max |diff| {np.max(np.abs(got - ref))}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 17, 64, 65])
def test_plain_sum_signed_zeros(gpu, K, dtype):
    # a sum of -0 terms is -0 and a mix of -0 and +0 is +0 (IEEE round to
    # nearest), for every operand count: one launch, one batch and a partial
    # one, a full launch, and a second launch continuing from fp64 partials
    A = _A()
    rng = np.random.default_rng(90 + K)
    base = rng.standard_normal((K, 4099)).astype(np.float32)
    base[:, :1000] = -0.0
    base[:, 1000:2000] = 0.0
    base[0, 1000:2000] = -0.0
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    grads = [torch.from_numpy(base[k].copy()).to(tdt) for k in range(K)]
    say(f"plain sum signed zeros K={K} {dtype}")
    out = A.plain_sum([g.to(gpu) for g in grads])
    torch.cuda.synchronize()
    ref = oracle.plain_sum([g.double().numpy() for g in grads], out_format=dtype)["out_rounded"]
    got = out.double().cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.all(np.signbit(got[:1000])) and (K == 1 or not np.any(np.signbit(got[1000:2000])))


def test_single_worker_is_exact_copy(gpu):
    A = _A()
    for dtype in ("f32", "f16", "bf16"):
        wl = W.random_case(1, RAGGED, dtype=dtype, seed=7)
        g = wl.grads[0].to(gpu)
        out = A.combine([g], wl.seg_offsets)
        torch.cuda.synchronize()
        assert torch.equal(out, g)


def test_offsets_beyond_2_pow_31(gpu):
    """K = 2 bf16 with 2^31 + 3500 elements: tiles past 2^31 (64-bit offsets).

    The middle segment (2^31 - 500 elements) holds the same gradient in
    both workers, so Adasum returns it exactly with coefficients 1/2; the
    small segments on either side are checked against the oracle.
    """
    A = _A()
    n0, n1, n2 = 1000, 2 ** 31 - 500, 3000
    off = np.array([0, n0, n0 + n1, n0 + n1 + n2], dtype=np.int64)
    say("offsets beyond 2^31", f"N={int(off[-1])}")
    g = torch.Generator(device=gpu).manual_seed(31)
    a = torch.empty(int(off[-1]), dtype=torch.bfloat16, device=gpu)
    b = torch.empty_like(a)
    a[n0:n0 + n1].normal_(generator=g)
    b[n0:n0 + n1].copy_(a[n0:n0 + n1])
    for t in (a, b):
        t[:n0].normal_(generator=g)
        t[n0 + n1:].normal_(generator=g)
    out, coeffs = A.combine([a, b], off, return_coeffs=True)
    torch.cuda.synchronize()
    assert torch.equal(out[n0:n0 + n1], a[n0:n0 + n1])
    c = coeffs.cpu().numpy()
    assert c[0, 1, 0] == 0.5 and c[0, 1, 1] == 0.5
    for s, (lo, hi) in ((0, (0, n0)), (2, (n0 + n1, int(off[-1])))):
        rows = [a[lo:hi].double().cpu().numpy(), b[lo:hi].double().cpu().numpy()]
        res, cf, _ = oracle.adasum_tree(rows)
        ref = oracle.round_to_format(res, "bf16")
        got = out[lo:hi].double().cpu().numpy()
        assert rel_l2(got, ref) <= TOL["bf16"], f"segment {s}"
        check_coeffs(c[:, s], np.asarray(cf).reshape(-1, 2), f"segment {s}")
    del a, b, out
    torch.cuda.empty_cache()


def test_nan_stays_in_its_segment(gpu):
    A = _A()
    wl = W.random_case(4, [100, 200, 300], seed=61)
    grads = [g.clone().to(gpu) for g in wl.grads]
    grads[2][150] = float("nan")  # inside segment 1
    out = A.combine(grads, wl.seg_offsets)
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.isnan(got[100:300]).all()
    assert not torch.isnan(got[:100]).any() and not torch.isnan(got[300:]).any()
    ref = oracle.combine([g.double().numpy() for g in wl.grads], wl.seg_offsets, out_format="f32")
    for lo, hi in ((0, 100), (300, 600)):
        np.testing.assert_allclose(got[lo:hi].double().numpy(), ref["out_rounded"][lo:hi], rtol=1e-6, atol=1e-7)


def test_fp16_subnormal_results_exact(gpu):
    # disjoint supports: the combine is the exact sum, so subnormal fp16
    # inputs must come back bit for bit (no flush to zero on load or store)
    A = _A()
    n = 2048
    tiny = torch.tensor([2.0 ** -24, 3 * 2.0 ** -24, -(2.0 ** -20), 1023 * 2.0 ** -24], dtype=torch.float16)
    gs = []
    for k in range(2):
        x = torch.zeros(n, dtype=torch.float16)
        x[k * 1024:(k + 1) * 1024] = tiny.repeat(256)
        gs.append(x.to(gpu))
    out = A.combine(gs, [0, n])
    torch.cuda.synchronize()
    assert torch.equal(out, gs[0] + gs[1])
    assert int((out.abs() < 2.0 ** -14).sum()) == n  # every value below the smallest normal: none flushed


def test_host_pointers_rejected_before_any_launch(gpu):
    """Host memory passed as an input or output is refused with ADASUM_EINVAL."""
    import ctypes
    from distributed_sgd_gradient_amd import _native
    lib = _native.lib()
    n = 4096
    a = torch.randn(n, device=gpu)
    b = torch.randn(n, device=gpu)
    out = torch.empty(n, device=gpu)
    host = np.zeros(n, dtype=np.float32)
    pinned = torch.zeros(n, dtype=torch.float32).pin_memory()
    off = np.array([0, n], dtype=np.int64)
    offp = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for bad_in, bad_out, what in ((host.ctypes.data, out.data_ptr(), "grads[1]"),
                                  (b.data_ptr(), pinned.data_ptr(), "out"),
                                  (pinned.data_ptr(), out.data_ptr(), "grads[1]")):
        ptrs = (ctypes.c_void_p * 2)(a.data_ptr(), bad_in)
        rc = lib.adasum_combine(ptrs, 2, offp, 1, 0, ctypes.c_void_p(bad_out), stream)
        assert rc == _native.EINVAL, what
        assert what in lib.adasum_last_error().decode()
    # the library still works afterwards
    ptrs = (ctypes.c_void_p * 2)(a.data_ptr(), b.data_ptr())
    assert lib.adasum_combine(ptrs, 2, offp, 1, 0, ctypes.c_void_p(out.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    ref = oracle.combine([a.double().cpu().numpy(), b.double().cpu().numpy()], off, out_format="f32")["out_rounded"]
    assert rel_l2(out.double().cpu().numpy(), ref) <= TOL["f32"]


def test_concurrent_calls_from_threads(gpu):
    """Four host threads, each on its own stream with its own shape and
    dtype, call the library at the same time through both entry points (the
    caller's workspace and the library's cached one); every result equals the
    single-threaded result bit for bit."""
    import threading

    A = _A()
    cases = [(5, "f32", [1000, 0, 70001]), (16, "f16", [4099, 12, 30000]), (24, "bf16", [77, 50000]),
             (3, "f32", [8193, 8193, 8193])]
    data = []
    for i, (K, dt, lengths) in enumerate(cases):
        wl = W.random_case(K, lengths, dtype=dt, seed=700 + i, kind="shared")
        grads = [g.to(gpu) for g in wl.grads]
        ref = A.combine(grads, wl.seg_offsets)
        data.append((grads, wl.seg_offsets, ref))
    torch.cuda.synchronize()
    say("concurrent: 4 threads x 20 calls")
    errors = []

    def worker(i):
        try:
            grads, off, ref = data[i]
            s = torch.cuda.Stream(device=gpu)
            with torch.cuda.stream(s):
                for r in range(20):
                    out = A.combine(grads, off) if r % 2 == 0 else A.combine_cached(grads, off)
                    s.synchronize()
                    if not torch.equal(out, ref):
                        errors.append((i, r, "differs"))
                        return
        except Exception as e:  # reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=90)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


@pytest.mark.parametrize("K,dtype,lengths", [
    (7, "f32", [1000, 0, 65537, 300]),          # a small combine: Gram pass and one fused launch
    (20, "f32", [300_000, 0, 5000, 3]),         # two stages, tile groups, the walk, exact and refining launches
    (40, "f16", [300_000, 7]),                  # one 64-operand block over tile groups
])
def test_graph_capture_and_replay(gpu, K, dtype, lengths):
    """A prepared combine (plan and workspace made by an earlier call) is
    captured in a graph; each of five replays, with the inputs changed in
    place and eager work and synchronisations in between, equals the eager
    combine of the same inputs bit for bit."""
    A = _A()
    wl = W.random_case(K, lengths, dtype=dtype, seed=808, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    out = torch.empty_like(grads[0])
    step = A.Combiner(grads, wl.seg_offsets, out=out)
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(5):
        for x in grads:
            x.mul_(1.5 if r % 2 == 0 else -0.75)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = A.combine(grads, wl.seg_offsets)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}"


def test_captured_shape_survives_cache_eviction(gpu):
    """A shape used under graph capture stays in the plan cache: after 70
    other shapes (more than the cache's 64) have been planned and run, the
    captured graph still replays to the eager result."""
    A = _A()
    wl = W.random_case(6, [4000, 1, 70001], dtype="f32", seed=811, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    out = torch.empty_like(grads[0])
    step = A.Combiner(grads, wl.seg_offsets, out=out)
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    small = [torch.randn(200, device=gpu) for _ in range(3)]
    for i in range(70):
        A.combine(small, [0, 10 + i, 200])
    torch.cuda.synchronize()
    for x in grads:
        x.mul_(-0.5)
    graph.replay()
    torch.cuda.synchronize()
    ref = A.combine(grads, wl.seg_offsets)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_captured_library_workspace_survives_growth(gpu):
    """adasum_combine's cached workspace, once used under graph capture, is
    not freed when a larger shape on the same stream grows it; the graph
    still replays to the eager result."""
    A = _A()
    wl = W.random_case(5, [3000, 17], dtype="f32", seed=812, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    out = torch.empty_like(grads[0])
    s = torch.cuda.Stream(device=gpu)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        A.combine_cached(grads, wl.seg_offsets, out=out)  # plans the shape and sizes the workspace
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        A.combine_cached(grads, wl.seg_offsets, out=out)
    big = W.random_case(20, [200000, 5], dtype="f32", seed=813, kind="shared")
    big_grads = [g.to(gpu) for g in big.grads]
    with torch.cuda.stream(s):
        A.combine_cached(big_grads, big.seg_offsets)  # a larger workspace on the same stream
    s.synchronize()
    for x in grads:
        x.mul_(2.0).add_(1.0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ref = A.combine(grads, wl.seg_offsets)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_prepared_combiner_matches_combine(gpu):
    """Combiner marshals once; every call reads the buffers' current contents."""
    A = _A()
    wl = W.random_case(5, RAGGED, dtype="f32", seed=77, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    comb = A.Combiner(grads, wl.seg_offsets, return_coeffs=True, return_ortho=True)
    for rep in range(3):
        if rep:
            for g in grads:
                g.mul_(0.5).add_(torch.randn_like(g))
        out = comb()
        ref, coeffs, ortho = A.combine(grads, wl.seg_offsets, return_coeffs=True, return_ortho=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(comb.coeffs, coeffs)
        assert torch.equal(torch.nan_to_num(comb.ortho, nan=-1.0), torch.nan_to_num(ortho, nan=-1.0))


@pytest.mark.parametrize("case", range(8))
def test_random_shapes(gpu, case):
    """Seeded random shapes: K, dtype, schedule and ragged segment lengths
    (empty and length-1 segments included) against the oracle."""
    rng = np.random.default_rng(4000 + case)
    K = int(rng.integers(1, 49))
    dtype = ["f32", "f16", "bf16"][case % 3]
    schedule = "chain" if case % 4 == 3 else "tree"
    nseg = int(rng.integers(1, 12))
    lengths = [int(x) for x in np.floor(np.exp(rng.uniform(0, np.log(60000), size=nseg)))]
    lengths[int(rng.integers(0, nseg))] = 0
    wl = W.random_case(K, lengths, dtype=dtype, seed=4000 + case, kind="shared")
    wl.grads = [g.to(gpu) for g in wl.grads]
    full_check(wl, f"random case {case}: lengths={lengths}", schedule)


@pytest.mark.parametrize("chunk", range(20))
def test_seeded_random_sweep(gpu, chunk):
    """300 seeded random shapes, in twenty chunks of 15: K log-uniform in [1, 400), all
    three dtypes, tree and chain, i.i.d. / shared-component / per-segment
    scaled values, values at the edges of the format (fp16 subnormals, bf16
    near 2^-100 and 2^60) or worker pairs that nearly cancel (relative gap
    log-uniform in [1e-7, 1e-1]), some all-zero workers, and segments from
    empty through one element to 60,000 rows.  Every output and every coefficient away
    from the zero discontinuity is compared with the oracle; all failures
    are reported together.  (A wider sweep of this kind found the two
    stage-boundary errors that the one-element chain tests above pin.)"""
    A = _A()
    bad = []
    for case in range(15 * chunk, 15 * chunk + 15):
        rng = np.random.default_rng(91000 + case)
        K = int(np.exp(rng.uniform(0, np.log(400))))
        dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
        schedule = "chain" if rng.random() < 0.4 else "tree"
        kind = ["normal", "shared", "scaled", "edge", "cancel"][int(rng.integers(0, 5))]
        lengths = []
        for _ in range(int(rng.integers(1, 9))):
            u = rng.random()
            lo, hi = (0, 1) if u < 0.05 else (1, 9) if u < 0.30 else (9, 300) if u < 0.55 else \
                (300, 5000) if u < 0.80 else (5000, 60000)
            lengths.append(int(rng.integers(lo, hi)))
        while K * max(sum(lengths), 1) > 2e7:
            lengths = [n // 2 for n in lengths]
        zero = tuple(sorted(set(rng.integers(0, K, size=int(rng.integers(1, 4))).tolist()))) \
            if rng.random() < 0.1 else ()
        if kind == "cancel":  # worker pairs cancelling to eps, eps log-uniform in [1e-7, 1e-1]
            eps = float(np.exp(rng.uniform(np.log(1e-7), np.log(1e-1))))
            wl = W.cancelling_pairs(K, lengths, eps, dtype=dtype, seed=91000 + case)
        else:
            wl = W.random_case(K, lengths, dtype=dtype, seed=91000 + case,
                               kind="normal" if kind == "edge" else kind, zero_workers=zero)
        if kind == "edge":  # exact power-of-two scaling into the format's edge ranges, then rounded to dtype
            scale = {"f32": 2.0 ** -120, "f16": 2.0 ** -20, "bf16": 2.0 ** (-100 if case % 2 else 60)}[dtype]
            wl.grads = [(g.double() * scale).to(g.dtype) for g in wl.grads]
        wl.grads = [g.to(gpu) for g in wl.grads]
        ev = evaluate(wl, schedule)
        if not passes(ev, dtype):
            bad.append((case, K, dtype, schedule, kind, lengths, zero, ev["rel_l2"], ev["seg_ratio"],
                        ev["coeff_err"]))
    say("seeded sweep", f"cases {15 * chunk}..{15 * chunk + 14}: {len(bad)} failures")
    assert not bad, bad


@pytest.mark.parametrize("chunk", range(4))
def test_many_segments_sweep(gpu, chunk):
    """20 seeded shapes (four chunks of 5) of 100 to 5,000 segments each (lengths log-uniform
    in [1, 10,000], a few empty), K from 2 to 20, all dtypes, both schedules:
    every output and coefficient against the oracle."""
    A = _A()
    bad = []
    for case in range(5 * chunk, 5 * chunk + 5):
        rng = np.random.default_rng(93000 + case)
        K = int(rng.integers(2, 21))
        dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
        schedule = "chain" if rng.random() < 0.4 else "tree"
        kind = ["normal", "shared", "scaled"][int(rng.integers(0, 3))]
        nseg = int(np.exp(rng.uniform(np.log(100), np.log(5000))))
        lengths = np.floor(np.exp(rng.uniform(0, np.log(10000), size=nseg))).astype(int)
        lengths[rng.random(nseg) < 0.03] = 0
        lengths = lengths.tolist()
        while K * max(sum(lengths), 1) > 3e7:
            lengths = [n // 2 for n in lengths]
        wl = W.random_case(K, lengths, dtype=dtype, seed=93000 + case, kind=kind)
        wl.grads = [g.to(gpu) for g in wl.grads]
        ev = evaluate(wl, schedule)
        if not passes(ev, dtype):
            bad.append((case, K, dtype, schedule, kind, nseg, ev["rel_l2"], ev["seg_ratio"], ev["coeff_err"]))
    say("many-segment sweep", f"cases {5 * chunk}..{5 * chunk + 4}: {len(bad)} failures")
    assert not bad, bad
