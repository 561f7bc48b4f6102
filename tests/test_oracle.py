"""Pins for the CPU oracle.

Each test checks the oracle against something other than itself: values
worked by hand from the definition (tests/golden/), closed forms the text
states in prose, an exact rational brute force, NumPy's own IEEE casts, or an
algebraic invariant.  The checks are chosen so that a plausible slip in the
oracle (swapped denominators, a wrong sign, a wrong pairing order, a dropped
carry, a segment leak, a wrong rounding mode) fails at least one of them.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
from oracle.rounding import round_to_format

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_golden_exact(ex):
    vecs = [[Fraction(v) for v in vec] for vec in ex["inputs"]]
    fn = exact.adasum_tree if ex["schedule"] == "tree" else exact.adasum_chain
    res, coeffs, _ = fn(vecs)
    assert res == [Fraction(v) for v in ex["result"]]
    assert [(ca, cb) for ca, cb in coeffs] == [(Fraction(a), Fraction(b)) for a, b in ex["coeffs"]]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_golden_fp64(ex):
    vecs = [np.array([float(Fraction(v)) for v in vec]) for vec in ex["inputs"]]
    fn = oracle.adasum_tree if ex["schedule"] == "tree" else oracle.adasum_chain
    res, coeffs, _ = fn(vecs)
    np.testing.assert_allclose(res, [float(Fraction(v)) for v in ex["result"]], rtol=1e-14, atol=1e-15)
    for (ca, cb), (ga, gb) in zip(coeffs, ex["coeffs"]):
        assert abs(ca - float(Fraction(ga))) <= 1e-14 and abs(cb - float(Fraction(gb))) <= 1e-14


def test_tree_and_chain_differ():
    # the operator is not associative: the pairing order matters
    g = [np.array(v, dtype=float) for v in ([1, 0], [1, 1], [0, 2], [-1, 1])]
    t, _, _ = oracle.adasum_tree(g)
    c, _, _ = oracle.adasum_chain(g)
    assert np.max(np.abs(t - c)) > 0.1


# ---------------------------------------------------------------- properties from the text

def test_orthogonal_inputs_sum():
    rng = np.random.default_rng(1)
    for K in (2, 3, 5, 8, 16):
        q, _ = np.linalg.qr(rng.standard_normal((40, K)))
        vecs = [q[:, k] * rng.uniform(0.1, 10.0) for k in range(K)]
        res, coeffs, _ = oracle.adasum_tree(vecs)
        np.testing.assert_allclose(res, np.sum(vecs, axis=0), rtol=0, atol=1e-12)
        assert oracle.orthogonality(vecs, [0, 40])[0] == pytest.approx(1.0, abs=1e-12)


def test_parallel_pair_average_any_norms():
    rng = np.random.default_rng(2)
    u = rng.standard_normal(17)
    for lam, mu in ((1.0, 2.0), (3.0, -0.5), (-2.0, -7.0), (5.0, -5.0), (1e-3, 1e3)):
        res, _, _ = oracle.adasum_pair(lam * u, mu * u)
        np.testing.assert_allclose(res, 0.5 * (lam + mu) * u, rtol=1e-12, atol=1e-12)


def test_identical_inputs_return_input():
    rng = np.random.default_rng(3)
    g = rng.standard_normal(33)
    for K in (1, 2, 3, 4, 7, 16, 64):
        res, _, _ = oracle.adasum_tree([g] * K)
        np.testing.assert_allclose(res, g, rtol=1e-13, atol=1e-14)
    # the orthogonality ratio of K equal gradients is 1/K (1/64 at K = 64)
    assert oracle.orthogonality([g] * 64, [0, 33])[0] == pytest.approx(1 / 64, rel=1e-12)


def test_mean_of_two_sequential_orders():
    # Emulating b1 then b2 scales g2 by (1 - g1.g2/|g2|^2); the other order
    # scales g1 by (1 - g1.g2/|g1|^2); the operator is the mean of the two.
    rng = np.random.default_rng(4)
    for _ in range(20):
        g1, g2 = rng.standard_normal(9), rng.standard_normal(9) + 0.5
        d = g1 @ g2
        s12 = g1 + (1 - d / (g2 @ g2)) * g2
        s21 = g2 + (1 - d / (g1 @ g1)) * g1
        res, _, _ = oracle.adasum_pair(g1, g2)
        np.testing.assert_allclose(res, 0.5 * (s12 + s21), rtol=1e-12, atol=1e-12)


def test_zero_norm_is_plain_sum():
    b = np.array([1.0, -2.0, 3.5])
    z = np.zeros(3)
    res, cf, _ = oracle.adasum_pair(z, b)
    assert np.array_equal(res, b) and cf == (1.0, 1.0)
    res, cf, _ = oracle.adasum_pair(b, z)
    assert np.array_equal(res, b) and cf == (1.0, 1.0)
    res, cf, _ = oracle.adasum_pair(z, z)
    assert np.array_equal(res, z) and cf == (1.0, 1.0)


def test_not_elementwise():
    # changing one coordinate of one input changes the other coordinates of
    # the result, which an elementwise reduction could never do
    a = np.array([1.0, 2.0, 3.0])
    b = np.array([0.5, -1.0, 2.0])
    r0, _, _ = oracle.adasum_pair(a, b)
    a2 = a.copy()
    a2[0] += 1.0
    r1, _, _ = oracle.adasum_pair(a2, b)
    assert np.all(np.abs(r1[1:] - r0[1:]) > 1e-6)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("K", range(1, 9))
def test_fp64_matches_exact_bruteforce(K):
    rng = np.random.default_rng(100 + K)
    for trial in range(6):
        n = int(rng.integers(1, 7))
        vecs = [rng.integers(-4, 5, size=n).astype(float) for _ in range(K)]
        if trial == 0 and K >= 2:
            vecs[1] = np.zeros(n)
        res, cf, st = oracle.adasum_tree(vecs)
        eres, ecf, est = exact.adasum_tree(vecs)
        scale = max(1.0, max(abs(float(v)) for v in eres))
        for x, e in zip(res, eres):
            assert abs(x - float(e)) <= 1e-13 * scale
        for (ca, cb), (ea, eb) in zip(cf, ecf):
            assert abs(ca - float(ea)) <= 1e-13 * max(1, abs(float(ea)))
            assert abs(cb - float(eb)) <= 1e-13 * max(1, abs(float(eb)))
        for i, ((d, A, B), (ed, eA, eB)) in enumerate(zip(st, est)):
            if i < K // 2:  # level 1 sees the integer inputs: exact
                assert (d, A, B) == (float(ed), float(eA), float(eB))
            for x, e in ((d, ed), (A, eA), (B, eB)):
                assert abs(x - float(e)) <= 1e-13 * max(1.0, abs(float(eA)), abs(float(eB)))


@pytest.mark.parametrize("K", [2, 3, 5, 8])
def test_chain_matches_exact_bruteforce(K):
    rng = np.random.default_rng(200 + K)
    vecs = [rng.integers(-3, 4, size=4).astype(float) for _ in range(K)]
    res, _, _ = oracle.adasum_chain(vecs)
    eres, _, _ = exact.adasum_chain(vecs)
    np.testing.assert_allclose(res, [float(e) for e in eres], rtol=1e-13, atol=1e-13)


def test_tree_schedule_shape():
    sched = oracle.tree_schedule(6)
    # 6 -> 3 nodes; 3 -> 1 node + carry; 2 -> 1 node
    assert [len(l) for l in sched] == [3, 1, 1]
    assert sched[0] == [(("leaf", 0), ("leaf", 1)), (("leaf", 2), ("leaf", 3)), (("leaf", 4), ("leaf", 5))]
    assert sched[1] == [(("node", 0), ("node", 1))]
    assert sched[2] == [(("node", 3), ("node", 2))]
    assert sum(len(l) for l in oracle.tree_schedule(37)) == 36
    assert oracle.tree_schedule(1) == []


# ---------------------------------------------------------------- invariants

def test_operand_input_norms_hand_derived():
    """Inputs with squared norms 1, 4, 9, 16, 25 (g_k = (k + 1) e_0, k = 0..4).
    Tree: (g0, g1) -> n0, (g2, g3) -> n1, g4 carried; (n0, n1) -> n2, g4
    carried; (n2, g4) -> n3.  So the operand sums are n0 (1, 4), n1 (9, 16),
    n2 (1 + 4, 9 + 16), n3 (1 + 4 + 9 + 16, 25).  Chain over the first four:
    (g0, g1), (g0..g1, g2), (g0..g2, g3) -> (1, 4), (5, 9), (14, 16)."""
    vecs = [np.array([k + 1.0, 0.0]) for k in range(5)]
    tree = oracle.operand_input_norms(vecs, "tree")
    assert tree.tolist() == [[1.0, 4.0], [9.0, 16.0], [5.0, 25.0], [30.0, 25.0]]
    chain = oracle.operand_input_norms(vecs[:4], "chain")
    assert chain.tolist() == [[1.0, 4.0], [5.0, 9.0], [14.0, 16.0]]
    assert oracle.operand_input_norms(vecs[:1], "tree").shape == (0, 2)
    # the root's two sums cover every input once, whatever K
    rng = np.random.default_rng(11)
    for K in range(2, 12):
        v = [rng.standard_normal(7) for _ in range(K)]
        total = sum(float(x @ x) for x in v)
        for sched in ("tree", "chain"):
            root = oracle.operand_input_norms(v, sched)[-1]
            assert abs(root.sum() - total) <= 1e-12 * total


UNSTABLE = 1e-7  # a tenth of the coefficient tolerance


def _unstable(vals, sched, trials=3):
    rows = [np.atleast_1d(np.asarray(v, dtype=np.float64)) for v in vals]
    st = oracle.stability(rows, [0, rows[0].size], sched, trials=trials)
    return (st["coeff_motion"][:, 0] > UNSTABLE).tolist(), st


def test_stability_hand_derived():
    """Scalars 1, -1 make the exactly zero node n0 = Adasum(1, -1) = 3/2 - 3/2;
    one-ulp noise makes it a tiny nonzero scalar, and for scalars Adasum(a, b)
    is (a + b) / 2 unless a is exactly zero, when it is b.  Tree of
    (1, -1, 2, 3): n2 = (n0, n1), so only n2's left coefficient moves (its
    right one stays 1 - n0 n1 / (2 n1^2)).  Tree of (1, -1, 2, 3, 4, 5, 6, 7):
    n4 = (n0, n1) moves on the left, and n6 = (n4, n5), whose operand n4 jumps
    from n1 to about n1 / 2, on both sides.  Chain of (1, -1, 2, 3): n1 =
    (n0, 2) on the left, then n2 = (n1, 3) on both.  Inputs with no
    cancellation move nothing; all-zero inputs stay exactly zero (their
    coefficients are exactly 1)."""
    assert _unstable([1, -1, 2, 3], "tree")[0] == [[False, False], [False, False], [True, False]]
    m8 = _unstable([1, -1, 2, 3, 4, 5, 6, 7], "tree")[0]
    assert m8 == [[False, False]] * 4 + [[True, False], [False, False], [True, True]]
    assert _unstable([1, -1, 2, 3], "chain")[0] == [[False, False], [True, False], [True, True]]
    assert not np.any(_unstable([1, 2, 3, 4, 5], "tree")[0])
    m, st = _unstable([0, 0, 0, 0], "tree")
    assert not np.any(m) and np.all(st["coeff_motion"] == 0.0) and np.all(st["base"]["coeffs"] == 1.0)


@pytest.mark.parametrize("sched", ["tree", "chain"])
def test_operand_input_norms_equal_operand_norms_for_orthogonal_inputs(sched):
    """Orthogonal inputs are summed, so every operand of every node is the
    plain sum of the inputs under it and its squared norm (the walk's own
    |a|^2 and |b|^2) equals the summed squared norms of those inputs."""
    rng = np.random.default_rng(12)
    for K in (2, 3, 5, 8, 11, 16, 17):
        q, _ = np.linalg.qr(rng.standard_normal((24, K)))
        vecs = [q[:, k] * rng.uniform(0.1, 10.0) for k in range(K)]
        fn = oracle.adasum_chain if sched == "chain" else oracle.adasum_tree
        _, _, st = fn(vecs)
        got = oracle.operand_input_norms(vecs, sched)
        np.testing.assert_allclose(got, np.asarray(st)[:, 1:3], rtol=1e-12)


@pytest.mark.parametrize("sched,K", [("tree", 8), ("tree", 13), ("chain", 6)])
def test_stability_marks_exactly_the_coefficients_that_jump(sched, K):
    """Inputs 2 and 3 (tree) or 0 and 1 (chain) are u and -u, whose merge is
    exactly zero (coefficient 1 above it).  Replacing -u by -(1 + 1e-6) u
    leaves a tiny nonzero merge.  A coefficient that depends continuously on
    the inputs moves by O(1e-6) (here at most 7e-7); the consumer's
    coefficient of the tiny operand and both coefficients of every node above
    it jump by O(1) in the geometry of the inputs (here at least 2.7e-3 in 4
    dimensions).  At the exact zero, one-ulp noise moves exactly the
    coefficients that jump.  Once perturbed, the tiny operand (|a|^2 about
    1e-12 of its inputs) is resolved by fp64 arithmetic: its coefficients are
    well defined there, and noise moves none of them."""
    rng = np.random.default_rng(13)
    vecs = [rng.standard_normal(4) for _ in range(K)]
    i = 2 if sched == "tree" else 0
    fn = oracle.adasum_chain if sched == "chain" else oracle.adasum_tree
    vecs[i + 1] = -vecs[i]
    _, c0, _ = fn(vecs)
    pert = list(vecs)
    pert[i + 1] = -(1.0 + 1e-6) * vecs[i]
    _, c1, _ = fn(pert)
    c0, c1 = np.asarray(c0), np.asarray(c1)
    jumped = np.abs(c1 - c0) > 3e-5 * np.maximum(1.0, np.abs(c0))
    assert jumped.sum() >= 3
    m0 = oracle.stability(vecs, [0, 4], sched, trials=3)["coeff_motion"][:, 0] > UNSTABLE
    np.testing.assert_array_equal(m0, jumped)
    m1 = oracle.stability(pert, [0, 4], sched, trials=3)["coeff_motion"][:, 0] > UNSTABLE
    assert not m1.any()


def test_stability_keeps_exact_zeros():
    """Zeros are exact data, not rounding: all-zero workers and an all-zero
    segment stay exactly zero under the noise, so their coefficients (exactly
    1) and that segment's output (exactly 0) do not move at all, while the
    other coefficients move by rounding only."""
    rng = np.random.default_rng(31)
    vecs = [rng.standard_normal(40) for _ in range(8)]
    for k in (0, 3):
        vecs[k][:] = 0.0
    for v in vecs:
        v[30:] = 0.0  # segment 1, [30, 40), is zero in every worker
    st = oracle.stability(vecs, [0, 30, 40], "tree", trials=3)
    c = st["base"]["coeffs"]
    assert np.all(c[:, 1] == 1.0) and np.all(st["coeff_motion"][:, 1] == 0.0)
    assert st["output_motion"][1] == 0.0
    zero_operand = c[:, 0] == 1.0
    assert zero_operand.sum() >= 2 and np.all(st["coeff_motion"][:, 0][zero_operand] == 0.0)
    assert 0.0 < float(st["coeff_motion"][:, 0].max()) < 1e-12


@pytest.mark.parametrize("vals", [[7, 0, -7, 1, 3, -7, 0, -2, 3, 3, -8],
                                  [0, 6, -4, 1, 3, -2, -6, 0, -7, 3, 1, 3]])
def test_stability_treats_rounding_residues_as_zero(vals):
    """Scalars at fp16's subnormal scale (multiples of 2^-24) whose trees
    have operands that are exactly zero in exact arithmetic (the Fraction
    oracle) but rounding residues of a few 1e-45 in fp64, about 1e-32 of the
    inputs under them.  Their coefficients are garbage on any fp64 path, and
    the nodes above inherit that however stable it is under noise; below
    ZERO_FLOOR they count as zero.  The coefficients marked as not determined
    at the discontinuity are exactly: the consumer's coefficient of every
    operand that is zero in exact arithmetic over inputs that are not all
    zero, and both coefficients of every node above it; and the output."""
    from fractions import Fraction

    from oracle import exact

    rows = [np.array([v * 2.0 ** -24]) for v in vals]
    _, _, st = oracle.adasum_tree(rows)
    _, _, st_exact = exact.adasum_tree([[Fraction(v, 2 ** 24)] for v in vals])
    opn = oracle.operand_input_norms(rows, "tree")
    exact_zero = (np.array([[s[1] == 0, s[2] == 0] for s in st_exact])) & (opn > 0)
    residue = exact_zero & (np.asarray(st)[:, 1:3] > 0)
    assert residue.any()  # fp64 left a nonzero residue where the exact value is zero
    parents = oracle.node_parents(len(vals) - 1, "tree")
    expect = exact_zero.copy()
    for i in np.flatnonzero(exact_zero.any(axis=1)):
        j = parents[i]
        while j >= 0:
            expect[j] = True
            j = parents[j]
    res = oracle.stability(rows, [0, 1], "tree")
    np.testing.assert_array_equal(np.isinf(res["coeff_motion"][:, 0]), expect)
    assert np.isinf(res["output_motion"][0])


def _planted(eps, K=4, n=300, seed=21):
    """Tree inputs with g1 = -(1 + eps) g0 + eps v: the level-1 node (g0, g1)
    is about eps of its operands, so the merge above sees |a|^2 / S of about
    2.25 eps^2."""
    rng = np.random.default_rng(seed)
    vecs = [rng.standard_normal(n) for _ in range(K)]
    vecs[1] = -(1.0 + eps) * vecs[0] + eps * vecs[1]
    return vecs


@pytest.mark.parametrize("eps2", [1e-10, 1e-12, 1e-14])
def test_resolved_cancellations_are_stable(eps2):
    """Planted cancellations with eps^2 = 1e-10, 1e-12, 1e-14: one-ulp noise
    on every input element moves the oracle's coefficients above them by less
    than 1e-8 of max(1, |c|), so every one of them is gated."""
    vecs = _planted(np.sqrt(eps2))
    _, _, st = oracle.adasum_tree(vecs)
    ratio = st[2][1] / oracle.operand_input_norms(vecs, "tree")[2][0]
    assert 1.0 * eps2 < ratio < 5.0 * eps2
    motion = oracle.stability(vecs, [0, 300], "tree", trials=4)["coeff_motion"]
    assert float(motion.max()) < 1e-8


def test_unresolved_cancellations_are_unstable():
    """Below the floor fp64 rounding decides the coefficient: with
    eps^2 = 1e-22 one-ulp noise moves the coefficient of the tiny operand by
    more than 1e-7 of it, and nothing else in the two-level tree."""
    motion = oracle.stability(_planted(1e-11), [0, 300], "tree", trials=4)["coeff_motion"][:, 0]
    assert (motion > UNSTABLE).tolist() == [[False, False], [False, False], [True, False]]


def test_stability_covers_every_coefficient_the_oracle_gets_wrong():
    """A chain of 40 two-element inputs in cancelling pairs (relative gap
    5e-8): later merges meet operands that are tiny against the inputs under
    them, with coefficients far from 1, and the fp64 oracle's own rounding
    moves them.  Against the same chain in 50-digit arithmetic, every
    coefficient the oracle has wrong by more than 1e-7 of max(1, |c|) is one
    that one-ulp noise moves by more than 1e-7 (and some are wrong)."""
    import mpmath as mp

    rng = np.random.default_rng(3)
    vecs = [rng.standard_normal(2) for _ in range(40)]
    for k in range(1, 40, 2):
        vecs[k] = -(1.0 + 5e-8) * vecs[k - 1] + 5e-8 * vecs[k]
    mp.mp.dps = 50
    acc = [mp.mpf(float(x)) for x in vecs[0]]
    ref = []
    for v in vecs[1:]:
        v = [mp.mpf(float(x)) for x in v]
        d = mp.fsum(a * b for a, b in zip(acc, v))
        A, B = mp.fsum(a * a for a in acc), mp.fsum(b * b for b in v)
        ca = mp.mpf(1) if A == 0 else 1 - d / (2 * A)
        cb = mp.mpf(1) if B == 0 else 1 - d / (2 * B)
        ref.append((float(ca), float(cb)))
        acc = [ca * a + cb * b for a, b in zip(acc, v)]
    ref = np.asarray(ref)
    st = oracle.stability(vecs, [0, 2], "chain", trials=3)
    got = st["base"]["coeffs"][:, 0]
    wrong = np.abs(got - ref) / np.maximum(1.0, np.abs(ref)) > UNSTABLE
    assert wrong.any()
    assert np.all(st["coeff_motion"][:, 0][wrong] > UNSTABLE)


def test_symmetry_and_scale_invariance():
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal(50), rng.standard_normal(50)
    r1, (ca, cb), _ = oracle.adasum_pair(a, b)
    r2, (cb2, ca2), _ = oracle.adasum_pair(b, a)
    np.testing.assert_allclose(r1, r2, rtol=1e-14, atol=1e-14)
    assert (ca, cb) == pytest.approx((ca2, cb2), rel=1e-14)
    for s in (1e-6, 3.0, 1e8):
        _, (sa, sb), _ = oracle.adasum_pair(s * a, s * b)
        assert (sa, sb) == pytest.approx((ca, cb), rel=1e-12)


def test_permutation_equivariance_within_segment():
    rng = np.random.default_rng(6)
    vecs = [rng.standard_normal(64) for _ in range(8)]
    perm = rng.permutation(64)
    r, _, _ = oracle.adasum_tree(vecs)
    rp, _, _ = oracle.adasum_tree([v[perm] for v in vecs])
    np.testing.assert_allclose(rp, r[perm], rtol=1e-12, atol=1e-13)


def test_segments_are_independent():
    rng = np.random.default_rng(7)
    off = [0, 10, 10, 35, 36, 80]
    vecs = [rng.standard_normal(80) for _ in range(5)]
    base = oracle.combine(vecs, off)
    pert = [v.copy() for v in vecs]
    pert[2][12:30] += 5.0  # only segment 2 ([10, 35))
    res = oracle.combine(pert, off)
    changed = np.abs(res["out"] - base["out"]) > 0
    assert changed[10:35].any()
    assert not changed[:10].any() and not changed[35:].any()
    # per-segment result equals the tree on that slice alone
    seg, _, _ = oracle.adasum_tree([v[35:36] for v in vecs])
    assert np.array_equal(base["out"][35:36], seg)


def test_emitted_norm_identity():
    # |c|^2 = ca^2 A + 2 ca cb d + cb^2 B, the statistic the next tree level needs
    rng = np.random.default_rng(8)
    a, b = rng.standard_normal(100), rng.standard_normal(100)
    c, (ca, cb), (d, A, B) = oracle.adasum_pair(a, b)
    assert c @ c == pytest.approx(ca * ca * A + 2 * ca * cb * d + cb * cb * B, rel=1e-12)


def test_combine_layout_and_empty_segments():
    rng = np.random.default_rng(9)
    off = [0, 0, 3, 3, 7]
    vecs = [rng.standard_normal(7).astype(np.float32) for _ in range(4)]
    res = oracle.combine(vecs, off, out_format="f32")
    assert res["coeffs"].shape == (3, 4, 2) and res["stats"].shape == (3, 4, 3)
    # an empty segment has zero-norm operands: coefficient 1, statistics 0
    assert np.all(res["coeffs"][:, 0] == 1.0) and np.all(res["stats"][:, 2] == 0.0)
    assert np.array_equal(res["out_rounded"], res["out"].astype(np.float32).astype(np.float64))
    assert oracle.combine(vecs[:1], off)["coeffs"].shape == (0, 4, 2)
    np.testing.assert_array_equal(oracle.combine(vecs[:1], off)["out"], vecs[0].astype(np.float64))
    with pytest.raises(ValueError):
        oracle.combine(vecs, [0, 5, 3, 7])
    with pytest.raises(ValueError):
        oracle.combine(vecs, [0, 3, 6])


def test_plain_sum_exact_order():
    rng = np.random.default_rng(10)
    vecs = [rng.integers(-1000, 1000, size=20).astype(float) for _ in range(6)]
    np.testing.assert_array_equal(oracle.plain_sum(vecs)["out"], np.sum(vecs, axis=0))
    # values spread over 40 binades, where the order of the additions shows:
    # each IEEE addition is the exact sum rounded once, float(Fraction + Fraction)
    vecs = [rng.standard_normal(50) * np.exp2(rng.integers(-20, 20, size=50)) for _ in range(6)]
    want = []
    for j in range(50):
        acc = vecs[0][j]
        for v in vecs[1:]:
            acc = float(Fraction(acc) + Fraction(v[j]))
        want.append(acc)
    got = oracle.plain_sum(vecs)["out"]
    assert got.tolist() == want
    assert oracle.plain_sum(vecs[::-1])["out"].tolist() != want  # the data is order-sensitive


def test_plain_sum_left_to_right_rounding():
    """Worker order decides the fp64 result: 1 + 2^53 is a tie between 2^53
    and 2^53 + 2 and rounds to the even 2^53, so 1 + 2^53 - 2^53 = 0, while
    2^53 - 2^53 + 1 = 1 and -2^53 + 2^53 + 1 = 1."""
    big = 2.0 ** 53
    assert oracle.plain_sum([np.array([1.0]), np.array([big]), np.array([-big])])["out"][0] == 0.0
    assert oracle.plain_sum([np.array([big]), np.array([-big]), np.array([1.0])])["out"][0] == 1.0
    assert oracle.plain_sum([np.array([-big]), np.array([big]), np.array([1.0])])["out"][0] == 1.0


def test_orthogonality_closed_forms():
    """Parallel inputs are averaged, so the pair (u, 3u) gives 2u and the
    ratio |2u|^2 / (|u|^2 + |3u|^2) = 4/10; an anti-parallel pair of equal
    norms gives 0; two orthogonal inputs give 1.  The hand-worked tree of
    four inputs (tests/golden, tree_K4) has result (37/68, 325/136) over
    inputs of squared norms 1, 2, 4, 2: ratio 111101/166464."""
    u = np.array([1.0, -2.0, 0.5])
    assert oracle.orthogonality([u, 3 * u], [0, 3])[0] == pytest.approx(0.4, rel=1e-14)
    assert oracle.orthogonality([u, -u], [0, 3])[0] == 0.0
    assert oracle.orthogonality([np.array([3.0, 0.0]), np.array([0.0, 5.0])], [0, 2])[0] == pytest.approx(1.0, rel=1e-15)
    ex = next(e for e in _golden() if e["name"] == "tree_K4")
    vecs = [np.array([float(Fraction(v)) for v in vec]) for vec in ex["inputs"]]
    want = float(sum(Fraction(v) ** 2 for v in ex["result"]) /
                 sum(Fraction(v) ** 2 for vec in ex["inputs"] for v in vec))
    assert want == pytest.approx(111101 / 166464, rel=1e-15)
    assert oracle.orthogonality(vecs, [0, 2])[0] == pytest.approx(want, rel=1e-14)


def test_orthogonality_zero_segment_nan():
    vecs = [np.zeros(4), np.zeros(4)]
    assert np.isnan(oracle.orthogonality(vecs, [0, 4])[0])


# ---------------------------------------------------------------- rounding

def _edge_values():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(20000) * np.exp(rng.uniform(-120, 120, 20000)),
        rng.standard_normal(20000) * np.exp(rng.uniform(-20, 12, 20000)),
        [0.0, -0.0, 1.0, -1.0, 65504.0, 65520.0, 65519.99, 6e-8, 3e-8, 2.98e-8,
         2.0 ** -149, 2.0 ** -150, 1.5 * 2.0 ** -149, 3.4028235e38, 3.4028236e38,
         np.inf, -np.inf, 1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 1e300, -1e-300],
    ])
    return vals


@pytest.mark.parametrize("fmt,npdt", [("f32", np.float32), ("f16", np.float16)])
def test_rounding_matches_numpy_casts(fmt, npdt):
    x = _edge_values()
    with np.errstate(over="ignore"):
        ref = x.astype(npdt).astype(np.float64)
    got = round_to_format(x, fmt)
    assert np.array_equal(got, ref, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_rounding_bf16_ties_and_library():
    # values exactly representable in fp32: torch's fp32 -> bf16 cast is RNE
    x = _edge_values().astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_to_format(x.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    assert round_to_format(1 + 2.0 ** -8, "bf16") == 1.0
    assert round_to_format(1 + 3 * 2.0 ** -8, "bf16") == 1 + 2.0 ** -6
    # directly from fp64 (no double rounding): just above the tie rounds up
    assert round_to_format(1 + 2.0 ** -8 + 2.0 ** -40, "bf16") == 1 + 2.0 ** -7
    assert round_to_format(3.4e38, "bf16") == np.inf  # beyond bf16's largest finite
    assert round_to_format(2.0 ** -133, "bf16") == 2.0 ** -133  # smallest subnormal
    assert round_to_format(2.0 ** -134, "bf16") == 0.0  # tie to even (zero)
