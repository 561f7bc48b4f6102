"""fp64 NumPy oracle for the Adasum gradient combiner.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Everything is computed in fp64 on the CPU, one segment at a time, in the plain
order of the definitions below.  NumPy's ``dot`` serves as the library
primitive for a dot product; nothing is blocked, fused or reordered.

Page references are to "Scaling Distributed Training with Adaptive
Summation" (arXiv 2006.02924):
  * the pairwise operator is the average of the two emulated sequential SGD
    orders (the derivation that follows Eq. 2: one order scales g2 by a
    scalar, the other order swaps the roles, and the two are averaged);
  * orthogonal inputs give the plain sum and parallel inputs the average
    (the discussion of the operator's properties before Figure 1);
  * the operator is applied per layer, not to the whole gradient (the
    paragraph after Figure 1);
  * more than two gradients are combined by applying the operator
    recursively (the paragraph on extending Adasum to n gradients, and the
    "recursive application" used in practice for bandwidth, Sec. 4);
  * the per-layer orthogonality ratio |Adasum(g_1..g_n)|^2 / sum_i |g_i|^2
    (Figure 1 and its discussion).
"""

import numpy as np

from .rounding import round_to_format


def adasum_pair(a, b):
    """Pairwise Adasum of two fp64 vectors.

    Returns ``(c, (ca, cb), (d, A, B))`` with d = a.b, A = |a|^2, B = |b|^2,
    ca = 1 - d / (2A), cb = 1 - d / (2B) and c = ca*a + cb*b.  An operand with
    zero norm gets coefficient 1, so the pair degenerates to the plain sum
    (the operator is otherwise undefined there).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = float(np.dot(a, b))
    A = float(np.dot(a, a))
    B = float(np.dot(b, b))
    ca = 1.0 if A == 0.0 else 1.0 - d / (2.0 * A)
    cb = 1.0 if B == 0.0 else 1.0 - d / (2.0 * B)
    return ca * a + cb * b, (ca, cb), (d, A, B)


def tree_schedule(K):
    """The fixed binary tree over K leaves, in level-major order.

    Level by level, the current list of vectors is paired left to right:
    (v0, v1), (v2, v3), ...; when the list has odd length its last vector is
    carried unchanged to the next level.  Returns a list of levels; each level
    is a list of ``(left, right)`` operand references, where a reference is
    ``("leaf", k)`` or ``("node", i)`` and node ids count pairs in the order
    they are listed (level 1 first).  K = 1 has no levels.
    """
    if K < 1:
        raise ValueError("K must be >= 1")
    current = [("leaf", k) for k in range(K)]
    levels = []
    next_id = 0
    while len(current) > 1:
        level = []
        nxt = []
        for j in range(len(current) // 2):
            level.append((current[2 * j], current[2 * j + 1]))
            nxt.append(("node", next_id))
            next_id += 1
        if len(current) % 2 == 1:
            nxt.append(current[-1])
        levels.append(level)
        current = nxt
    return levels


def adasum_tree(vectors):
    """Combine K fp64 vectors with the fixed binary tree.

    Returns ``(result, coeffs, stats)``: ``coeffs[i] = (ca, cb)`` and
    ``stats[i] = (d, A, B)`` of node i in level-major order (K - 1 nodes).
    """
    vectors = [np.asarray(v, dtype=np.float64) for v in vectors]
    K = len(vectors)
    nodes = []
    coeffs = []
    stats = []

    def value(ref):
        kind, i = ref
        return vectors[i] if kind == "leaf" else nodes[i]

    for level in tree_schedule(K):
        produced = []
        for left, right in level:
            c, cf, st = adasum_pair(value(left), value(right))
            produced.append(c)
            coeffs.append(cf)
            stats.append(st)
        # nodes of this level become addressable only after the whole level
        nodes.extend(produced)
    result = vectors[0].copy() if K == 1 else nodes[-1]
    return result, coeffs, stats


def adasum_chain(vectors):
    """Linear recursion g[0, n+1] = Adasum(g[0, n], g[n+1]).

    The text first extends the operator to n gradients this way (the
    effective gradient of b_0..b_n meeting b_(n+1)).  Returns
    ``(result, coeffs, stats)`` with one entry per step (K - 1 of them).
    """
    vectors = [np.asarray(v, dtype=np.float64) for v in vectors]
    acc = vectors[0].copy()
    coeffs, stats = [], []
    for v in vectors[1:]:
        acc, cf, st = adasum_pair(acc, v)
        coeffs.append(cf)
        stats.append(st)
    return acc, coeffs, stats


def _check_offsets(seg_offsets, n):
    off = np.asarray(seg_offsets, dtype=np.int64)
    if off.ndim != 1 or off.size < 1 or off[0] != 0 or np.any(np.diff(off) < 0):
        raise ValueError("seg_offsets must start at 0 and be non-decreasing")
    if off[-1] != n:
        raise ValueError("seg_offsets[-1] must equal the vector length")
    return off


def _as_rows(inputs):
    rows = [np.asarray(x, dtype=np.float64).reshape(-1) for x in inputs]
    if not rows:
        raise ValueError("need at least one input")
    n = rows[0].size
    if any(r.size != n for r in rows):
        raise ValueError("all inputs must have the same length")
    return rows, n


def _combine_with(fn, inputs, seg_offsets, out_format):
    rows, n = _as_rows(inputs)
    K = len(rows)
    off = _check_offsets(seg_offsets, n)
    nseg = off.size - 1
    out = np.zeros(n, dtype=np.float64)
    coeffs = np.ones((max(K - 1, 0), nseg, 2), dtype=np.float64)
    stats = np.zeros((max(K - 1, 0), nseg, 3), dtype=np.float64)
    for s in range(nseg):
        lo, hi = int(off[s]), int(off[s + 1])
        res, cf, st = fn([r[lo:hi] for r in rows])
        out[lo:hi] = res
        for i in range(K - 1):
            coeffs[i, s] = cf[i]
            stats[i, s] = st[i]
    result = {"out": out, "coeffs": coeffs, "stats": stats}
    if out_format is not None:
        result["out_rounded"] = round_to_format(out, out_format)
    return result


def combine(inputs, seg_offsets, out_format=None):
    """Per-segment tree Adasum of K equal-length vectors.

    ``inputs`` is a sequence of K 1-D arrays (any real dtype; widened to fp64
    exactly), ``seg_offsets`` the CSR offsets [0, ..., N] of the segments
    (layers).  Each segment is combined on its own.  Returns a dict with
    ``out`` (fp64), ``coeffs`` [K-1, nseg, 2], ``stats`` [K-1, nseg, 3] in
    level-major node order, and ``out_rounded`` (fp64 holding values of
    ``out_format``) when a format name is given.
    """
    return _combine_with(adasum_tree, inputs, seg_offsets, out_format)


def combine_chain(inputs, seg_offsets, out_format=None):
    """Per-segment linear-chain Adasum; same layout as :func:`combine`."""
    return _combine_with(adasum_chain, inputs, seg_offsets, out_format)


def plain_sum(inputs, seg_offsets=None, out_format=None):
    """Synchronous-SGD combination: the plain sum of the K gradients.

    The allreduce that Adasum replaces sums the local gradients (Sec. 2 of
    the text, on synchronous SGD).  Summed in worker order in fp64.
    """
    rows, n = _as_rows(inputs)
    if seg_offsets is not None:
        _check_offsets(seg_offsets, n)
    acc = rows[0].copy()
    for r in rows[1:]:
        acc = acc + r
    result = {"out": acc}
    if out_format is not None:
        result["out_rounded"] = round_to_format(acc, out_format)
    return result


def orthogonality(inputs, seg_offsets):
    """Per-segment ratio |Adasum(g_1..g_K)|^2 / sum_k |g_k|^2 (Figure 1).

    1 for mutually orthogonal inputs, 1/K for K identical inputs.  A segment
    whose inputs are all zero (or that is empty) has an undefined ratio and
    returns NaN.
    """
    rows, n = _as_rows(inputs)
    off = _check_offsets(seg_offsets, n)
    res = combine(rows, off)["out"]
    ratios = np.empty(off.size - 1, dtype=np.float64)
    for s in range(off.size - 1):
        lo, hi = int(off[s]), int(off[s + 1])
        den = sum(float(np.dot(r[lo:hi], r[lo:hi])) for r in rows)
        num = float(np.dot(res[lo:hi], res[lo:hi]))
        ratios[s] = np.nan if den == 0.0 else num / den
    return ratios


def operand_input_norms(vectors, schedule="tree"):
    """Per node, in node order: the summed squared norms of the input vectors
    under its left operand and under its right operand, (S_L, S_R).

    The operator is discontinuous at a zero operand (coefficient 1 there, see
    ``adasum_pair``), so a node whose operand norm |a|^2 is tiny against S_L
    is a near-cancellation at which the coefficient is not a stable quantity.
    ``schedule`` is "tree" (``tree_schedule``) or "chain" (the running result
    meets g_1, g_2, ... in turn).  Returns an array [K-1, 2].
    """
    norms = [float(np.dot(v, v)) for v in (np.asarray(x, dtype=np.float64) for x in vectors)]
    K = len(norms)
    out = []
    if schedule == "chain":
        acc = norms[0] if K else 0.0
        for k in range(1, K):
            out.append((acc, norms[k]))
            acc += norms[k]
    else:
        under = {("leaf", k): norms[k] for k in range(K)}
        node = 0
        for level in tree_schedule(K):
            for left, right in level:
                out.append((under[left], under[right]))
                under[("node", node)] = under[left] + under[right]
                node += 1
    return np.asarray(out, dtype=np.float64).reshape(-1, 2)


def _ulp_noise(rows, rng):
    """Every nonzero finite element moved to an adjacent fp64 value, toward
    or away from zero at random (one unit in the last place: plus or minus 1
    on the bit pattern); zeros (exact data, such as an all-zero worker) stay
    as they are, and so do infinities, NaNs and the largest finite
    magnitudes."""
    big = np.finfo(np.float64).max
    out = []
    for r in rows:
        r = np.ascontiguousarray(r, dtype=np.float64)
        bits = r.view(np.int64)
        coin = np.unpackbits(np.frombuffer(rng.bytes((r.size + 7) // 8), dtype=np.uint8), count=r.size)
        step = coin.astype(np.int64)
        step <<= 1
        step -= 1
        moved = bits + step
        if not (np.isfinite(r).all() and float(np.abs(r).max(initial=0.0)) < big):
            keep = ~np.isfinite(r) | (np.abs(r) == big)
            moved[keep] = bits[keep]
        zero = r == 0.0
        moved[zero] = bits[zero]
        out.append(moved.view(np.float64))
    return out


def node_parents(n_nodes, schedule="tree"):
    """Parent node of every node (-1 for the root), in node order."""
    parent = [-1] * n_nodes
    if schedule == "chain":
        for i in range(n_nodes - 1):
            parent[i] = i + 1
        return parent
    node = 0
    for level in tree_schedule(n_nodes + 1):
        for left, right in level:
            for kind, i in (left, right):
                if kind == "node":
                    parent[i] = node
            node += 1
    return parent


# An operand whose squared norm is at most this fraction of the summed squared
# norms of the input gradients under it is below about 2^-45 of their size, a
# few hundred units of fp64 rounding: to fp64 arithmetic it is zero, whether
# or not the rounding happened to leave it exactly zero.
ZERO_FLOOR = 2.0 ** -90


def stability(inputs, seg_offsets, schedule="tree", trials=2, seed=0):
    """How far this oracle's own results move under rounding-size noise.

    The operator is discontinuous at a zero operand (coefficient 1 there,
    another limit next to it), and under deep cancellation (a node far
    smaller than the inputs under it) fp64 arithmetic no longer determines
    the coefficients above it, nor, in a long chain, the results built on
    them.  This reruns the per-segment combine ``trials`` times, each time
    with every nonzero input element moved by one fp64 ulp in a random
    direction (seeded).  An operand whose squared norm is at most
    ZERO_FLOOR of the inputs under it (which are not all zero) sits at the
    discontinuity itself, whatever the noise does (an exact negation can
    survive it, rounding can absorb it, and a rounding residue can be as
    stable as it is wrong): its consumer's coefficient of it, both
    coefficients of every node above that consumer and the segment's output
    count as not determined.
    Returns

      ``base``           the unperturbed result (as ``combine`` or
                         ``combine_chain`` returns it);
      ``coeff_motion``   [K-1, nseg, 2], the largest
                         |c' - c| / max(1, |c|) over the trials (inf at an
                         exact zero and above it);
      ``output_motion``  [nseg], the largest ||out' - out|| / ||out|| of
                         each segment (0 for an all-zero or empty segment,
                         inf above an exact zero).

    A coefficient or output that moves by a sizeable fraction of its
    tolerance is not determined by the data through fp64 arithmetic, so this
    oracle is no reference for it.
    """
    rows, n = _as_rows(inputs)
    off = _check_offsets(seg_offsets, n)
    fn = combine_chain if schedule == "chain" else combine
    base = fn(rows, off)
    rng = np.random.default_rng(seed)
    nseg = off.size - 1
    cmov = np.zeros_like(base["coeffs"])
    omov = np.zeros(nseg)
    for _ in range(trials):
        res = fn(_ulp_noise(rows, rng), off)
        with np.errstate(invalid="ignore"):
            d = np.abs(res["coeffs"] - base["coeffs"]) / np.maximum(1.0, np.abs(base["coeffs"]))
        cmov = np.fmax(cmov, np.where(np.isnan(d) & ~np.isnan(base["coeffs"]), np.inf, d))
        for s in range(nseg):
            lo, hi = int(off[s]), int(off[s + 1])
            ref = base["out"][lo:hi]
            den = float(np.linalg.norm(ref))
            num = float(np.linalg.norm(res["out"][lo:hi] - ref))
            omov[s] = max(omov[s], num / den if den > 0 else num)
    # operands that are zero to fp64 over inputs that are not all zero, and
    # everything above them; the segment's summed input norms bound those
    # under any operand, so only segments with a candidate are looked at
    if base["stats"].size:
        nonempty = off[1:] > off[:-1]
        total = np.zeros(nseg)
        for r in rows:
            total[nonempty] += np.add.reduceat(r * r, off[:-1][nonempty]) if r.size else 0.0
        candidate = base["stats"][:, :, 1:3] <= ZERO_FLOOR * total[None, :, None]
    else:
        candidate = np.zeros(base["stats"].shape[:2] + (2,), dtype=bool)
    if candidate.any():
        parent = node_parents(base["stats"].shape[0], schedule)
        for s in np.flatnonzero(candidate.any(axis=(0, 2))):
            lo, hi = int(off[s]), int(off[s + 1])
            opn = operand_input_norms([r[lo:hi] for r in rows], schedule)
            at_zero = (base["stats"][:, s, 1:3] <= ZERO_FLOOR * opn) & (opn > 0)
            for i, side in zip(*np.nonzero(at_zero)):
                cmov[i, s, side] = np.inf
                j = parent[i]
                while j >= 0:
                    cmov[j, s, :] = np.inf
                    j = parent[j]
                omov[s] = np.inf
    return {"base": base, "coeff_motion": cmov, "output_motion": omov}
