"""Exact rational Adasum, for brute force on tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The same definitions as ``oracle.adasum`` with every value a
``fractions.Fraction``, so the results carry no rounding at all.  Inputs are
converted with ``Fraction(float)``, which is exact for binary floats.
"""

from fractions import Fraction


def _dot(x, y):
    return sum((p * q for p, q in zip(x, y)), Fraction(0))


def adasum_pair(a, b):
    """Exact pairwise Adasum; returns ``(c, (ca, cb), (d, A, B))``."""
    a = [Fraction(v) for v in a]
    b = [Fraction(v) for v in b]
    d, A, B = _dot(a, b), _dot(a, a), _dot(b, b)
    ca = Fraction(1) if A == 0 else 1 - d / (2 * A)
    cb = Fraction(1) if B == 0 else 1 - d / (2 * B)
    return [ca * x + cb * y for x, y in zip(a, b)], (ca, cb), (d, A, B)


def adasum_tree(vectors):
    """Exact tree Adasum: pairs (0,1),(2,3),... level by level, odd last
    vector carried.  Returns ``(result, coeffs, stats)`` in level-major
    node order."""
    current = [[Fraction(v) for v in vec] for vec in vectors]
    coeffs, stats = [], []
    while len(current) > 1:
        nxt = []
        for j in range(len(current) // 2):
            c, cf, st = adasum_pair(current[2 * j], current[2 * j + 1])
            nxt.append(c)
            coeffs.append(cf)
            stats.append(st)
        if len(current) % 2 == 1:
            nxt.append(current[-1])
        current = nxt
    return current[0], coeffs, stats


def adasum_chain(vectors):
    """Exact linear chain g[0, n+1] = Adasum(g[0, n], g[n+1])."""
    acc = [Fraction(v) for v in vectors[0]]
    coeffs, stats = [], []
    for vec in vectors[1:]:
        acc, cf, st = adasum_pair(acc, vec)
        coeffs.append(cf)
        stats.append(st)
    return acc, coeffs, stats
