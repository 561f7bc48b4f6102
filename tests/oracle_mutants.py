"""Planted mistakes in the CPU oracle, to show that its pins catch them.

TEST INFRASTRUCTURE ONLY.  ``python tests/oracle_mutants.py NAME`` replaces
one oracle function with a copy that carries the mistake NAME (in this
process only; nothing on disk changes), runs the oracle's pins
(tests/test_oracle.py) and prints one JSON line with the pins that failed.
``none`` plants nothing.  tests/test_oracle_mutations.py runs every mutant.

Each mistake is one a careful reader could plausibly make from the text: a
denominator taken from the wrong operand, a sign, the factor 1/2, the
zero-norm rule, the order of the returned coefficients or statistics, the
carry or the pairing of the tree, the chain's operand order, statistics
taken over the whole vector instead of per layer, a rounding mode, the
subnormal range, the orthogonality ratio's squares, the plain sum's order,
and the parity helpers (the stability check's noise taken in ulps of fp32
instead of fp64, or no noise at all, its zero floor at exact zeros only or
as wide as 1e-8; the chain's accumulated input norms).
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle import adasum as _ad  # noqa: E402
from oracle import rounding as _rd  # noqa: E402

_orig = {name: getattr(_ad, name) for name in
         ("tree_schedule", "adasum_chain", "orthogonality", "plain_sum", "operand_input_norms")}
_orig_round = _rd.round_to_format


def _pair_with(rule):
    """adasum_pair with the coefficients and statistics given by ``rule``."""
    def pair(a, b):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        d, A, B = float(np.dot(a, b)), float(np.dot(a, a)), float(np.dot(b, b))
        ca, cb, cf, st = rule(d, A, B)
        return ca * a + cb * b, cf, st
    return pair


def _right(d, A, B):
    return (1.0 if A == 0.0 else 1.0 - d / (2.0 * A)), (1.0 if B == 0.0 else 1.0 - d / (2.0 * B))


def _denominators_swapped(d, A, B):
    ca = 1.0 if B == 0.0 else 1.0 - d / (2.0 * B)
    cb = 1.0 if A == 0.0 else 1.0 - d / (2.0 * A)
    return ca, cb, (ca, cb), (d, A, B)


def _sign_flipped(d, A, B):
    ca = 1.0 if A == 0.0 else 1.0 + d / (2.0 * A)
    cb = 1.0 if B == 0.0 else 1.0 + d / (2.0 * B)
    return ca, cb, (ca, cb), (d, A, B)


def _half_dropped(d, A, B):
    ca = 1.0 if A == 0.0 else 1.0 - d / A
    cb = 1.0 if B == 0.0 else 1.0 - d / B
    return ca, cb, (ca, cb), (d, A, B)


def _zero_norm_coeff_zero(d, A, B):
    ca = 0.0 if A == 0.0 else 1.0 - d / (2.0 * A)
    cb = 0.0 if B == 0.0 else 1.0 - d / (2.0 * B)
    return ca, cb, (ca, cb), (d, A, B)


def _coeffs_reported_swapped(d, A, B):
    ca, cb = _right(d, A, B)
    return ca, cb, (cb, ca), (d, A, B)


def _stats_reported_swapped(d, A, B):
    ca, cb = _right(d, A, B)
    return ca, cb, (ca, cb), (d, B, A)


def _schedule_with(pairing, carry):
    """tree_schedule with another pairing of each level or carry rule."""
    def schedule(K):
        if K < 1:
            raise ValueError("K must be >= 1")
        current = [("leaf", k) for k in range(K)]
        levels, nid = [], 0
        while len(current) > 1:
            m = len(current) // 2
            pairs = pairing(current, m)
            nxt = []
            for _ in pairs:
                nxt.append(("node", nid))
                nid += 1
            if len(current) % 2 == 1:
                nxt = carry(current[-1], nxt)
            levels.append(pairs)
            current = nxt
        return levels
    return schedule


def _adjacent(cur, m):
    return [(cur[2 * j], cur[2 * j + 1]) for j in range(m)]


def _mirrored(cur, m):
    n = 2 * m
    return [(cur[j], cur[n - 1 - j]) for j in range(m)]


def _carry_last(odd, nxt):
    return nxt + [odd]


def _carry_first(odd, nxt):
    return [odd] + nxt


def _carry_dropped(odd, nxt):
    return nxt if nxt else [odd]


def _chain_operands_reversed(vectors):
    vectors = [np.asarray(v, dtype=np.float64) for v in vectors]
    acc = vectors[0].copy()
    coeffs, stats = [], []
    for v in vectors[1:]:
        acc, cf, st = oracle.adasum.adasum_pair(v, acc)
        coeffs.append(cf)
        stats.append(st)
    return acc, coeffs, stats


def _combine_over_whole_vector(fn, inputs, seg_offsets, out_format):
    """Statistics taken over all N elements instead of per segment."""
    rows, n = _ad._as_rows(inputs)
    off = _ad._check_offsets(seg_offsets, n)
    K, nseg = len(rows), off.size - 1
    res, cf, st = fn(rows)
    coeffs = np.ones((max(K - 1, 0), nseg, 2))
    stats = np.zeros((max(K - 1, 0), nseg, 3))
    for i in range(K - 1):
        coeffs[i, :] = cf[i]
        stats[i, :] = st[i]
    result = {"out": np.array(res, dtype=np.float64), "coeffs": coeffs, "stats": stats}
    if out_format is not None:
        result["out_rounded"] = _rd.round_to_format(result["out"], out_format)
    return result


def _round_with(to_int, subnormals=True):
    def round_to_format(x, fmt):
        p, emin, emax = _rd.FORMATS[fmt]
        x = np.asarray(x, dtype=np.float64)
        _, e = np.frexp(x)
        q = np.maximum(e - p, emin - p + 1) if subnormals else e - p
        with np.errstate(invalid="ignore", over="ignore"):
            y = np.ldexp(to_int(np.ldexp(x, -q)), q)
            y = np.where(np.isfinite(x) & (np.abs(y) >= np.ldexp(1.0, emax + 1)), np.copysign(np.inf, x), y)
            y = np.where(np.isfinite(x), y, x)
        return y
    return round_to_format


def _ties_away(v):
    return np.copysign(np.floor(np.abs(v) + 0.5), v)


def _orthogonality_unsquared(inputs, seg_offsets):
    return np.sqrt(_orig["orthogonality"](inputs, seg_offsets))


def _plain_sum_reversed(inputs, seg_offsets=None, out_format=None):
    return _orig["plain_sum"](list(inputs)[::-1], seg_offsets, out_format)


def _noise_in_fp32_ulps(rows, rng):
    out = []
    for r in rows:
        f = np.ascontiguousarray(r, dtype=np.float32)
        step = np.where(rng.random(r.size) < 0.5, 1, -1).astype(np.int32)
        moved = (f.view(np.int32) + step).view(np.float32).astype(np.float64)
        out.append(np.where(np.isfinite(r) & (r != 0.0), moved, r))
    return out


def _no_noise(rows, rng):
    return [np.array(r, copy=True) for r in rows]


def _chain_norms_not_accumulated(vectors, schedule="tree"):
    if schedule != "chain":
        return _orig["operand_input_norms"](vectors, schedule)
    norms = [float(np.dot(v, v)) for v in (np.asarray(x, dtype=np.float64) for x in vectors)]
    return np.asarray([(norms[k - 1], norms[k]) for k in range(1, len(norms))], dtype=np.float64).reshape(-1, 2)


# name -> {attribute of oracle.adasum / oracle.rounding: replacement}
MUTANTS = {
    "none": {},
    "denominators_swapped": {"adasum_pair": _pair_with(_denominators_swapped)},
    "sign_flipped": {"adasum_pair": _pair_with(_sign_flipped)},
    "half_dropped": {"adasum_pair": _pair_with(_half_dropped)},
    "zero_norm_coeff_zero": {"adasum_pair": _pair_with(_zero_norm_coeff_zero)},
    "coeffs_reported_swapped": {"adasum_pair": _pair_with(_coeffs_reported_swapped)},
    "stats_reported_swapped": {"adasum_pair": _pair_with(_stats_reported_swapped)},
    "pairing_mirrored": {"tree_schedule": _schedule_with(_mirrored, _carry_last)},
    "carry_first": {"tree_schedule": _schedule_with(_adjacent, _carry_first)},
    "carry_dropped": {"tree_schedule": _schedule_with(_adjacent, _carry_dropped)},
    "chain_operands_reversed": {"adasum_chain": _chain_operands_reversed},
    "stats_over_whole_vector": {"_combine_with": _combine_over_whole_vector},
    "rounding_truncates": {"round_to_format": _round_with(np.trunc)},
    "rounding_ties_away": {"round_to_format": _round_with(_ties_away)},
    "rounding_flushes_subnormal_range": {"round_to_format": _round_with(np.rint, subnormals=False)},
    "orthogonality_unsquared": {"orthogonality": _orthogonality_unsquared},
    "plain_sum_reversed": {"plain_sum": _plain_sum_reversed},
    "stability_noise_in_fp32_ulps": {"_ulp_noise": _noise_in_fp32_ulps},
    "stability_without_noise": {"_ulp_noise": _no_noise},
    "stability_exact_zeros_only": {"ZERO_FLOOR": 0.0},
    "stability_zero_floor_too_wide": {"ZERO_FLOOR": 1e-8},
    "chain_norms_not_accumulated": {"operand_input_norms": _chain_norms_not_accumulated},
}


def plant(name):
    """Install mutant ``name`` in every namespace the pins reach it through."""
    for attr, fn in MUTANTS[name].items():
        for mod in (_ad, _rd, oracle):
            if hasattr(mod, attr):
                setattr(mod, attr, fn)


class _Failures:
    def __init__(self):
        self.failed, self.passed = [], 0

    def pytest_runtest_logreport(self, report):
        if report.failed:
            self.failed.append(report.nodeid.split("::", 1)[-1])
        elif report.when == "call" and report.passed:
            self.passed += 1


def main(name):
    import pytest
    plant(name)
    col = _Failures()
    pytest.main([os.path.join(ROOT, "tests", "test_oracle.py"), "-q", "-p", "no:cacheprovider",
                 "--tb=no", "--no-header", "-o", "addopts="], plugins=[col])
    print(json.dumps({"mutant": name, "failed": col.failed, "passed": col.passed}), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
