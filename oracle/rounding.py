"""Round fp64 values to an IEEE binary format, round-to-nearest-even.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The combined gradient is returned in the dtype of the inputs; the oracle
computes in fp64 and rounds once at the end.  This module is that rounding,
written from the IEEE 754 definition: a finite x is scaled so that the unit
in the last place of its binade (or the subnormal quantum, whichever is
larger) becomes 1, rounded to the nearest integer with ties to even, and
scaled back; a result at or beyond 2**(emax+1) overflows to infinity.
"""

import numpy as np

# name -> (precision p in bits incl. the implicit bit, emin, emax)
FORMATS = {
    "f32": (24, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def round_to_format(x, fmt):
    """Return fp64 array holding round_RNE(x) in format ``fmt``.

    Every returned value is exactly representable in ``fmt`` (or is +-inf /
    NaN), so a later cast to that format is exact.
    """
    p, emin, emax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    # x = m * 2**e with 0.5 <= |m| < 1, so the binade is [2**(e-1), 2**e) and
    # its ulp is 2**(e - p).  Below 2**emin the quantum stays 2**(emin - p + 1).
    _, e = np.frexp(x)
    q = np.maximum(e - p, emin - p + 1)
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        y = np.where(np.isfinite(x) & (np.abs(y) >= np.ldexp(1.0, emax + 1)),
                     np.copysign(np.inf, x), y)
        y = np.where(np.isfinite(x), y, x)
    return y
