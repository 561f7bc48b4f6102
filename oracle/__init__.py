"""Plain, slow CPU oracle for the Adasum gradient combiner.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports it,
and this package imports nothing from the product path.

Source: M. Maleki et al., "Scaling Distributed Training with Adaptive
Summation" (arXiv 2006.02924).  The display equations of that text did not
survive extraction, so the pairwise operator is taken in the form

    Adasum(a, b) = (1 - a.b / (2 |a|^2)) a + (1 - a.b / (2 |b|^2)) b

and checked against everything the prose still fixes (orthogonal inputs are
summed, parallel inputs are averaged, the operator is the mean of the two
emulated sequential orders, it is applied per layer, it is not elementwise).

Modules
  adasum    fp64 NumPy oracle: pairwise operator, binary tree, per-segment
            combine, orthogonality ratio, plain sum, linear chain, the input
            norms under each node's operands, and the stability of the
            oracle's own results under rounding-size noise (which coefficients
            and outputs fp64 arithmetic does not determine, at the operator's
            discontinuity and under deep cancellation).
  exact     the same definitions in exact rational arithmetic (fractions),
            for brute force on tiny inputs.
  rounding  IEEE round-to-nearest-even from fp64 to fp32 / fp16 / bf16.

Parity status: every function here is pinned by CPU tests in
tests/test_oracle.py (closed forms, hand-derived worked examples, exact
brute force, library cross-checks, invariants).  No function is unpinned.
"""

from .adasum import (  # noqa: F401
    ZERO_FLOOR,
    adasum_pair,
    adasum_tree,
    adasum_chain,
    combine,
    combine_chain,
    plain_sum,
    orthogonality,
    operand_input_norms,
    node_parents,
    stability,
    tree_schedule,
)
from .rounding import round_to_format  # noqa: F401
