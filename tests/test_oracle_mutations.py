"""The oracle's pins catch plausible mistakes planted in the oracle (CPU).

tests/oracle_mutants.py plants one mistake per child process (denominators,
sign, the factor 1/2, the zero-norm rule, reported coefficient and statistic
order, tree pairing and carry, chain operand order, per-layer statistics,
rounding mode and subnormal range, the orthogonality ratio, plain-sum order,
the parity helpers) and runs tests/test_oracle.py.  Every mutant must fail
at least two pins; the unmutated oracle must fail none.
"""

import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import oracle_mutants  # noqa: E402

MIN_FAILED = 2


@pytest.fixture(scope="module")
def outcomes():
    env = dict(os.environ, OMP_NUM_THREADS="1", PYTHONDONTWRITEBYTECODE="1")
    names = list(oracle_mutants.MUTANTS)
    res = {}
    for i in range(0, len(names), 8):
        procs = {n: subprocess.Popen([sys.executable, os.path.join(HERE, "oracle_mutants.py"), n],
                                     stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env)
                 for n in names[i:i + 8]}
        for n, p in procs.items():
            out, err = p.communicate(timeout=600)
            lines = [ln for ln in out.splitlines() if ln.startswith("{")]
            assert lines, f"mutant {n} printed no result:\n{out[-2000:]}\n{err[-2000:]}"
            res[n] = json.loads(lines[-1])
    return res


def test_unmutated_oracle_passes_every_pin(outcomes):
    r = outcomes["none"]
    assert r["failed"] == [] and r["passed"] > 0


@pytest.mark.parametrize("name", [n for n in oracle_mutants.MUTANTS if n != "none"])
def test_mutant_is_caught(outcomes, name):
    r = outcomes[name]
    print(f"{name}: {len(r['failed'])} pins fail: {', '.join(r['failed'])}")
    assert len(r["failed"]) >= MIN_FAILED, r
