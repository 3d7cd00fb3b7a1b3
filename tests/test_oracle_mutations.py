"""Each planted oracle mistake (tests/oracle_mutants.py) must make the pin suite fail (CPU only).

The pins are meant to catch a plausible error anywhere in the oracle; this runs them once per
mutant in a fresh interpreter, with the mutant applied by tests/conftest.py, and requires a
failure. A mutant the pins miss names a gap in the pins. Two tests are left out of these runs: the
brute-force routing comparison and the golden file restate the oracle's own score formula (the
element loops re-type it; the golden values were written by the oracle), so a mutant must be caught
by a pin that fixes the score from outside.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import oracle_mutants  # noqa: E402


def _run_pins(mutant):
    env = dict(os.environ, PISA_ORACLE_MUTANT=mutant, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q",
           "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not test_routing_matches_sort and not test_golden_tiny_taylor"]
    r = subprocess.run(cmd, cwd=os.path.dirname(HERE), env=env, capture_output=True, text=True, timeout=600)
    return mutant, r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes():
    with ThreadPoolExecutor(max_workers=4) as ex:
        return {m: (rc, out) for m, rc, out in ex.map(_run_pins, sorted(oracle_mutants.MUTANTS))}


@pytest.mark.parametrize("mutant", sorted(oracle_mutants.MUTANTS))
def test_pins_catch_mutant(mutant, outcomes):
    rc, out = outcomes[mutant]
    assert rc == 1, f"pins did not fail under mutant {mutant} (exit {rc}):\n{out}"
