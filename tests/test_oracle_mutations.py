"""The oracle's pins catch plausible mistakes planted in the oracle (CPU).

Each mutant of tests/oracle_mutants.py edits one place of one oracle module
(the full tree: a tie order, a sign, a child or row index, a GQA map, a
scale, the tie measure's pair or denominator, an accumulation or rounding
mode, the bf16 widening; the growing cache: depth, open-node means, existing
nodes, blocks cut at n; the spheres: max radius, the bound's |q| and r,
strict comparisons, overflow; the causal prefill: the prefix length, the
query's position, keys read, the tie measure) and runs that module's pins
that do not compare with stored oracle outputs.  The unmutated oracles must
pass them and every mutant must fail at least one.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests import oracle_mutants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "oracle_mutants.py")


def _run(name: str) -> str:
    r = subprocess.run([sys.executable, DRIVER, name], capture_output=True, text=True,
                       cwd=ROOT, timeout=600)
    for line in r.stdout.splitlines():
        if line.startswith(f"PIN_RUN {name} "):
            return line.split(" ", 2)[2]
    return f"NO RESULT (rc {r.returncode}): {(r.stdout + r.stderr)[-400:]}"


@pytest.mark.parametrize("module", sorted(oracle_mutants.PIN_FILES))
def test_unmutated_oracle_passes_the_pins(module):
    assert _run(f"none:{module}") == "PASSED"


@pytest.mark.timeout(900)
def test_every_mutant_fails_a_pin():
    names = sorted(oracle_mutants.MUTANTS)
    assert len(names) >= 40
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = dict(zip(names, ex.map(_run, names)))
    missed = {n: r for n, r in results.items() if r != "FAILED"}
    assert not missed, f"mutants the pins do not catch: {missed}"
