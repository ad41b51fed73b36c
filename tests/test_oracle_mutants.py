"""Each planted mistake in a copy of the oracle must fail at least one pin.

The copies are the oracle source with one text patch of oracle_mutants.py
applied, built on the CPU; the real oracle is untouched.  This checks that
the pins can tell a wrong oracle apart.
"""
import os

import pytest

import oracle
import pins
from oracle_mutants import MUTANTS


def test_patches_apply_to_the_oracle_source():
    """Every patch's original text occurs exactly once in the oracle source."""
    src = open(oracle.SOURCE).read()
    for n, (_, pairs) in MUTANTS.items():
        for old, _new in pairs:
            assert src.count(old) == 1, n


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(tmp_path, mutant):
    desc, pairs = MUTANTS[mutant]
    src = open(oracle.SOURCE).read()
    for old, new in pairs:
        assert src.count(old) == 1
        src = src.replace(old, new)
    c_path = tmp_path / f"oracle_m{mutant}.c"
    c_path.write_text(src)
    path = str(tmp_path / f"liboracle_m{mutant}.so")
    oracle.build(path, source=str(c_path))
    orc = oracle.Oracle(path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError):
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant} ({desc}) passes every pin"
