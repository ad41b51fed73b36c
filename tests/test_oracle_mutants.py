"""Each planted mistake in a copy of the oracle must fail at least one pin.

The copies are built on the CPU with -DORACLE_MUTANT=n; the real oracle is
built without it.  This checks that the pins can tell a wrong oracle apart.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    1: "strict > instead of >= at the threshold",
    2: "row scale also covers outlier columns",
    3: "weight scale per input column",
    4: "round half away from zero",
    5: "dequantize by 127 instead of 127^2",
    6: "recovered weight missing SCB/127",
    7: "bias dropped",
    8: "outlier entries left in CA",
    9: "outlier part subtracted",
    10: "outlier gather ignores the index list",
    11: "int8 product drops a term",
    12: "per-tensor scale taken per row",
    13: "E4M3 ties rounded away from zero",
    14: "FP8 product dequantized by 448 instead of 448^2",
    15: "E4M3 subnormals flushed to zero",
    16: "FP8 scale uses the int8 range 127",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(tmp_path, mutant):
    path = str(tmp_path / f"liboracle_m{mutant}.so")
    oracle.build(path, mutant=mutant)
    orc = oracle.Oracle(path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, oracle.OracleError):
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant} ({MUTANTS[mutant]}) passes every pin"
