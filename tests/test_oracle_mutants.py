"""Each planted mistake in the oracle (compile-time ORACLE_MUTANT) must be
caught by at least one pin: a dropped k term, A read column-major, truncating
instead of rounding, ReLU before the scale, the scale dropped, subnormals
decoded as normals, ties rounded away from zero, a binary32 running sum, and
in the epilogue variants a dropped bias, a bias indexed by row, GELU without
its cubic term, the bias added after the activation."""
import os

import pytest

import oracle_pins as P

MUTANTS = {
    1: "last k term dropped",
    2: "A indexed column-major",
    3: "truncation instead of round-to-nearest-even",
    4: "ReLU applied before the scale",
    5: "scale dropped",
    6: "subnormal inputs decoded with an implicit 1",
    7: "ties rounded away from zero",
    8: "binary32 running sum",
    9: "bias dropped",
    10: "bias indexed by row instead of column",
    11: "GELU without the cubic term",
    12: "bias added after the activation",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"mutant{m}")
def test_pins_catch_mutant(tmp_path, mutant):
    from oracle import oracle

    path = os.path.join(str(tmp_path), f"liboracle_m{mutant}.so")
    oracle.build(path, mutant=mutant)
    orc = oracle.Oracle(path)
    assert orc.mutant == mutant
    caught = []
    for pin in P.ALL_PINS:
        try:
            fails = pin(orc)
        except Exception as e:  # a crash in a pin also counts as caught
            fails = [f"{pin.__name__} raised {e!r}"]
        if fails:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {mutant} ({MUTANTS[mutant]})"
