"""Every planted mistake in the oracle must be caught by at least one pin.

The oracle source carries compile-time mutants (KDA_ORACLE_MUTANT=1..15): decay after the
write, read before the write, decay of the value rows, a flipped delta sign, a wrong GQA head
map, a dropped scale, a skipped sigmoid, a skipped L2 norm, a transposed initial state, beta on
v only, the gate of the previous token, base-2 instead of natural exp, and a scalar gate read
from the query/key head instead of the value head.  Each is built
into its own library here and run through the pin set.
"""
import os

import pytest

from oracle import build_oracle
import oracle_pins

MUTANTS = list(range(1, 16))


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(tmp_path, mutant):
    path = str(tmp_path / f"liboracle_m{mutant}.so")
    build_oracle(path, mutant=mutant)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(path)
        except AssertionError as e:
            caught.append(f"{pin.__name__}: {str(e).splitlines()[0]}")
    assert caught, f"planted mistake {mutant} passed every pin"
    os.remove(path)
