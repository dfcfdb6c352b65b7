"""The fp64 oracle against its pins (CPU only)."""
import pytest

from oracle import build_oracle, load_oracle
from oracle.oracle import LIB
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    build_oracle(LIB)
    load_oracle(LIB)
    return LIB


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(lib, pin):
    pin(lib)
