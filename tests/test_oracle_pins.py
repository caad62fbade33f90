"""The fp64 oracle against what the definitions and the pages fix (CPU only)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
