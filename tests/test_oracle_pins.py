"""CPU pins of the oracle (no GPU): library casts, spec tables, exact brute force, closed forms."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
