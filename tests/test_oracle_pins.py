"""The oracle against its pins (worked examples, closed forms, invariants)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
