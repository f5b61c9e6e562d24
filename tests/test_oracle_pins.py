"""The CPU oracle against closed forms, library routines, invariants and brute force."""
import pytest

from .oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(ref, pin):
    pin(ref)
