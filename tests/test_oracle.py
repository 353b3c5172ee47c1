"""The CPU oracle against its pins (closed forms, invariants, library routines, brute force)."""

import pytest

import pins
from oracle import ref


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(ref)
