"""The CPU oracle against its pins (closed forms, invariants, brute force,
finite differences, hand-derived worked examples). CPU only."""

import pytest

from oracle_pins import ALL_PINS, real_ns


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(real_ns())
