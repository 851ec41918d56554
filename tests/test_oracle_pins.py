"""The oracle agrees with every pin (closed forms, brute force, invariants, golden rows)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def L():
    return oracle.lib()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin, L):
    pin(L)
