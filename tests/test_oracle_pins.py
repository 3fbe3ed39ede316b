"""The fp64 oracle against closed forms, a library routine, brute force and invariants (CPU)."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle.gqla)
