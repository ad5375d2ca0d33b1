"""The CPU reference against its pins (closed forms, invariances, brute force,
finite differences, torch's CPU fp64 SDPA + autograd)."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())
