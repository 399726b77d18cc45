"""The CPU oracle against its pins (closed forms, invariants, library
routines, finite differences, brute force). No GPU needed."""
import pytest

from oracle import l3_oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(l3_oracle)
