"""Every pin of the CPU oracle (tests/oracle_pins.py) against the oracle."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__[4:])
def test_pin(pin):
    pin(oracle.lib())
