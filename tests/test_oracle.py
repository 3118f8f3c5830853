"""The CPU oracle against facts outside itself (see tests/oracle_pins.py)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())


def test_oracle_uses_threads():
    assert oracle.num_threads() >= 1
