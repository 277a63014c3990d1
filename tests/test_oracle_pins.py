"""The CPU oracle against its pins (see ``tests/pins.py``)."""
import pytest

import oracle

from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle)
