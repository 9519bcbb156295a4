"""The float64 oracle against independent sources (CPU only)."""
import pytest

import oracle
import _pins


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
