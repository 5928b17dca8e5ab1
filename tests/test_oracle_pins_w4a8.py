"""The W4A8 oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins_w4a8


@pytest.mark.parametrize("pin", oracle_pins_w4a8.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)
