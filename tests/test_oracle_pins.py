"""The oracle against its pins (no GPU)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle)
