"""The CPU oracle against what the ZeroGR pages and the mathematics fix."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
