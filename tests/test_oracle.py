"""The fp64 oracle against its pins (CPU only).  See tests/oracle_pins.py for what each pin is."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(None)
