"""The fp64 oracle against what the pages and the mathematics fix (CPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()
