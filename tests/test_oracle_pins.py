"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_oracle_pin(ora, pin):
    pin(ora)
