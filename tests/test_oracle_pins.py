"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(ref, pin):
    pin(ref)
