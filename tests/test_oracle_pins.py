"""The CPU oracle against its pins (closed forms, library reductions, brute force, finite
differences).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
