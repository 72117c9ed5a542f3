"""The CPU oracle against every pin (values the pages print, closed forms, textbook routines,
brute force).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(olib, pin):
    pin(olib)
