"""The CPU oracle against its pins (values printed on the pages, closed forms,
independent library routines and the exact-rational brute force)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__[4:])
def test_pin(orc, pin):
    pin(orc)
