"""The oracle against its pins (CPU only).  See tests/pins.py for what each pin
compares with; none of them re-derives a result with the oracle's own code."""
import pytest

import oracle as O
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O.load())
