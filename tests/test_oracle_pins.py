"""The CPU oracle against its pins (hand blocks, exact arithmetic, library
fp16 conversion, brute force). No GPU."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
