"""The CPU oracle against its pins (closed forms, hand-packed blocks, brute force,
textbook integer matmul, invariants).  CPU only."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
