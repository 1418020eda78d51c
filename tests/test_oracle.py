"""The CPU oracle against its pins (closed forms, library routines, brute
force, invariants, hand-derived fixtures). No GPU."""
import pytest

import oracle.logo as O
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)
