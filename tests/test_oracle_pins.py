"""The CPU oracle against its pins (closed forms, special cases, expansion, invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib.run)
