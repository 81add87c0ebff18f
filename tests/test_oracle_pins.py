"""The CPU oracle against closed forms, a hand example, a dense library
computation and exact invariances (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
