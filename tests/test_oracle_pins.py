"""The CPU oracle against the pins that the pages and the mathematics fix
(closed forms, invariants, brute force on tiny shapes)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
