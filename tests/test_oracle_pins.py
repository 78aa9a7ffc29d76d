"""The CPU oracle against closed forms, invariants, a dense library routine and
the counts the pages print (see oracle_pins.py for what each pin fixes)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
