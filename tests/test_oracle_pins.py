"""The CPU oracle against brute force, library routines, closed forms,
invariants and the pages' worked example (no GPU needed)."""

import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
