"""The CPU oracle checked against brute force, library routines, closed forms and
invariants (no GPU)."""
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
