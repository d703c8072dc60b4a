"""The CPU oracle checked against what the pages and mathematics fix
(hand-worked examples, closed forms, constructed decompositions, brute force,
library routines).  CPU only."""
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.mbok_oracle)
