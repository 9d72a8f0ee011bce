"""The oracle against its pins (closed forms, library routines, brute force,
invariants).  CPU only."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.gmm_oracle)
