"""The oracle's assignment, start and fit-loop functions against their pins
(a published generator output, uniformity, scikit-learn).  CPU only."""
import pytest

import oracle
from oracle import gmm_assign_fit
from tests import oracle_pins_assign_fit as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(gmm_assign_fit, oracle.gmm_oracle)
