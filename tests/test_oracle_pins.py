"""The CPU oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
