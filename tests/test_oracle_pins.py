"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle)
