"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()      # builds from rmsnorm_oracle.c if missing or stale


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)
