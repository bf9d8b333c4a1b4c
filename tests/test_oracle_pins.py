"""The float64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
