"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle.fp64 as L
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(L)
