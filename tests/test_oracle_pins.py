"""The oracle against what the pages and mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def L():
    return oracle.lib()


@pytest.mark.parametrize("pin", pins.QUICK_PINS, ids=lambda f: f.__name__)
def test_pin(L, pin):
    pin(L)
