"""The oracle against facts fixed outside itself (CPU only)."""

import numpy as np
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    with np.errstate(all="raise", under="ignore"):
        pin()
