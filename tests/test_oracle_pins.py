"""The CPU oracle against its pins (hand-worked fixtures, closed forms, exact arithmetic,
library special cases and invariants); see oracle_pins.py."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_argument_errors(orc):
    import numpy as np
    x = np.zeros((2, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.fused([x], x, np.zeros(9, np.uint16), 1e-6)
    with pytest.raises(TypeError):
        orc.reduce([x.astype(np.int32)])
