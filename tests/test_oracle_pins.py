"""The fp64 oracle against closed forms, brute force, scipy and a worked example."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_rejects_bad_shapes(orc):
    import numpy as np
    h0 = np.zeros((1, 3, 2, 2))
    x = np.zeros((1, 1, 3, 2))
    B = np.zeros((1, 1, 2, 2))
    with pytest.raises((ValueError, AssertionError)):
        # 3 heads cannot be split into 2 groups
        orc.conventional(h0, x, B, B, np.zeros((1, 1, 3)), np.zeros(3), np.zeros(3))
