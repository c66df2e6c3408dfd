"""The fp64 oracle against its pins (library routines, closed forms,
invariants, brute force and a hand-worked example)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_max_rel_err_metric():
    import numpy as np
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    assert oracle.max_rel_err(ref, ref) == 0.0
    assert oracle.max_rel_err(ref + np.array([[0.0, 0.0], [0.0, 0.4]]), ref) == pytest.approx(0.1)
    assert oracle.max_rel_err(np.zeros(3), np.zeros(3)) == 0.0
