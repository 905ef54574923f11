"""The fp64 oracle against everything that fixes it from outside (see pins.py)."""
import numpy as np
import pytest

import pins
from oracle import oracle as O


@pytest.fixture(scope="module")
def lib():
    return O.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_bias_length_checked(lib):
    x = np.zeros((1, 2, 3))
    w = np.zeros((2, 2, 2))
    with pytest.raises(O.OracleError):
        O.convtranspose(x, w, np.zeros(3), lib=lib)


def test_empty_outputs(lib):
    # N = 0: an empty Y of the resolved shape
    y = O.convtranspose(np.zeros((0, 2, 4)), np.ones((2, 3, 2)), None, lib=lib, strides=[2])
    assert y.shape == (0, 3, 8)
    # L = 0 with a kernel longer than the stride: footprint d(K-1)+1-s
    y = O.convtranspose(np.zeros((1, 1, 0)), np.ones((1, 1, 4)), np.array([5.0]), lib=lib,
                        strides=[2])
    assert y.shape == (1, 1, 2) and np.all(y == 5.0)
    # C = 0: Y is the bias
    y = O.convtranspose(np.zeros((1, 0, 3)), np.zeros((0, 2, 3)), np.array([1.0, 2.0]), lib=lib)
    assert y.shape == (1, 2, 5) and np.all(y[0, 0] == 1.0) and np.all(y[0, 1] == 2.0)


def test_thread_count_independent(lib, monkeypatch):
    rng = np.random.default_rng(3)
    x, w, b, attrs = pins.random_case(rng, nsp=2)
    y1 = O.convtranspose(x, w, b, lib=lib, **attrs)
    y2 = O.convtranspose(x, w, b, lib=lib, **attrs)
    assert np.array_equal(y1, y2)
