"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS, BWD_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.forward)


def test_oracle_rejects_bad_arguments():
    import numpy as np
    lib = oracle.load()
    out = np.zeros(1)
    assert lib.oracle_lce_forward(None, None, None, 1, 0, 1, 0, None, 0, None, None, None) == -1
    assert lib.oracle_lce_forward(None, None, None, 1, 1, 0, 0, None, 0, None, None, None) == -1
    assert lib.oracle_lce_forward(None, None, None, 1, 1, 1, 7, None, 0, None, None, None) == -1
    h = np.zeros((1, 1), np.float32)
    y = np.zeros(1, np.int32)
    rows = np.array([5], np.int64)
    assert lib.oracle_lce_forward(h.ctypes.data, h.ctypes.data, y.ctypes.data, 1, 1, 1, 1,
                                  rows.ctypes.data, 1, out.ctypes.data, out.ctypes.data,
                                  out.ctypes.data) == -1


def test_oracle_empty_batch():
    import torch
    loss, lse, zt = oracle.forward(torch.zeros(0, 4), torch.zeros(3, 4), torch.zeros(0, dtype=torch.int32))
    assert loss.shape == (0,) and lse.shape == (0,)


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_oracle_backward_pin(pin):
    pin(oracle.forward, oracle.backward)


def test_oracle_backward_rejects_bad_arguments():
    import numpy as np
    lib = oracle.load()
    assert lib.oracle_lce_backward(None, None, None, None, 1, 0, 1, 0, None, 0, None, None, None, None) == -1
    h = np.zeros((1, 1), np.float32)
    y = np.zeros(1, np.int32)
    g = np.ones(1)
    out = np.zeros(1)
    rows = np.array([3], np.int64)
    assert lib.oracle_lce_backward(h.ctypes.data, h.ctypes.data, y.ctypes.data, g.ctypes.data, 1, 1, 1, 1,
                                   rows.ctypes.data, 1, out.ctypes.data, None, None, None) == -1
