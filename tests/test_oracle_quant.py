"""Pins of oracle.dequantize, the quantised-head format (CPU only).

Each expected value is a closed form worked out by hand from the format's
definition w = bf16(fl32(fl32(scale * q) + bias)), chosen so that a plausible
slip fails one of them: a swapped nibble order, a wrong group index, a fused
multiply-add instead of two roundings, truncation instead of ties-to-even, or
a dropped bias or scale.
"""
import numpy as np
import pytest
import torch

import oracle


def _vals(bits16):
    return torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16)).view(torch.bfloat16).float().numpy()


def _f32(x):
    return np.array(x, dtype=np.float32)


def test_hand_example_8bit():
    codes = np.arange(8, dtype=np.uint8).reshape(1, 8)
    w = _vals(oracle.dequantize(codes, _f32([[0.5]]), _f32([[-1.0]]), 8, 8))
    assert w.tolist() == [[-1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 2.5]]


def test_nibble_order_4bit():
    # byte 0x21 holds weight 0 = 1 (low nibble) and weight 1 = 2 (high nibble)
    codes = np.array([[0x21, 0x43, 0x65, 0x87]], dtype=np.uint8)
    w = _vals(oracle.dequantize(codes, _f32([[1.0]]), _f32([[0.0]]), 4, 8))
    assert w.tolist() == [[1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0]]


def test_unit_scale_zero_bias_is_the_code():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(5, 64), dtype=np.uint8)
    w = _vals(oracle.dequantize(codes, np.ones((5, 2), np.float32), np.zeros((5, 2), np.float32), 8, 32))
    assert np.array_equal(w, codes.astype(np.float32))     # integers up to 255 are exact in bf16


def test_group_index_is_d_over_group():
    codes = np.ones((1, 16), dtype=np.uint8)
    w = _vals(oracle.dequantize(codes, _f32([[1.0, 2.0]]), _f32([[0.0, 10.0]]), 8, 8))
    assert w.tolist() == [[1.0] * 8 + [12.0] * 8]


def test_bf16_ties_round_to_even():
    # scale 2^-8, bias 1: q = 1 gives 1 + 2^-8, exactly between 1 and 1 + 2^-7 -> 1 (even);
    # q = 3 gives 1 + 3 * 2^-8, between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6;
    # q = 5 gives 1 + 5 * 2^-8 -> tie between 1 + 2^-6 (even) and 1 + 3 * 2^-7 -> 1 + 2^-6
    codes = np.array([[1, 3, 5, 2, 0, 0, 0, 0]], dtype=np.uint8)
    w = _vals(oracle.dequantize(codes, _f32([[2.0 ** -8]]), _f32([[1.0]]), 8, 8))
    assert w[0, :4].tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7]


def test_two_float32_roundings_not_one():
    # scale = fl32(1/3) = 0.3333333432674408, q = 3: the exact product 1.0000000298...
    # rounds to 1.0 in float32, so with bias -1 the weight is exactly 0; a fused
    # multiply-add would keep 2.98e-8.
    third = np.float32(1.0) / np.float32(3.0)
    codes = np.array([[3] * 8], dtype=np.uint8)
    w = _vals(oracle.dequantize(codes, _f32([[third]]), _f32([[-1.0]]), 8, 8))
    assert np.all(w == 0.0)
    fused = float(np.float64(third) * 3.0 - 1.0)
    assert fused > 2.9e-8                                       # what the fused form would give


def test_bias_and_scale_both_enter():
    codes = np.full((1, 8), 4, dtype=np.uint8)
    w = _vals(oracle.dequantize(codes, _f32([[0.25]]), _f32([[0.5]]), 8, 8))
    assert np.all(w == 1.5)


def test_rejects_bad_arguments():
    codes = np.zeros((2, 16), dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.dequantize(codes, np.ones((2, 2), np.float32), np.ones((2, 2), np.float32), 3, 8)
    with pytest.raises(ValueError):
        oracle.dequantize(codes, np.ones((2, 3), np.float32), np.ones((2, 3), np.float32), 8, 6)
