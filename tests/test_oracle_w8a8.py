"""Pins of the oracle's W8A8 quantized linear (baracuda_kernels::quantize,
module quantized_linear: a fused W8A8 quantized matmul; the reading is
symmetric s8 codes, one fp32 scale per activation row and per weight output
channel, y = ((float)acc * sx[m]) * sw[n] with acc the exact integer dot
product).  Each pin comes from arithmetic that does not use the oracle."""
import numpy as np
import pytest

import oracle as orc


def bf16_to_f32(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


def test_hand_example():
    # acc = 1*3 + (-2)*4 + 127*(-128) = -16261; scales 0.5 and 0.25 are exact
    qx = np.array([[1, -2, 127]], np.int8)
    qw = np.array([[3, 4, -128]], np.int8)
    y = orc.w8a8_linear(qx, np.array([0.5], np.float32), qw, np.array([0.25], np.float32), "f32")
    assert y[0, 0] == np.float32(-16261 / 8)


def test_unit_scales_equal_integer_matmul():
    rng = np.random.default_rng(1)
    qx = rng.integers(-128, 128, (7, 200)).astype(np.int8)
    qw = rng.integers(-128, 128, (5, 200)).astype(np.int8)
    exact = qx.astype(np.int64) @ qw.astype(np.int64).T           # |acc| < 2^24: exact in binary32
    assert np.abs(exact).max() < 2 ** 24
    y = orc.w8a8_linear(qx, np.ones(7, np.float32), qw, np.ones(5, np.float32), "f32")
    assert np.array_equal(y.astype(np.float64), exact.astype(np.float64))


def test_power_of_two_scales_are_exact():
    rng = np.random.default_rng(2)
    qx = rng.integers(-128, 128, (4, 64)).astype(np.int8)
    qw = rng.integers(-128, 128, (6, 64)).astype(np.int8)
    ex = rng.integers(-20, 5, 4)
    ew = rng.integers(-20, 5, 6)
    sx = np.ldexp(1.0, ex).astype(np.float32)
    sw = np.ldexp(1.0, ew).astype(np.float32)
    y = orc.w8a8_linear(qx, sx, qw, sw, "f32")
    exact = (qx.astype(np.int64) @ qw.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), np.ldexp(exact, ex[:, None] + ew[None, :]))


def test_large_sum_rounds_once_to_nearest():
    # acc = 127 * 127 * 1041 = 16790289 = 2^24 + 13073: odd and above 2^24,
    # a tie between 16790288 and 16790290; nearest-even keeps 16790288
    # (16790288 / 2 is even)
    K = 1041
    qx = np.full((1, K), 127, np.int8)
    qw = np.full((1, K), 127, np.int8)
    y = orc.w8a8_linear(qx, np.ones(1, np.float32), qw, np.ones(1, np.float32), "f32")
    assert 127 * 127 * K == 16790289
    assert int(y[0, 0]) == 16790288


def test_sign_symmetry_and_scale_order():
    rng = np.random.default_rng(3)
    qx = rng.integers(-127, 128, (5, 96)).astype(np.int8)
    qw = rng.integers(-127, 128, (4, 96)).astype(np.int8)
    sx = rng.uniform(1e-3, 1e-1, 5).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-1, 4).astype(np.float32)
    y = orc.w8a8_linear(qx, sx, qw, sw, "f32")
    yn = orc.w8a8_linear(-qx, sx, qw, sw, "f32")
    assert np.array_equal(yn, -y)
    # within one rounding of each multiplication of the exact real product
    exact = (qx.astype(np.int64) @ qw.astype(np.int64).T) * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    assert np.all(np.abs(y - exact) <= 3 * 2.0 ** -24 * np.abs(exact))


def test_bf16_output_is_nearest_even():
    # y values 1 + 2^-8 (a tie between bf16 1 and 1 + 2^-7: goes to the even 1)
    # and 1 + 3 * 2^-8 (a tie that goes up to 1 + 2^-6)
    qx = np.array([[1], [1]], np.int8)
    qw = np.array([[1]], np.int8)
    sx = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8], np.float32)
    y = orc.w8a8_linear(qx, sx, qw, np.ones(1, np.float32), "bf16")
    assert bf16_to_f32(y[:, 0]).tolist() == [1.0, 1 + 2.0 ** -6]


def test_rejects_overlong_k():
    with pytest.raises(ValueError):
        orc.w8a8_linear(np.zeros((1, 131072), np.int8), np.ones(1, np.float32), np.zeros((1, 131072), np.int8),
                        np.ones(1, np.float32), "f32")
