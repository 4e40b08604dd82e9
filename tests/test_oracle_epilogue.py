"""Pins of the oracle's fused epilogue (CPU only).

Reading (the Momenta talk, section "Graph層面", folds bias and ReLU into the
convolution; the order is a ResNet block's tail): float y = act(conv +
bias[k] + residual) with normaliser den + |bias| + |residual|; int8 y =
clamp(rne(fp32(acc + bias[k]) * scale[k] + fp32(residual)), lo, 127) with
lo = 0 under ReLU, -127 otherwise.

Every expected value is worked out by hand and written down as a literal, so
the pins do not restate the oracle's formula.  The values are chosen so that
each plausible slip changes at least one of them: ReLU applied before the
residual, a dropped or wrongly indexed bias, the bias added after the
scaling, the residual added before it, a ReLU floor of -127, a normaliser
without the added terms.
"""
import numpy as np
import pytest

import oracle


def _worked_float():
    # N=2, C=1, 1x2 image, K=2 (1x1 kernel: w[0] = 3, w[1] = -1)
    x = np.array([[[[1.0, -2.0]]], [[[0.5, 4.0]]]])
    w = np.array([[[[3.0]]], [[[-1.0]]]])
    bias = np.array([0.5, -0.25])
    res = np.array([[[[-1.0, 10.0]], [[2.0, -8.0]]],
                    [[[0.0, -1.0]], [[-3.0, 0.5]]]])
    return x, w, bias, res


def pin_float_bias_residual_relu():
    x, w, bias, res = _worked_float()
    y, den = oracle.conv2d_fused(x, w, bias, res, relu=True)
    # conv: n0: k0 [3, -6], k1 [-1, 2]; n1: k0 [1.5, 12], k1 [-0.5, -4]
    # + bias: n0: [3.5, -5.5], [-1.25, 1.75]; n1: [2, 12.5], [-0.75, -4.25]
    # + residual: n0: [2.5, 4.5], [0.75, -6.25]; n1: [2, 11.5], [-3.75, -3.75]
    # ReLU
    expect = np.array([[[[2.5, 4.5]], [[0.75, 0.0]]], [[[2.0, 11.5]], [[0.0, 0.0]]]])
    assert np.array_equal(y, expect), y
    # den = |x w| + |bias| + |residual|
    expect_den = np.array([[[[4.5, 16.5]], [[3.25, 10.25]]], [[[2.0, 13.5]], [[3.75, 4.75]]]])
    assert np.array_equal(den, expect_den), den


def pin_float_without_relu():
    x, w, bias, res = _worked_float()
    y, _ = oracle.conv2d_fused(x, w, bias, res, relu=False)
    expect = np.array([[[[2.5, 4.5]], [[0.75, -6.25]]], [[[2.0, 11.5]], [[-3.75, -3.75]]]])
    assert np.array_equal(y, expect), y


def pin_float_bias_only():
    x, w, bias, _ = _worked_float()
    y, den = oracle.conv2d_fused(x, w, bias)
    expect = np.array([[[[3.5, -5.5]], [[-1.25, 1.75]]], [[[2.0, 12.5]], [[-0.75, -4.25]]]])
    assert np.array_equal(y, expect), y
    expect_den = np.array([[[[3.5, 6.5]], [[1.25, 2.25]]], [[[2.0, 12.5]], [[0.75, 4.25]]]])
    assert np.array_equal(den, expect_den), den


def pin_float_no_epilogue_is_plain_conv():
    x, w, _, _ = _worked_float()
    y, den = oracle.conv2d_fused(x, w)
    y0, den0 = oracle.conv2d(x, w)
    assert np.array_equal(y, y0) and np.array_equal(den, den0)


def pin_int8_bias_before_scale():
    # (7 + 1) * 0.25 = 2; bias after the scaling would give 7*0.25 + 1 = 2.75 -> 3
    assert oracle.requant_epi_one(7, 0.25, bias=1) == 2
    # (100 + 28) * 0.5 = 64, + residual 3 = 67
    assert oracle.requant_epi_one(100, 0.5, bias=28, residual=3) == 67


def pin_int8_residual_after_scale():
    # 5 * 0.5 = 2.5 -> 2 (ties to even); + residual 1 -> 3.5 -> 4; the residual
    # added to the accumulator first would give (5 + 1) * 0.5 = 3
    assert oracle.requant_epi_one(5, 0.5) == 2
    assert oracle.requant_epi_one(5, 0.5, residual=1) == 4
    # 11 * 0.5 = 5.5, - 1 = 4.5 -> 4 (ties to even); the residual added to the
    # accumulator first would give (11 - 1) * 0.5 = 5
    assert oracle.requant_epi_one(11, 0.5, residual=-1) == 4
    assert oracle.requant_epi_one(11, 0.5) == 6  # 5.5 -> 6


def pin_int8_relu_floor():
    assert oracle.requant_epi_one(-100, 0.5, residual=10, relu=True) == 0
    assert oracle.requant_epi_one(-100, 0.5, residual=10) == -40
    assert oracle.requant_epi_one(-1000, 1.0) == -127
    assert oracle.requant_epi_one(-1000, 1.0, relu=True) == 0
    assert oracle.requant_epi_one(1000, 1.0, relu=True) == 127
    # -0.5 rounds to -0 -> 0 under either floor
    assert oracle.requant_epi_one(-1, 0.5, relu=True) == 0


def pin_int8_tensor_channels():
    # N=1, K=2, HW=2: bias and scale per output channel
    acc = np.array([[[10, -30], [4, 6]]], dtype=np.int64)
    scale = np.array([0.5, 2.0], dtype=np.float32)
    bias = np.array([-2, 1], dtype=np.int32)
    res = np.array([[[1, 2], [-20, 0]]], dtype=np.int8)
    y = oracle.requant_epi(acc, scale, bias, res, relu=False)
    # k0: (10-2)*0.5+1 = 5, (-30-2)*0.5+2 = -14; k1: (4+1)*2-20 = -10, (6+1)*2 = 14
    assert y.tolist() == [[[5, -14], [-10, 14]]], y.tolist()
    y = oracle.requant_epi(acc, scale, bias, res, relu=True)
    assert y.tolist() == [[[5, 0], [0, 14]]], y.tolist()


def pin_int8_bias_overflow_rejected():
    acc = np.array([[[2**31 - 10]]], dtype=np.int64)
    with pytest.raises(OverflowError):
        oracle.requant_epi(acc, np.array([1.0], np.float32), np.array([20], np.int32))


PINS = [pin_float_bias_residual_relu, pin_float_without_relu, pin_float_bias_only,
        pin_float_no_epilogue_is_plain_conv, pin_int8_bias_before_scale, pin_int8_residual_after_scale,
        pin_int8_relu_floor, pin_int8_tensor_channels, pin_int8_bias_overflow_rejected]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_epilogue_pin(pin):
    pin()
