"""Pins of the float pass/fail metric ``oracle.normalised_error`` (CPU only).

The metric (the reading of the tolerance used by every float parity test):
err = max_i |y_hat_i - y_i| / den_i with den_i = sum |x * w| over output i's
terms; an output with den_i = 0 has only zero terms, so it must be exactly 0
(else err = +inf); a NaN or infinity anywhere in y_hat gives +inf.

Every expected value below is worked out by hand.  The second half plants
plausible slips in a copy of the function (dividing by max(den), inverting
the den = 0 rule, dropping the absolute value, averaging instead of taking
the maximum, letting NaN through, ...) and checks that at least one pin
catches each.
"""
import inspect
import math

import numpy as np
import pytest

import oracle


def pin_per_element_division(f):
    # errors 0.5 / 0.5 = 1.0 and 0 / 10 = 0: the maximum is 1.0.  Dividing by
    # max(den) would give 0.05, dividing the max deviation by the mean den 0.095.
    got = f([1.0, 2.0], [1.5, 2.0], [0.5, 10.0])
    assert got == 1.0, got


def pin_maximum_not_mean(f):
    # per-output errors 0.25, 0.0, 0.75 -> 0.75 (mean 1/3, sum 1.0)
    got = f([1.25, 3.0, -1.0], [1.0, 3.0, -0.25], [1.0, 4.0, 1.0])
    assert got == 0.75, got


def pin_absolute_deviation(f):
    # y_hat below y: |0 - 1| / 2 = 0.5 (a signed deviation would give -0.5)
    got = f([0.0], [1.0], [2.0])
    assert got == 0.5, got


def pin_zero_den_ignored(f):
    # den = 0 with y_hat = 0 is left out: only |3 - 2| / 2 counts
    got = f([0.0, 3.0], [0.0, 2.0], [0.0, 2.0])
    assert got == 0.5, got


def pin_zero_den_nonzero_output(f):
    # den = 0 but y_hat != 0 (even a tiny value) is an outright failure
    got = f([1e-30, 2.0], [0.0, 2.0], [0.0, 2.0])
    assert got == math.inf, got


def pin_all_zero_den(f):
    got = f(np.zeros((2, 3)), np.zeros((2, 3)), np.zeros((2, 3)))
    assert got == 0.0, got


def pin_nan_fails(f):
    got = f([np.nan, 1.0], [1.0, 1.0], [1.0, 1.0])
    assert got == math.inf, got
    got = f([1.0, np.nan], [1.0, 0.0], [1.0, 0.0])
    assert got == math.inf, got


def pin_inf_fails(f):
    got = f([np.inf], [1.0], [1.0])
    assert got == math.inf, got


def pin_multidimensional(f):
    # the metric is over every element of an [N, K, OH, OW] tensor
    y = np.zeros((2, 2, 2, 2))
    den = np.ones((2, 2, 2, 2))
    y_hat = y.copy()
    y_hat[1, 0, 1, 1] = 0.125
    y_hat[0, 1, 0, 0] = -0.0625
    got = f(y_hat, y, den)
    assert got == 0.125, got


def pin_shape_mismatch_rejected(f):
    with pytest.raises(ValueError):
        f(np.zeros(3), np.zeros(4), np.ones(4))


PINS = [pin_per_element_division, pin_maximum_not_mean, pin_absolute_deviation, pin_zero_den_ignored,
        pin_zero_den_nonzero_output, pin_all_zero_den, pin_nan_fails, pin_inf_fails, pin_multidimensional,
        pin_shape_mismatch_rejected]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_metric_pin(pin):
    pin(oracle.normalised_error)


# ------------------------------------------------------------ planted slips

SLIPS = {
    "divide_by_max_den": ("/ den[nz]))", "/ np.max(den)))"),
    "mean_not_max": ("return float(np.max(np.abs(", "return float(np.mean(np.abs("),
    "signed_deviation": ("np.abs(y_hat[nz] - y[nz])", "(y_hat[nz] - y[nz])"),
    "zero_den_rule_inverted": ("if np.any(y_hat[zero] != 0):", "if np.any(y_hat[zero] == 0):"),
    "zero_den_not_checked": ("if np.any(y_hat[zero] != 0):", "if False:"),
    "nan_let_through": ("if not np.all(np.isfinite(y_hat)):", "if False:"),
    "nan_and_zero_den_unchecked": ("if not np.all(np.isfinite(y_hat)):\n        return float(\"inf\")\n"
                                   "    zero = den == 0\n    if np.any(y_hat[zero] != 0):",
                                   "zero = den == 0\n    if False:"),
    "all_zero_returns_inf": ("if np.all(zero):\n        return 0.0", "if np.all(zero):\n        return float('inf')"),
    "relative_to_y": ("/ den[nz]))", "/ np.maximum(np.abs(y[nz]), 1.0)))"),
    "shape_not_checked": ("if y_hat.shape != y.shape or y.shape != den.shape:", "if False:"),
}


def planted(old, new):
    src = inspect.getsource(oracle.normalised_error)
    assert old in src, "slip pattern %r no longer matches normalised_error" % old
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["normalised_error"]


@pytest.mark.parametrize("name", sorted(SLIPS))
def test_planted_slip_is_caught(name):
    f = planted(*SLIPS[name])
    caught = []
    for pin in PINS:
        try:
            pin(f)
        except (AssertionError, ValueError, IndexError, FloatingPointError, TypeError):
            caught.append(pin.__name__)
        except BaseException as e:  # pytest.raises failing counts as caught too
            if type(e).__name__ == "Failed":
                caught.append(pin.__name__)
            else:
                raise
    assert caught, "planted slip %r was not caught by any metric pin" % name
