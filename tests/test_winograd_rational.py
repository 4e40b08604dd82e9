"""Winograd minimal filtering in exact rationals (CPU only).

The MegEngine inference article (section "Winograd") names F(2x2,3x3) and
F(6x6,3x3), says they cut multiplies by 2.25x and 5.06x, and describes the
three steps (transform, batched element-wise product, inverse transform).
These tests pin that the matrices built from the chosen interpolation points
compute correlation *exactly*, in 1-D and nested 2-D, and that the multiply
counts are the ones the article quotes.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import winograd_rational as wr


@pytest.mark.parametrize("m,points", [(2, wr.POINTS_F2), (6, wr.POINTS_F6),
                                      (4, (0, 1, -1, 2, -2, wr.INF))])
def test_1d_exact(m, points):
    at, g, bt = wr.matrices(m, 3, points)
    rng = np.random.default_rng(m)
    for _ in range(20):
        d = [int(v) for v in rng.integers(-50, 51, m + 2)]
        k = [int(v) for v in rng.integers(-50, 51, 3)]
        assert wr.winograd_1d(d, k, at, g, bt) == wr.correlate_1d(d, k, m)


@pytest.mark.parametrize("m,points", [(2, wr.POINTS_F2), (6, wr.POINTS_F6)])
def test_2d_exact(m, points):
    at, g, bt = wr.matrices(m, 3, points)
    rng = np.random.default_rng(10 + m)
    for _ in range(3):
        d = rng.integers(-20, 21, (m + 2, m + 2)).tolist()
        k = [[Fraction(int(v), 7) for v in row] for row in rng.integers(-20, 21, (3, 3))]
        assert wr.winograd_2d(d, k, at, g, bt) == wr.correlate_2d(d, k, m)


def test_multiply_counts():
    m2, d2 = wr.multiplies_per_tile(2, 3)
    m6, d6 = wr.multiplies_per_tile(6, 3)
    assert (m2, d2) == (16, 36)
    assert (m6, d6) == (64, 324)
    assert Fraction(d2, m2) == Fraction(9, 4)          # "2.25x"
    assert round(d6 / m6, 2) == 5.06                    # "5.06x"
    # asymptotic bound r^2 = 9 for 3x3 kernels ("up to 9x" in the Momenta talk)
    assert all(Fraction(m * m * 9, (m + 2) ** 2) < 9 for m in range(1, 64))


def test_f2_matrices_shape_and_values():
    at, g, bt = wr.matrices(2, 3, wr.POINTS_F2)
    assert at == [[1, 1, 1, 0], [0, 1, -1, 1]]
    assert g == [[1, 0, 0], [1, 1, 1], [1, -1, 1], [0, 0, 1]]
    half = Fraction(1, 2)
    assert bt == [[1, 0, -1, 0], [0, half, half, 0], [0, -half, half, 0], [0, -1, 0, 1]]


def test_f6_transform_magnitudes():
    """Large transform entries are why F(6x6) loses precision (max |A^T| = 32)."""
    at, g, bt = wr.matrices(6, 3, wr.POINTS_F6)
    assert max(abs(v) for r in at for v in r) == 32
    assert max(abs(v) for r in bt for v in r) == Fraction(21, 4)


def test_wrong_points_break_exactness():
    """A repeated point or a dropped infinity point does not give an algorithm."""
    with pytest.raises(ValueError):
        wr.matrices(2, 3, (0, 1, 1, wr.INF))
    at, g, bt = wr.matrices(2, 3, (0, 1, -1, 2))  # finite points only: still exact
    d, k = [3, -1, 4, 1], [5, -9, 2]
    assert wr.winograd_1d(d, k, at, g, bt) == wr.correlate_1d(d, k, 2)
    bad_bt = [row[:] for row in bt]
    bad_bt[1][1] += 1
    assert wr.winograd_1d(d, k, at, g, bad_bt) != wr.correlate_1d(d, k, 2)
