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


def test_f2_int8_operands_exact_in_fp16():
    """int8 Winograd F(2x2) with a float intermediate (MegEngine Beta release
    article, section "业界领先的原生 ARM 推理性能"): with the points
    {0, 1, -1, inf}, G = V_3 is integer and B^T has entries 0, +-1/2, +-1, so
    for int8 inputs (-128 .. 127) every B^T d B is a multiple of 1/4 with
    magnitude <= 512 and every G g G^T an integer with magnitude <= 1152.
    Both sets are exact in fp16, and each product is exact in fp32: the only
    rounding left is in the fp32 sums."""
    at, g, bt = wr.matrices(2, 3, wr.POINTS_F2)
    bt_abs = [[abs(v) for v in row] for row in bt]
    g_abs = [[abs(v) for v in row] for row in g]
    # bound on each transformed position: every input of magnitude 128 with
    # the sign of its coefficient (int8 holds 128 only as -128, so the true
    # maximum is a little lower; the bound is what the fp16 check needs)
    u_max = max(sum(bt_abs[i][k] * bt_abs[j][l] for k in range(4) for l in range(4)) * 128
                for i in range(4) for j in range(4))
    v_max = max(sum(g_abs[i][r] * g_abs[j][s] for r in range(3) for s in range(3)) * 128
                for i in range(4) for j in range(4))
    assert u_max == 512 and v_max == 1152
    # denominators: B^T d B in quarters, G g G^T integral
    for i in range(4):
        for j in range(4):
            for k in range(4):
                for l in range(4):
                    assert (4 * bt[i][k] * bt[j][l]).denominator == 1
    assert all(Fraction(v).denominator == 1 for row in g for v in row)
    # a worst-case int8 tile, through the rational path, stays within it
    i, j = 0, 0
    d = [[-128 if bt[i][k] * bt[j][l] < 0 else 127 for l in range(4)] for k in range(4)]
    u = wr._matmul(wr._matmul(bt, [[Fraction(v) for v in row] for row in d]), wr._transpose(bt))
    assert abs(u[0][0]) <= 512 and all((4 * v).denominator == 1 for row in u for v in row)
    # every representable value is exact in fp16, every product in fp32
    quarters = np.arange(-2048, 2049, dtype=np.float64) / 4.0
    assert np.array_equal(quarters.astype(np.float16).astype(np.float64), quarters)
    ints = np.arange(-1152, 1153, dtype=np.float64)
    assert np.array_equal(ints.astype(np.float16).astype(np.float64), ints)
    prod_max_quarters = 2048 * 1152
    assert prod_max_quarters < 2 ** 24


def test_f2_int8_float_sums_exact_below_2_22():
    """The int8 F(2x2) result is exact while every fp32 partial sum stays below
    2^22: in units of 1/4 that is below 2^24, where fp32 holds every integer.
    Checked by carrying a small problem through fp16 operands and fp32 sums in
    numpy and comparing with exact integer correlation (brute force)."""
    at, g, bt = wr.matrices(2, 3, wr.POINTS_F2)
    AT = np.array([[float(v) for v in row] for row in at])
    G = np.array([[float(v) for v in row] for row in g])
    BT = np.array([[float(v) for v in row] for row in bt])
    rng = np.random.default_rng(22)
    C = 24
    d = rng.integers(-128, 128, (C, 4, 4))
    w = rng.integers(-128, 128, (C, 3, 3))
    U = np.einsum("ik,ckl,jl->cij", BT, d.astype(np.float64), BT).astype(np.float16)
    V = np.einsum("ir,crs,js->cij", G, w.astype(np.float64), G).astype(np.float16)
    M = np.zeros((4, 4), dtype=np.float32)
    for c in range(C):  # fp32 sums, one channel at a time
        M = (M + U[c].astype(np.float32) * V[c].astype(np.float32)).astype(np.float32)
    assert np.abs(M).max() < 2 ** 22
    Y = (AT.astype(np.float32) @ M @ AT.T.astype(np.float32)).astype(np.float32)
    exact = np.array([[sum(int(d[c, i + r, j + s]) * int(w[c, r, s]) for c in range(C) for r in range(3)
                           for s in range(3)) for j in range(2)] for i in range(2)])
    assert np.array_equal(np.rint(Y).astype(np.int64), exact)
    assert np.array_equal(Y.astype(np.float64), exact.astype(np.float64))
