"""Exact-rational Winograd minimal filtering F(m, r) -- TEST INFRASTRUCTURE ONLY.

The MegEngine inference article (aminer.cn research report), section
"Winograd", names F(2x2,3x3) and F(6x6,3x3) and describes the method as
trading multiplies for adds in three steps: transform the input tile and the
weights, multiply the transformed tiles element-wise (batched over tiles and
channels it becomes a batched matrix product), transform the product back.
It cites Lavin and Gray ("Fast algorithms for convolutional neural networks")
for the method; it gives no matrices and no interpolation points.

This module builds the three matrices from first principles, in exact
rationals (``fractions.Fraction``), so the tests can show that a given choice
of points yields an *exact* algorithm for correlation:

    linear convolution of u (m taps) with g (r taps) by evaluation at
    alpha = m + r - 1 points (one of them may be "infinity", which picks the
    leading coefficient) and interpolation:
        s = V^{-1} [ (V_r g) * (V_m u) ]
    correlation y_i = sum_j d_{i+j} g_j is the transpose of that linear map in
    u, hence
        y = V_m^T [ (V_r g) * (V^{-T} d) ],
    i.e. A^T = V_m^T (m x alpha), G = V_r (alpha x r), B^T = V^{-T}.
    2-D nesting: Y = A^T [ (G g G^T) * (B^T d B) ] A.

Points used (readings, the pages name none): {0, 1, -1, inf} for F(2,3) and
{0, 1, -1, 2, -2, 1/2, -1/2, inf} for F(6,3).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence, Union

INF = "inf"
Point = Union[Fraction, int, str]

POINTS_F2 = (0, 1, -1, INF)
POINTS_F6 = (0, 1, -1, 2, -2, Fraction(1, 2), Fraction(-1, 2), INF)

Matrix = List[List[Fraction]]


def _eval_matrix(points: Sequence[Point], ncoef: int) -> Matrix:
    """Rows evaluate a polynomial with ``ncoef`` coefficients at each point.

    The infinity point returns the leading coefficient.
    """
    rows = []
    for p in points:
        if p == INF:
            rows.append([Fraction(0)] * (ncoef - 1) + [Fraction(1)])
        else:
            q = Fraction(p)
            rows.append([q ** j for j in range(ncoef)])
    return rows


def _transpose(a: Matrix) -> Matrix:
    return [list(col) for col in zip(*a)]


def _matmul(a: Matrix, b: Matrix) -> Matrix:
    bt = _transpose(b)
    return [[sum((x * y for x, y in zip(row, col)), Fraction(0)) for col in bt] for row in a]


def _inverse(a: Matrix) -> Matrix:
    """Gauss-Jordan inverse over the rationals."""
    n = len(a)
    m = [list(row) + [Fraction(int(i == j)) for j in range(n)] for i, row in enumerate(a)]
    for col in range(n):
        piv = next(r for r in range(col, n) if m[r][col] != 0)
        m[col], m[piv] = m[piv], m[col]
        inv = 1 / m[col][col]
        m[col] = [v * inv for v in m[col]]
        for r in range(n):
            if r != col and m[r][col] != 0:
                f = m[r][col]
                m[r] = [vr - f * vc for vr, vc in zip(m[r], m[col])]
    return [row[n:] for row in m]


def matrices(m: int, r: int, points: Sequence[Point]):
    """Return (AT, G, BT) for F(m, r) built at the given alpha = m + r - 1 points."""
    alpha = m + r - 1
    if len(points) != alpha or len(set(points)) != alpha:
        raise ValueError("need %d distinct points" % alpha)
    v = _eval_matrix(points, alpha)
    vm = _eval_matrix(points, m)
    vr = _eval_matrix(points, r)
    at = _transpose(vm)
    g = vr
    bt = _transpose(_inverse(v))
    return at, g, bt


def correlate_1d(d: Sequence, g: Sequence, m: int) -> list:
    """Direct valid correlation y_i = sum_j d[i + j] g[j], i < m."""
    return [sum((Fraction(d[i + j]) * Fraction(g[j]) for j in range(len(g))), Fraction(0))
            for i in range(m)]


def winograd_1d(d: Sequence, g: Sequence, at: Matrix, gm: Matrix, bt: Matrix) -> list:
    dv = [[Fraction(v)] for v in d]
    gv = [[Fraction(v)] for v in g]
    u = _matmul(gm, gv)
    v = _matmul(bt, dv)
    mvec = [[u[i][0] * v[i][0]] for i in range(len(u))]
    return [row[0] for row in _matmul(at, mvec)]


def correlate_2d(d, g, m: int) -> Matrix:
    r = len(g)
    return [[sum((Fraction(d[i + a][j + b]) * Fraction(g[a][b]) for a in range(r) for b in range(r)),
                 Fraction(0)) for j in range(m)] for i in range(m)]


def winograd_2d(d, g, at: Matrix, gm: Matrix, bt: Matrix) -> Matrix:
    dq = [[Fraction(v) for v in row] for row in d]
    gq = [[Fraction(v) for v in row] for row in g]
    u = _matmul(_matmul(gm, gq), _transpose(gm))
    v = _matmul(_matmul(bt, dq), _transpose(bt))
    mm = [[u[i][j] * v[i][j] for j in range(len(u))] for i in range(len(u))]
    return _matmul(_matmul(at, mm), _transpose(at))


def multiplies_per_tile(m: int, r: int):
    """(element-wise multiplies of F(m x m, r x r), multiplies of direct correlation)."""
    alpha = m + r - 1
    return alpha * alpha, m * m * r * r
