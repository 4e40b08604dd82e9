"""Pins of the oracle's bottleneck block (CPU only).

The block (Momenta talk, sections "優化1：Bottleneck" and "Operator的粒度"):
1x1 C -> M, 3x3 M -> M with zero padding 1, 1x1 M -> K, stride 1, each
convolution followed by its epilogue (bias, the residual at the end, ReLU).
Pinned against: an independent pure-Python loop nest on tiny shapes (every
epilogue combination), the closed form of a block whose 3x3 is the identity
(a product of the two 1x1 weight matrices, by numpy's matmul), and the
normaliser's defining properties.
"""
import itertools

import numpy as np
import pytest

import oracle


def _block_loops(x, w1, w2, w3, b1, b2, b3, res, relu):
    """The block written as plain loops, straight from its definition."""
    N, C, H, W = x.shape
    M, K = w1.shape[0], w3.shape[0]
    act = [lambda v, r=r: max(v, 0.0) if r else v for r in relu]
    t1 = [[[[0.0] * W for _ in range(H)] for _ in range(M)] for _ in range(N)]
    for n, m, h, ww in itertools.product(range(N), range(M), range(H), range(W)):
        s = sum(float(x[n, c, h, ww]) * float(w1[m, c, 0, 0]) for c in range(C))
        t1[n][m][h][ww] = act[0](s + (float(b1[m]) if b1 is not None else 0.0))
    t2 = [[[[0.0] * W for _ in range(H)] for _ in range(M)] for _ in range(N)]
    for n, m2, h, ww in itertools.product(range(N), range(M), range(H), range(W)):
        s = 0.0
        for m, r, q in itertools.product(range(M), range(3), range(3)):
            ih, iw = h + r - 1, ww + q - 1
            if 0 <= ih < H and 0 <= iw < W:
                s += t1[n][m][ih][iw] * float(w2[m2, m, r, q])
        t2[n][m2][h][ww] = act[1](s + (float(b2[m2]) if b2 is not None else 0.0))
    y = np.zeros((N, K, H, W))
    for n, k, h, ww in itertools.product(range(N), range(K), range(H), range(W)):
        s = sum(t2[n][m][h][ww] * float(w3[k, m, 0, 0]) for m in range(M))
        s += float(b3[k]) if b3 is not None else 0.0
        s += float(res[n, k, h, ww]) if res is not None else 0.0
        y[n, k, h, ww] = act[2](s)
    return y


@pytest.mark.parametrize("relu", list(itertools.product([False, True], repeat=3)))
@pytest.mark.parametrize("with_bias,with_res", [(False, False), (True, False), (True, True), (False, True)])
def test_block_matches_loop_nest(relu, with_bias, with_res):
    rng = np.random.default_rng(sum(relu) * 7 + with_bias * 2 + with_res)
    N, C, M, K, H, W = 2, 3, 2, 3, 4, 5
    x = rng.uniform(-1, 1, (N, C, H, W))
    w1 = rng.uniform(-1, 1, (M, C, 1, 1))
    w2 = rng.uniform(-1, 1, (M, M, 3, 3))
    w3 = rng.uniform(-1, 1, (K, M, 1, 1))
    b1, b2, b3 = (rng.uniform(-1, 1, M), rng.uniform(-1, 1, M), rng.uniform(-1, 1, K)) if with_bias else (None,) * 3
    res = rng.uniform(-1, 1, (N, K, H, W)) if with_res else None
    y, den = oracle.bottleneck(x, w1, w2, w3, b1, b2, b3, res, relu)
    ref = _block_loops(x, w1, w2, w3, b1, b2, b3, res, relu)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.all(den >= np.abs(y) - 1e-12)


def test_identity_middle_is_product_of_1x1_weights():
    """With the 3x3 the identity (centre tap 1 on the diagonal) and no
    epilogue, the block is one 1x1 convolution with weights w3 @ w1."""
    rng = np.random.default_rng(5)
    N, C, M, K, H, W = 2, 8, 4, 6, 5, 7
    x = rng.standard_normal((N, C, H, W))
    w1 = rng.standard_normal((M, C, 1, 1))
    w3 = rng.standard_normal((K, M, 1, 1))
    w2 = np.zeros((M, M, 3, 3))
    for m in range(M):
        w2[m, m, 1, 1] = 1.0
    y, _ = oracle.bottleneck(x, w1, w2, w3)
    wk = w3[:, :, 0, 0] @ w1[:, :, 0, 0]                      # [K, C]
    ref = np.matmul(wk, x.reshape(N, C, H * W)).reshape(N, K, H, W)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_normaliser_equals_value_for_nonnegative_data():
    """All inputs, weights, biases and the residual non-negative: no term
    cancels, so the chained normaliser equals the value itself."""
    rng = np.random.default_rng(9)
    N, C, M, K, H, W = 1, 4, 3, 5, 6, 6
    x = rng.uniform(0, 1, (N, C, H, W))
    w1, w2, w3 = rng.uniform(0, 1, (M, C, 1, 1)), rng.uniform(0, 1, (M, M, 3, 3)), rng.uniform(0, 1, (K, M, 1, 1))
    b1, b2, b3 = rng.uniform(0, 1, M), rng.uniform(0, 1, M), rng.uniform(0, 1, K)
    res = rng.uniform(0, 1, (N, K, H, W))
    y, den = oracle.bottleneck(x, w1, w2, w3, b1, b2, b3, res, (True, True, True))
    np.testing.assert_allclose(den, y, rtol=1e-12)


def test_corner_sees_only_its_window():
    """An impulse in the corner of t1's input reaches only the 2x2 outputs its
    3x3 window covers (zero padding, no wrap-around)."""
    N, C, M, K, H, W = 1, 1, 1, 1, 6, 7
    x = np.zeros((N, C, H, W))
    x[0, 0, 0, 0] = 1.0
    ones = lambda *s: np.ones(s)  # noqa: E731
    y, _ = oracle.bottleneck(x, ones(M, C, 1, 1), ones(M, M, 3, 3), ones(K, M, 1, 1))
    nz = np.argwhere(y[0, 0] != 0)
    assert sorted(map(tuple, nz)) == [(0, 0), (0, 1), (1, 0), (1, 1)]
