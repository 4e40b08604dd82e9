"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test ties the oracle to something it does not compute itself: the worked
example printed in the convolution-summary blog post, closed-form output
sizes, an independent numpy im2col + matmul brute force, library routines
(torch CPU conv2d in float64, scipy correlate2d, numpy matmul), and exact
invariants (delta kernel, linearity, translation, conv <-> fully connected,
groups as concatenation).  Together they make a dropped term, a flipped
kernel, a wrong stride/padding/dilation/group index or a transposed operand in
the oracle fail at least one test (see test_oracle_mutations.py).
"""
import itertools
import os
import re
import zlib

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PRIMES = [2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41, 43, 47, 53, 59, 61, 67, 71, 73]


# ----------------------------------------------------------------- references

def im2col_conv(x, w, stride, pad, dil, groups, dtype):
    """Independent brute force: explicit im2col gather + one matmul per group."""
    N, C, H, W = x.shape
    K, Cg, R, S = w.shape
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    OH = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    OW = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    xp = np.zeros((N, C, H + 2 * ph, W + 2 * pw), dtype=dtype)
    xp[:, :, ph:ph + H, pw:pw + W] = x
    # cols[n, c, r, s, oh, ow]
    cols = np.empty((N, C, R, S, OH, OW), dtype=dtype)
    for r in range(R):
        for s in range(S):
            cols[:, :, r, s] = xp[:, :, r * dh: r * dh + sh * (OH - 1) + 1: sh,
                                  s * dw: s * dw + sw * (OW - 1) + 1: sw]
    Kg = K // groups
    y = np.empty((N, K, OH, OW), dtype=dtype)
    for g in range(groups):
        a = w[g * Kg:(g + 1) * Kg].reshape(Kg, Cg * R * S).astype(dtype)
        b = cols[:, g * Cg:(g + 1) * Cg].reshape(N, Cg * R * S, OH * OW)
        y[:, g * Kg:(g + 1) * Kg] = np.matmul(a, b).reshape(N, Kg, OH, OW)
    return y


def random_case(rng):
    groups_choice = rng.integers(0, 3)
    Cg = int(rng.integers(1, 4))
    if groups_choice == 0:
        G = 1
    elif groups_choice == 1:
        G = 2
    else:
        G = int(rng.integers(2, 5))  # depthwise-like when Cg == 1
    C = Cg * G
    K = G * int(rng.integers(1, 4))
    R = int(rng.choice([1, 3, 5, 7]))
    S = int(rng.choice([1, 3, 5, 7]))
    dh, dw = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    ph, pw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    H = int(rng.integers(max(1, dh * (R - 1) + 1 - 2 * ph), 18)) | 1
    W = int(rng.integers(max(1, dw * (S - 1) + 1 - 2 * pw), 18)) | 1
    N = int(rng.integers(1, 3))
    if oracle.output_size(H, R, sh, ph, dh) <= 0 or oracle.output_size(W, S, sw, pw, dw) <= 0:
        return None
    return dict(N=N, C=C, H=H, W=W, K=K, R=R, S=S, stride=(sh, sw), pad=(ph, pw), dil=(dh, dw), G=G)


def cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        c = random_case(rng)
        if c is not None:
            out.append(c)
    return out


# ------------------------------------------------------------ worked example

def load_worked_example():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "worked_example_stride2.txt"))
             if l.strip() and not l.startswith("#")]
    spec = {}
    outputs = []
    for l in lines:
        m = re.match(r"^(\d+) (\d+) = (.+)$", l)
        if m:
            outputs.append((int(m.group(1)), int(m.group(2)), m.group(3)))
        else:
            key, val = l.split(":", 1)
            spec[key.strip()] = val.strip()
    rows = [r.split() for r in spec["input_rows"].split("|")]
    krows = [r.split() for r in spec["kernel_rows"].split("|")]
    return spec, rows, krows, outputs


def test_worked_example_stride2():
    spec, rows, krows, outputs = load_worked_example()
    names = [v for r in rows for v in r] + [v for r in krows for v in r]
    val = dict(zip(names, PRIMES))
    x = np.array([[[[val[v] for v in r] for r in rows]]], dtype=np.float64)
    w = np.array([[[[val[v] for v in r] for r in krows]]], dtype=np.float64)
    stride = int(spec["stride"])
    y, den = oracle.conv2d(x, w, stride=stride, padding=int(spec["padding"]))
    assert list(y.shape[2:]) == [int(v) for v in spec["output_shape"].split()]
    for (i, j, expr) in outputs:
        expected = eval(expr, {}, dict(val))  # expression printed on the page
        assert y[0, 0, i, j] == expected
        assert den[0, 0, i, j] == expected  # all terms positive
    # the same example through the int8 path
    acc = oracle.conv2d_int8(x.astype(np.int8), w.astype(np.int8), stride=stride)
    for (i, j, expr) in outputs:
        assert acc[0, 0, i, j] == eval(expr, {}, dict(val))


def test_no_kernel_flip():
    """Correlation, not convolution: a one-hot kernel at (0, 0) reads input (oh, ow)."""
    x = np.arange(1, 26, dtype=np.float64).reshape(1, 1, 5, 5)
    w = np.zeros((1, 1, 3, 3))
    w[0, 0, 0, 0] = 1.0
    y, _ = oracle.conv2d(x, w)
    np.testing.assert_array_equal(y[0, 0], x[0, 0, :3, :3])


# ----------------------------------------------------------------- shapes

@pytest.mark.parametrize("inp,k,s,p,d,expected", [
    (4, 2, 2, 0, 1, 2),      # the blog's 4x4 -> 2x2 example
    (224, 3, 2, 1, 1, 112),  # MobileNet-style stem
    (224, 7, 2, 3, 1, 112),  # ResNet stem
    (56, 1, 2, 0, 1, 28),    # ResNet 1x1 stride-2 downsample
    (56, 3, 1, 1, 1, 56),    # "same" 3x3
    (10, 10, 1, 0, 1, 1),    # kernel as large as the input: fully connected
    (7, 3, 1, 0, 3, 1),      # dilation 3 spans 7
    (6, 3, 1, 0, 3, 0),      # ... and does not fit in 6
    (5, 3, 3, 1, 1, 2),
])
def test_output_size(inp, k, s, p, d, expected):
    assert oracle.output_size(inp, k, s, p, d) == expected


def test_invalid_problems_rejected():
    x = np.zeros((1, 4, 5, 5))
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((3, 2, 3, 3)), groups=2)  # K not divisible by G
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((2, 4, 7, 7)))  # kernel larger than input
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((2, 3, 3, 3)))  # C mismatch


# ------------------------------------------------------------- brute force

@pytest.mark.parametrize("case", cases(40, 1234), ids=lambda c: "N%(N)dC%(C)dH%(H)dW%(W)dK%(K)dR%(R)dS%(S)dG%(G)d" % c)
def test_vs_im2col_bruteforce(case):
    rng = np.random.default_rng(zlib.crc32(repr(sorted(case.items())).encode()))
    xs = (case["N"], case["C"], case["H"], case["W"])
    ws = (case["K"], case["C"] // case["G"], case["R"], case["S"])
    # integer path: exact
    xi = rng.integers(-127, 128, size=xs, dtype=np.int8)
    wi = rng.integers(-127, 128, size=ws, dtype=np.int8)
    acc = oracle.conv2d_int8(xi, wi, case["stride"], case["pad"], case["dil"], case["G"])
    ref = im2col_conv(xi.astype(np.int64), wi.astype(np.int64), case["stride"], case["pad"], case["dil"],
                      case["G"], np.int64)
    np.testing.assert_array_equal(acc, ref)
    # float path
    xf = rng.standard_normal(xs)
    wf = rng.standard_normal(ws)
    y, den = oracle.conv2d(xf, wf, case["stride"], case["pad"], case["dil"], case["G"])
    ref = im2col_conv(xf, wf, case["stride"], case["pad"], case["dil"], case["G"], np.float64)
    refden = im2col_conv(np.abs(xf), np.abs(wf), case["stride"], case["pad"], case["dil"], case["G"], np.float64)
    assert np.all(np.abs(y - ref) <= 1e-12 * np.maximum(refden, 1e-300))
    np.testing.assert_allclose(den, refden, rtol=1e-12, atol=0)


@pytest.mark.parametrize("case", cases(25, 99), ids=lambda c: "N%(N)dC%(C)dH%(H)dW%(W)dK%(K)dG%(G)d" % c)
def test_vs_torch_conv2d_fp64(case):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    xs = (case["N"], case["C"], case["H"], case["W"])
    ws = (case["K"], case["C"] // case["G"], case["R"], case["S"])
    xf = rng.uniform(-1, 1, xs)
    wf = rng.uniform(-1, 1, ws)
    y, den = oracle.conv2d(xf, wf, case["stride"], case["pad"], case["dil"], case["G"])
    ref = torch.nn.functional.conv2d(torch.from_numpy(xf), torch.from_numpy(wf), stride=case["stride"],
                                     padding=case["pad"], dilation=case["dil"], groups=case["G"]).numpy()
    assert y.shape == ref.shape
    assert np.all(np.abs(y - ref) <= 1e-12 * den + 1e-300)


def test_single_channel_is_scipy_correlate2d():
    signal = pytest.importorskip("scipy.signal")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 11))
    w = rng.standard_normal((3, 4))
    y, _ = oracle.conv2d(x[None, None], w[None, None])
    np.testing.assert_allclose(y[0, 0], signal.correlate2d(x, w, mode="valid"), rtol=1e-12, atol=1e-12)
    # "same"-style zero padding for an odd kernel
    w3 = rng.standard_normal((3, 3))
    y, _ = oracle.conv2d(x[None, None], w3[None, None], padding=1)
    np.testing.assert_allclose(y[0, 0], signal.correlate2d(x, w3, mode="same"), rtol=1e-12, atol=1e-12)


# ------------------------------------------------- textbook reductions

def test_1x1_is_matmul():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 6, 5, 7))
    w = rng.standard_normal((4, 6, 1, 1))
    y, _ = oracle.conv2d(x, w)
    ref = np.einsum("kc,ncp->nkp", w[:, :, 0, 0], x.reshape(2, 6, 35)).reshape(2, 4, 5, 7)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_kernel_as_large_as_input_is_fully_connected():
    """The blog's conv <-> FC equivalence: R=H, S=W, no padding is an FC layer."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, 3, 10, 10))
    w = rng.standard_normal((100, 3, 10, 10))
    y, _ = oracle.conv2d(x, w)
    assert y.shape == (3, 100, 1, 1)
    ref = x.reshape(3, 300) @ w.reshape(100, 300).T
    np.testing.assert_allclose(y[:, :, 0, 0], ref, rtol=1e-12, atol=1e-12)


def test_conv_is_sparse_fully_connected():
    """The blog's other direction: a 3x3 'same' conv on 10x10x3 -> 10x10x1 is an FC
    layer of 300 inputs whose weights are zero outside each 27-element window."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, 3, 10, 10))
    w = rng.standard_normal((1, 3, 3, 3))
    fc = np.zeros((100, 3, 10, 10))
    for oh in range(10):
        for ow in range(10):
            for c in range(3):
                for r in range(3):
                    for s in range(3):
                        ih, iw = oh - 1 + r, ow - 1 + s
                        if 0 <= ih < 10 and 0 <= iw < 10:
                            fc[oh * 10 + ow, c, ih, iw] = w[0, c, r, s]
    assert np.count_nonzero(fc[55]) == 27  # an interior output uses 27 of 300 inputs
    y, _ = oracle.conv2d(x, w, padding=1)
    np.testing.assert_allclose(y.reshape(100), fc.reshape(100, 300) @ x.reshape(300), rtol=1e-12, atol=1e-12)


def test_groups_are_concatenated_convolutions():
    rng = np.random.default_rng(14)
    G = 3
    x = rng.standard_normal((2, 6, 8, 9))
    w = rng.standard_normal((9, 2, 3, 3))
    y, _ = oracle.conv2d(x, w, stride=(1, 2), padding=1, groups=G)
    parts = [oracle.conv2d(x[:, 2 * g:2 * g + 2], w[3 * g:3 * g + 3], stride=(1, 2), padding=1)[0]
             for g in range(G)]
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=1))


def test_depthwise_is_per_channel_correlation():
    signal = pytest.importorskip("scipy.signal")
    rng = np.random.default_rng(15)
    x = rng.standard_normal((1, 4, 7, 8))
    w = rng.standard_normal((4, 1, 3, 3))
    y, _ = oracle.conv2d(x, w, padding=1, groups=4)
    for c in range(4):
        np.testing.assert_allclose(y[0, c], signal.correlate2d(x[0, c], w[c, 0], mode="same"),
                                   rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- invariants

@pytest.mark.parametrize("R,S", [(1, 1), (3, 3), (5, 3), (7, 7)])
def test_delta_kernel_is_identity(R, S):
    rng = np.random.default_rng(16)
    C = 5
    x = rng.standard_normal((2, C, 9, 8))
    w = np.zeros((C, C, R, S))
    for c in range(C):
        w[c, c, R // 2, S // 2] = 1.0
    y, _ = oracle.conv2d(x, w, padding=(R // 2, S // 2))
    np.testing.assert_array_equal(y, x)
    xi = rng.integers(-127, 128, size=(2, C, 9, 8), dtype=np.int8)
    acc = oracle.conv2d_int8(xi, w.astype(np.int8), padding=(R // 2, S // 2))
    np.testing.assert_array_equal(acc, xi.astype(np.int64))
    np.testing.assert_array_equal(oracle.requant(acc, np.ones(C, np.float32)), xi)


def test_linearity_exact():
    rng = np.random.default_rng(17)
    x1 = rng.integers(-40, 41, size=(2, 4, 9, 9))
    x2 = rng.integers(-40, 41, size=(2, 4, 9, 9))
    w = rng.integers(-127, 128, size=(3, 4, 3, 3))
    a, b = 2, -1
    lhs = oracle.conv2d_int8((a * x1 + b * x2).astype(np.int8), w.astype(np.int8), stride=2, padding=1)
    rhs = a * oracle.conv2d_int8(x1.astype(np.int8), w.astype(np.int8), stride=2, padding=1) + \
        b * oracle.conv2d_int8(x2.astype(np.int8), w.astype(np.int8), stride=2, padding=1)
    np.testing.assert_array_equal(lhs, rhs)
    # linearity in the weights too, through the fp64 path (integers are exact)
    w1 = rng.integers(-50, 51, size=(3, 4, 3, 3)).astype(np.float64)
    w2 = rng.integers(-50, 51, size=(3, 4, 3, 3)).astype(np.float64)
    xf = x1.astype(np.float64)
    lhs, _ = oracle.conv2d(xf, 3 * w1 - 2 * w2, padding=1)
    rhs = 3 * oracle.conv2d(xf, w1, padding=1)[0] - 2 * oracle.conv2d(xf, w2, padding=1)[0]
    np.testing.assert_array_equal(lhs, rhs)


def test_translation_equivariance():
    """Stride 1, no padding: shifting the input shifts the output (interior)."""
    rng = np.random.default_rng(18)
    x = rng.integers(-127, 128, size=(1, 3, 14, 15), dtype=np.int8)
    w = rng.integers(-127, 128, size=(2, 3, 3, 5), dtype=np.int8)
    full = oracle.conv2d_int8(x, w)
    dy, dx = 2, 3
    shifted = oracle.conv2d_int8(np.ascontiguousarray(x[:, :, dy:, dx:]), w)
    np.testing.assert_array_equal(shifted, full[:, :, dy:, dx:])


def test_den_properties():
    rng = np.random.default_rng(19)
    x = rng.standard_normal((2, 4, 7, 7))
    w = rng.standard_normal((3, 4, 3, 3))
    y, den = oracle.conv2d(x, w, padding=2, dilation=2)
    assert np.all(den >= np.abs(y))
    y2, den2 = oracle.conv2d(np.abs(x), np.abs(w), padding=2, dilation=2)
    np.testing.assert_allclose(den, y2, rtol=1e-12)
    np.testing.assert_allclose(den2, y2, rtol=1e-12)
    # an output that sees only padding has den == 0 and y == 0
    y3, den3 = oracle.conv2d(np.ones((1, 1, 2, 2)), np.ones((1, 1, 1, 1)), padding=1)
    assert den3[0, 0, 0, 0] == 0 and y3[0, 0, 0, 0] == 0
    assert den3[0, 0, 1, 1] == 1


def test_int8_and_fp64_paths_agree_exactly():
    rng = np.random.default_rng(20)
    x = rng.integers(-127, 128, size=(2, 6, 9, 10), dtype=np.int8)
    w = rng.integers(-127, 128, size=(4, 3, 3, 3), dtype=np.int8)
    acc = oracle.conv2d_int8(x, w, stride=(2, 1), padding=1, groups=2)
    y, _ = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), stride=(2, 1), padding=1, groups=2)
    np.testing.assert_array_equal(acc, y.astype(np.int64))


def test_points_match_full():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 4, 9, 9))
    w = rng.standard_normal((6, 2, 3, 3))
    y, den = oracle.conv2d(x, w, stride=2, padding=1, groups=2)
    idx = np.array(list(itertools.product(range(2), range(6), range(5), range(5))))
    yp, dp = oracle.conv2d_points(x, w, idx, stride=2, padding=1, groups=2)
    np.testing.assert_array_equal(yp, y.reshape(-1))
    np.testing.assert_array_equal(dp, den.reshape(-1))
    xi = rng.integers(-127, 128, size=(2, 4, 9, 9), dtype=np.int8)
    wi = rng.integers(-127, 128, size=(6, 2, 3, 3), dtype=np.int8)
    acc = oracle.conv2d_int8(xi, wi, stride=2, padding=1, groups=2)
    ap = oracle.conv2d_int8_points(xi, wi, idx, stride=2, padding=1, groups=2)
    np.testing.assert_array_equal(ap, acc.reshape(-1))
    with pytest.raises(ValueError):
        oracle.conv2d_points(x, w, np.array([[0, 6, 0, 0]]), stride=2, padding=1, groups=2)


# ---------------------------------------------------------------- requant

def test_requant_ties_to_even():
    assert [oracle.requant_one(a, 0.5) for a in (3, 5, -3, 1, -1, 7)] == [2, 2, -2, 0, 0, 4]
    assert [oracle.requant_one(a, 0.25) for a in (2, 6, 10, -6)] == [0, 2, 2, -2]


def test_requant_saturates_symmetrically():
    assert oracle.requant_one(1000, 1.0) == 127
    assert oracle.requant_one(-1000, 1.0) == -127  # never -128
    assert oracle.requant_one(254, 0.5) == 127
    assert oracle.requant_one(-255, 0.5) == -127   # -127.5 -> -128 by rne, clamped to -127
    assert oracle.requant_one(2**31 - 1, 1.0) == 127


def test_requant_converts_acc_to_fp32_first():
    """fp32(acc) is rounded before the multiply: 2^25 + 2^19 + 1 becomes
    2^25 + 2^19 in fp32, so acc * 2^-20 = 32.5 rounds (ties to even) to 32,
    where the exact product 32.50000095 would give 33."""
    acc = 2**25 + 2**19 + 1
    assert float(np.float32(acc)) == 2**25 + 2**19
    assert oracle.requant_one(acc, 2.0**-20) == 32
    assert oracle.requant_one(acc + 4, 2.0**-20) == 33
    # 2^30 + 63 becomes 2^30 in fp32; with the scale one fp32 step below
    # 63.5 * 2^-30 the fp32 product is exactly 63.5 - 2^-18 -> 63, while the
    # exact product, 63.5 - 9e-8, would round to the fp32 value 63.5 -> 64
    acc = 2**30 + 63
    scale = 127 * 2.0**-31 - 2.0**-48
    assert float(np.float32(scale)) == scale and float(np.float32(acc)) == 2**30
    assert oracle.requant_one(acc, scale) == 63


def test_requant_array_matches_scalar_rule():
    rng = np.random.default_rng(22)
    acc = rng.integers(-2**20, 2**20, size=(2, 3, 4, 5))
    scale = rng.uniform(1e-5, 1e-3, size=3).astype(np.float32)
    y = oracle.requant(acc, scale)
    for idx in itertools.product(range(2), range(3), range(4), range(5)):
        assert y[idx] == oracle.requant_one(int(acc[idx]), float(scale[idx[1]]))
    with pytest.raises(OverflowError):
        oracle.requant(np.full((1, 1, 1), 2**31), np.ones(1, np.float32))


def test_int8_accumulator_bound_for_resnet18():
    """127^2 * C * R * S < 2^31 for every int8 ResNet-18 layer: int32 accumulation is exact."""
    from cnn_convolution_fwd_amd.workloads import resnet18_layers
    worst = max(127 * 127 * (L.c // L.groups) * L.r * L.s for L in resnet18_layers())
    assert worst == 127 * 127 * 512 * 9 == 74_322_432
    assert worst < 2**31
