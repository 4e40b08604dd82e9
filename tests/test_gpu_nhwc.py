"""GPU parity of the NHWC path: the NHWC implicit GEMM against the oracle, and
cfwd_convert_layout between NCHW, NHWC and NCHWX.

MegEngine CPU-inference article, section "结论": a network-wide mixed choice
of layouts is named as the next step; it needs kernels per layout and
conversions between them.  The oracle works on logical NCHW; NHWC tensors
are transposed with numpy (workloads.to_nhwc / from_nhwc, pinned in
test_layout_np.py).  Bars: the single-layer tolerances (fp32 1e-5, bf16 1e-2
normalised error); conversions are copies, so bit-exact.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from cnn_convolution_fwd_amd import binding as B
from cnn_convolution_fwd_amd.workloads import (Layer, epilogue_inputs, float_problem, from_nhwc, pack_nchwx,
                                                random_float_problem, to_nhwc, unpack_nchwx)
from tests.gpu_util import TOL, from_device, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SHAPES = [
    # name, N, C, H, W, K, R, S, stride, pad, dil
    ("3x3_c40_k70", 2, 40, 13, 17, 70, 3, 3, 1, 1, 1),     # ragged channel chunk, ragged K, pixels past a tile
    ("3x3_s2_k200", 1, 64, 15, 30, 200, 3, 3, 2, 1, 1),   # two K tiles, stride 2
    ("1x1_c256", 2, 256, 8, 8, 64, 1, 1, 1, 0, 1),        # eight chunks
    ("5x5_d2", 1, 24, 15, 14, 20, 5, 5, 1, 4, 2),         # dilation, wide padding
    ("7x7_s2_c8", 2, 8, 20, 22, 36, 7, 7, 2, 3, 1),       # stem-like, one small chunk
    ("1px", 1, 16, 1, 1, 8, 1, 1, 1, 0, 1),               # one output pixel
]


def run_nhwc(x, w, dtype, st, pd, dl, bias=None, res=None, relu=False, cfg=-1):
    torch = torch_cuda()
    xd = to_device(to_nhwc(x), dtype)
    wd = to_device(w, dtype)
    bd = torch.from_numpy(bias).cuda() if bias is not None else None
    rd = to_device(to_nhwc(res), dtype) if res is not None else None
    y = B.conv2d_fwd(xd, wd, st, pd, dl, 1, "NHWC", algo_kind="implicit_gemm" if cfg >= 0 else "auto", config_id=cfg,
                     bias=bd, residual=rd, relu=relu)
    return from_nhwc(from_device(y, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_nhwc_conv(case, dtype):
    name, N, C, H, W, K, R, S, st, pd, dl = case
    L = Layer(name, C, K, H, W, R, S, 1, 0, 1, 1)
    pr = random_float_problem(L, N, dtype, zlib.crc32((name + dtype + "nhwc").encode()))
    x_nhwc = to_device(to_nhwc(pr.x), dtype)
    desc = B.desc_for(x_nhwc, to_device(pr.w, dtype), st, pd, dl, 1, "NHWC")
    cands = [(a.kind, a.config_id) for a in B.list_candidates(desc)]
    assert cands and all(k == B.ALGO_IMPLICIT_GEMM for k, _ in cands), cands
    ref, den = oracle.conv2d(pr.x, pr.w, st, pd, dl, 1)
    for _, cfg in cands:
        say("nhwc", name, dtype, "config", cfg)
        y = run_nhwc(pr.x, pr.w, dtype, st, pd, dl, cfg=cfg)
        err = oracle.normalised_error(y, ref, den)
        say("  normalised error %.3g" % err)
        assert err <= TOL[dtype], "%s %s config %d: %.3g" % (name, dtype, cfg, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nhwc_epilogue(dtype):
    N, C, H, W, K = 2, 48, 11, 13, 72
    L = Layer("epi", C, K, H, W, 3, 3, 1, 1, 1, 1)
    pr = random_float_problem(L, N, dtype, 91)
    epi = epilogue_inputs((N, K, H, W), dtype, 92)
    ref, den = oracle.conv2d_fused(pr.x, pr.w, epi.bias, epi.residual, True, 1, 1)
    xd = to_device(to_nhwc(pr.x), dtype)
    for a in B.list_candidates(B.desc_for(xd, to_device(pr.w, dtype), 1, 1, 1, 1, "NHWC")):
        y = run_nhwc(pr.x, pr.w, dtype, 1, 1, 1, epi.bias, epi.residual, True, cfg=a.config_id)
        err = oracle.normalised_error(y, ref, den)
        say("nhwc epilogue", dtype, a.config_id, "%.3g" % err)
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nhwc_resnet3x3_full_size(dtype):
    """The ResNet 3x3 256-channel layer (N=32, 56x56) in NHWC, whole tensor."""
    pr = float_problem(3, 0, dtype=dtype)
    ref, den = oracle.conv2d(pr.x, pr.w, 1, 1)
    xd = to_device(to_nhwc(pr.x), dtype)
    for a in B.list_candidates(B.desc_for(xd, to_device(pr.w, dtype), 1, 1, 1, 1, "NHWC")):
        say("nhwc resnet3x3 full", dtype, "config", a.config_id)
        y = run_nhwc(pr.x, pr.w, dtype, 1, 1, 1, cfg=a.config_id)
        err = oracle.normalised_error(y, ref, den)
        say("  normalised error %.3g" % err)
        assert err <= TOL[dtype]


def test_nhwc_fastrun_gate_uses_converted_reference():
    """Fast-Run on an NHWC problem: its reference runs on x converted to NCHW
    and is converted back; the one candidate passes the gate and lands in the map."""
    torch = torch_cuda()
    B.fastrun_clear()
    L = Layer("fr", 32, 48, 12, 12, 3, 3, 1, 1, 1, 1)
    pr = random_float_problem(L, 2, "f32", 5)
    xd, wd = to_device(to_nhwc(pr.x), "f32"), to_device(pr.w, "f32")
    best, y = B.fastrun_select(xd, wd, 1, 1, 1, 1, "NHWC")
    ref, den = oracle.conv2d(pr.x, pr.w, 1, 1)
    assert oracle.normalised_error(from_nhwc(from_device(y, "f32")), ref, den) <= TOL["f32"]
    assert best.kind == B.ALGO_IMPLICIT_GEMM
    assert B.fastrun_lookup(B.desc_for(xd, wd, 1, 1, 1, 1, "NHWC")).key() == best.key()
    B.fastrun_clear()
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("C", [5, 32, 70])
def test_convert_layout_roundtrips(dtype, C):
    N, H, W = 2, 9, 13
    rng = np.random.default_rng(C)
    if dtype == "i8":
        x = rng.integers(-127, 128, (N, C, H, W)).astype(np.int8)
    else:
        x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    xd = to_device(x, dtype)
    say("convert", dtype, C)
    nhwc = B.convert_layout(xd, "NCHW", "NHWC")
    np.testing.assert_array_equal(from_device(nhwc, dtype), from_device(to_device(to_nhwc(x), dtype), dtype))
    back = B.convert_layout(nhwc, "NHWC", "NCHW")
    np.testing.assert_array_equal(from_device(back, dtype), from_device(xd, dtype))
    for xb in (4, 8):
        p = B.convert_layout(nhwc, "NHWC", "NCHWX", xb)
        np.testing.assert_array_equal(from_device(p, dtype), from_device(to_device(pack_nchwx(x, xb), dtype), dtype))
        q = B.convert_layout(p, "NCHWX", "NCHW", channels=C)
        np.testing.assert_array_equal(from_device(q, dtype), from_device(xd, dtype))
        assert unpack_nchwx(from_device(p, dtype), C).shape == x.shape
