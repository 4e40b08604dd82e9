"""GPU parity of int8 Winograd F(2x2,3x3) with a float intermediate (MegEngine
Beta release article, section "业界领先的原生 ARM 推理性能": int8 Winograd that
computes in float, with no narrowing of the weights).

The method's result is the convolution itself, so the oracle is the exact one:
int64 accumulation, then clamp(rne(fp32(acc) * scale[k]), -127, 127) (or the
fused form with bias, residual and ReLU).  The float intermediate is exact
while every fp32 partial sum stays below 2^22 in magnitude (the fp16
operands are exact: tests/test_winograd_rational.py); beyond that an fp32
rounding can move an accumulator across a requantisation boundary.  The bar,
as in the library's Fast-Run gate for this candidate: no output more than 1
away from the exact one, on every element; the number of outputs that differ
at all is printed and must stay a small fraction.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from cnn_convolution_fwd_amd import binding as B
from cnn_convolution_fwd_amd.workloads import (CONFIGS, Layer, epilogue_inputs, int8_problem, pack_nchwx,
                                                random_int8_problem, unpack_nchwx)
from tests.gpu_util import from_device, output_to_host, run_conv, to_device, torch_cuda

pytestmark = pytest.mark.gpu

ALGO = "winograd_f2x2_3x3"
MAX_DIFF_FRACTION = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    ndiff = int((d != 0).sum())
    say("  %s: max |diff| %d, %d of %d outputs differ" % (name, int(d.max()) if d.size else 0, ndiff, d.size))
    assert d.size == 0 or d.max() <= 1, "%s: an output is %d away from the exact one" % (name, int(d.max()))
    assert ndiff <= MAX_DIFF_FRACTION * max(d.size, 1), "%s: %d of %d outputs differ" % (name, ndiff, d.size)


SMALL = [
    # name, N, C, H, W, K, pad
    ("c20_13x17_k24", 2, 20, 13, 17, 24, 1),      # one ragged channel chunk, odd output sizes
    ("c70_9x30_k70", 1, 70, 9, 30, 70, 1),        # three chunks (last ragged), second K block ragged
    ("c64_16x16_k64_p0", 2, 64, 16, 16, 64, 0),  # no padding, tiles exactly cover the output
    ("c33_10x72_k130_p2", 1, 33, 10, 72, 130, 2),  # padding 2, three K blocks
    ("c96_7x7_k40_n5", 5, 96, 7, 7, 40, 1),       # a tile block spanning images
    ("c8_1x1_k8", 1, 8, 1, 1, 8, 1),              # one output pixel: a single tile
    ("c512_8x8_k64", 1, 512, 8, 8, 64, 1),        # deep reduction: 16 chunks
]
LAYOUTS = [("NCHW", None), ("NCHWX", 4), ("NCHWX", 8)]


@pytest.mark.parametrize("prepared", [False, True], ids=["ws", "prepared"])
@pytest.mark.parametrize("layout,xb", LAYOUTS, ids=["nchw", "nchw4", "nchw8"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_int8_winograd_small(case, layout, xb, prepared):
    torch_cuda()
    name, N, C, H, W, K, pd = case
    L = Layer(name, C, K, H, W, 3, 3, 1, pd, 1, 1)
    pr = random_int8_problem(L, N, zlib.crc32((name + "wi8").encode()))
    ref, _ = oracle.conv2d_int8_requant(pr.x, pr.w, pr.scale, 1, pd, 1, 1)
    say("int8 winograd", name, layout, xb, "prepared" if prepared else "workspace")
    y = run_conv(pr.x, pr.w, "i8", 1, pd, 1, 1, layout, xb, ALGO, 0, scale=pr.scale, prepared=prepared)
    check(name, y, ref)


def test_int8_winograd_extreme_magnitudes():
    """Inputs and weights near +-127 with random signs and 1024 channels: the
    channel sums pass 2^22, so the fp32 sums round; still within 1."""
    torch_cuda()
    rng = np.random.default_rng(1024)
    N, C, H, W, K = 1, 1024, 6, 10, 64
    x = (rng.choice([-1, 1], (N, C, H, W)) * rng.integers(120, 128, (N, C, H, W))).astype(np.int8)
    w = (rng.choice([-1, 1], (K, C, 3, 3)) * rng.integers(120, 128, (K, C, 3, 3))).astype(np.int8)
    # spread the outputs over the whole int8 range (a few saturate)
    scale = np.full(K, 127.0 / (3.0 * 124.0 * 124.0 * np.sqrt(C * 9)), dtype=np.float32)
    ref, acc = oracle.conv2d_int8_requant(x, w, scale, 1, 1, 1, 1)
    say("int8 winograd extreme magnitudes: max |acc| %d" % int(np.abs(acc).max()))
    y = run_conv(x, w, "i8", 1, 1, 1, 1, "NCHWX", 4, ALGO, 0, scale=scale)
    check("extreme", y, ref)


VARIANTS = [("bias_res_relu", True, True, True), ("bias_only", True, False, False), ("res_relu", False, True, True)]


@pytest.mark.parametrize("variant", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("layout,xb", LAYOUTS, ids=["nchw", "nchw4", "nchw8"])
def test_int8_winograd_epilogue(layout, xb, variant):
    torch = torch_cuda()
    vname, use_bias, use_res, relu = variant
    N, C, H, W, K = 2, 40, 13, 18, 72
    L = Layer("epi", C, K, H, W, 3, 3, 1, 1, 1, 1)
    seed = zlib.crc32(("wi8epi" + vname).encode())
    pr = random_int8_problem(L, N, seed)
    epi = epilogue_inputs((N, K, H, W), "i8", seed + 1)
    bias = epi.bias if use_bias else None
    res = epi.residual if use_res else None
    ref, _ = oracle.conv2d_int8_requant_fused(pr.x, pr.w, pr.scale, bias, res, relu, 1, 1, 1, 1)
    xin = pack_nchwx(pr.x, xb) if layout == "NCHWX" else pr.x
    xd, wd = to_device(xin, "i8"), to_device(pr.w, "i8")
    bd = torch.from_numpy(bias).cuda() if bias is not None else None
    rd = to_device(pack_nchwx(res, xb) if layout == "NCHWX" else res, "i8") if res is not None else None
    sd = torch.from_numpy(pr.scale).cuda()
    say("int8 winograd epilogue", layout, xb, vname)
    y = B.conv2d_fwd(xd, wd, 1, 1, 1, 1, layout, channels=C, algo_kind=ALGO, config_id=0, requant_scale=sd,
                     bias=bd, residual=rd, relu=relu)
    check("epilogue " + vname, output_to_host(y, "i8", layout, K), ref)


STRIDE1 = [i for i, L in enumerate(CONFIGS[5].layers) if L.r == 3 and L.stride == 1]


@pytest.mark.parametrize("layer_idx", STRIDE1, ids=[CONFIGS[5].layers[i].name for i in STRIDE1])
def test_int8_winograd_resnet18_layer_n2(layer_idx):
    """ResNet-18 int8 3x3 stride-1 layers, NCHW4, N=2, whole tensors."""
    torch_cuda()
    L = CONFIGS[5].layers[layer_idx]
    pr = int8_problem(5, layer_idx, n=2)
    ref, _ = oracle.conv2d_int8_requant(pr.x, pr.w, pr.scale, L.stride, L.pad, L.dil, L.groups)
    say("int8 winograd resnet18", L.name)
    y = run_conv(pr.x, pr.w, "i8", 1, 1, 1, 1, "NCHWX", 4, ALGO, 0, scale=pr.scale)
    check(L.name, y, ref)


def test_int8_winograd_fastrun_opt_in():
    """Only after the opt-in does Fast-Run time int8 Winograd; whatever it
    picks, the output is within 1 of the exact result (exact if not Winograd)."""
    torch = torch_cuda()
    L = CONFIGS[5].layers[1]
    pr = int8_problem(5, 1, n=4)
    xd = to_device(pack_nchwx(pr.x, 4), "i8")
    wd = to_device(pr.w, "i8")
    sd = torch.from_numpy(pr.scale).cuda()
    ref, _ = oracle.conv2d_int8_requant(pr.x, pr.w, pr.scale, L.stride, L.pad, L.dil, L.groups)
    desc = B.desc_for(xd, wd, L.stride, L.pad, L.dil, L.groups, "NCHWX", channels=L.c)
    B.fastrun_clear()
    try:
        assert B.ALGO_WINOGRAD_F2X2_3X3 not in [a.kind for a in B.list_candidates(desc)]
        B.fastrun_allow_inexact_int8(True)
        assert B.ALGO_WINOGRAD_F2X2_3X3 in [a.kind for a in B.list_candidates(desc)]
        say("int8 winograd fastrun opt-in", L.name)
        best, y = B.fastrun_select(xd, wd, L.stride, L.pad, L.dil, L.groups, "NCHWX", channels=L.c,
                                   requant_scale=sd)
        got = unpack_nchwx(from_device(y, "i8"), L.k)
        say("  chose", B.algo_name(best), "%.4f ms" % best.median_ms)
        if best.kind == B.ALGO_WINOGRAD_F2X2_3X3:
            check("fastrun", got, ref)
        else:
            assert np.array_equal(got, ref)
    finally:
        B.fastrun_allow_inexact_int8(False)
        B.fastrun_clear()
    torch.cuda.synchronize()
