"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Floating point: max over outputs of |y_gpu - y| / sum|x*w| must stay within
1e-5 (fp32 implicit GEMM / direct), 1e-3 (fp32 Winograd) or 1e-2 (bf16).
int8: outputs bit-identical to the oracle's int64 accumulation followed by
clamp(rne(fp32(acc) * scale[k]), -127, 127).

Small shapes are compared element by element over every candidate algorithm
the library lists (the full-size benchmark layers are in test_gpu_full.py).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from cnn_convolution_fwd_amd import binding as B
from cnn_convolution_fwd_amd.workloads import (CONFIGS, Layer, float_problem, int8_problem, pack_nchwx,
                                                random_float_problem, random_int8_problem)
from tests.gpu_util import TOL, TOL_WINOGRAD, candidates_for, run_conv, torch_cuda

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = [
    # name, N, C, H, W, K, R, S, stride, pad, dil, groups
    ("3x3_s1_ragged", 2, 20, 13, 17, 24, 3, 3, 1, 1, 1, 1),
    ("3x3_s2", 1, 35, 9, 30, 70, 3, 3, 2, 1, 1, 1),
    ("1x1", 3, 16, 8, 8, 16, 1, 1, 1, 0, 1, 1),
    ("1x1_s2", 2, 40, 14, 14, 72, 1, 1, 2, 0, 1, 1),
    ("1x1_ragged", 3, 20, 6, 10, 40, 1, 1, 1, 0, 1, 1),
    ("1x1_wide_k", 2, 64, 8, 8, 300, 1, 1, 1, 0, 1, 1),
    ("5x5_d2", 1, 12, 15, 14, 20, 5, 5, 1, 4, 2, 1),
    ("grouped", 2, 12, 10, 11, 18, 3, 3, 1, 1, 1, 3),
    ("depthwise", 2, 16, 12, 16, 16, 3, 3, 1, 1, 1, 16),
    ("dw_wave_split", 3, 5, 9, 24, 5, 3, 3, 1, 1, 1, 5),
    ("dw_w20", 2, 3, 7, 20, 3, 3, 3, 1, 1, 1, 3),
    ("stem7x7s2", 2, 3, 20, 22, 8, 7, 7, 2, 3, 1, 1),
    ("tiny", 1, 1, 1, 1, 1, 1, 1, 1, 0, 1, 1),
    ("asym", 1, 9, 7, 33, 130, 3, 1, (2, 1), (0, 1), 1, 1),
    ("multi_tile_k", 1, 70, 6, 6, 200, 3, 3, 1, 1, 1, 1),
    ("wide_row", 1, 8, 3, 300, 16, 3, 3, 1, 1, 1, 1),
    # tiles of several whole 56-wide output rows whose last row band runs
    # past the output, ragged channel chunk and output-channel tile; stride 2
    ("rows56_ragged", 2, 40, 19, 56, 72, 3, 3, 1, 1, 1, 1),
    ("rows28_s2", 1, 24, 40, 56, 40, 3, 3, 2, 1, 1, 1),
    # few input channels with output planes a multiple of the gather form's
    # workgroup (its input rows staged in LDS), padding on every side
    ("stem3x3s2_32", 2, 3, 32, 32, 32, 3, 3, 2, 1, 1, 1),
    ("stem7x7s2_32", 2, 3, 32, 32, 64, 7, 7, 2, 3, 1, 1),
    ("c4_k40_s1", 1, 4, 16, 24, 40, 3, 3, 1, 1, 1, 1),
    # int8 NCHW4 stem kernel: two 64-channel groups (the second half full),
    # five filter rows (three K steps), a ragged 16-pixel fragment; and the
    # narrowest rows it takes (W = 4: every load window clamped at both ends)
    ("stem_k96_5x5", 1, 3, 9, 21, 96, 5, 5, 1, 2, 1, 1),
    ("stem_w4", 2, 4, 6, 4, 16, 3, 3, 1, 1, 1, 1),
    # operand windows wholly past a row's end or start (taps 4..7 at the
    # last columns of a stride-1 7x7; an 8x8 filter with padding 7)
    ("stem7x7s1_p3", 1, 3, 12, 13, 16, 7, 7, 1, 3, 1, 1),
    ("stem8x8_p7", 1, 4, 10, 9, 8, 8, 8, 1, 7, 1, 1),
    # fused Winograd F(2x2) tile blocks: 8 x 8 tiles with pad 0 and an output
    # width that is not a multiple of 8; two 32-tile column blocks with a
    # ragged channel chunk and output-channel block
    ("wino_p0_w16", 2, 48, 16, 16, 64, 3, 3, 1, 0, 1, 1),
    ("wino_w72", 1, 33, 10, 72, 70, 3, 3, 1, 1, 1, 1),
    # deep 7x7 layer: int8 has four 64-channel chunks, so every split of the
    # reduction over workgroups runs (ragged last split with 3 of 4)
    ("deep7x7_c256", 2, 256, 7, 7, 72, 3, 3, 1, 1, 1, 1),
    # 3x3 with no vertical and one column of horizontal padding (Winograd
    # tile blocks with different row and column offsets)
    ("asym_pad_3x3", 2, 24, 12, 16, 40, 3, 3, 1, (0, 1), 1, 1),
    # few input channels, K = 37: a second k block whose last NCHW4 word holds
    # one real channel (staged gather form: padding channels must be zero)
    ("stem_k37_s2", 2, 3, 32, 32, 37, 3, 3, 2, 1, 1, 1),
    ("c4_k37_s1", 1, 4, 16, 16, 37, 3, 3, 1, 1, 1, 1),
    # depthwise with 96 channels and 20 rows: strip, band and channel indices
    # through divisions by 96 and by the band count
    ("dw_c96", 3, 96, 20, 32, 96, 3, 3, 1, 1, 1, 96),
    # int8 split reductions: four chunks with a ragged last one and K = 37
    # (partial tiles of padded channel blocks); three chunks in two splits
    # of two and one; a 1x1 stride-2 layer with four chunks
    ("split_c200_k37", 2, 200, 9, 11, 37, 3, 3, 1, 1, 1, 1),
    ("split_c130_3chunks", 3, 130, 7, 7, 72, 3, 3, 1, 1, 1, 1),
    ("split_1x1_s2_c256", 2, 256, 14, 14, 64, 1, 1, 2, 0, 1, 1),
    # int8 resident patch (every channel chunk's patch in LDS at once):
    # stride 2 with a batch that leaves a partial image tile; three chunks
    # with odd image sizes and K = 40; 1x1 stride 2; dilation 2; a patch too
    # big for LDS whole (the tile shrinks to fewer rows)
    ("res_c128_s2_n3", 3, 128, 14, 14, 72, 3, 3, 2, 1, 1, 1),
    ("res_c192_9x11", 2, 192, 9, 11, 40, 3, 3, 1, 1, 1, 1),
    ("res_1x1_s2_c128", 3, 128, 13, 13, 72, 1, 1, 2, 0, 1, 1),
    ("res_d2_c64", 2, 64, 10, 10, 40, 3, 3, 1, 2, 2, 1),
    ("res_c512_20x20", 1, 512, 20, 20, 64, 3, 3, 1, 1, 1, 1),
]

LAYOUTS = [("NCHW", None), ("NCHWX", 4), ("NCHWX", 8)]


def tol_for(dtype, algo):
    return (TOL_WINOGRAD if algo.startswith("winograd_f6x6") else TOL)[dtype]


def check_float(name, y, ref, den, dtype, algo):
    assert y.shape == ref.shape, (name, y.shape, ref.shape)
    err = oracle.normalised_error(y, ref, den)
    assert err <= tol_for(dtype, algo), "%s: normalised error %.3g > %.1g" % (name, err, tol_for(dtype, algo))
    return err


@pytest.mark.parametrize("layout,xb", LAYOUTS, ids=["nchw", "nchw4", "nchw8"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_all_candidates(case, dtype, layout, xb):
    torch_cuda()
    name, N, C, H, W, K, R, S, st, pd, dl, G = case
    L = Layer(name, C, K, H, W, R, S, 1, 0, 1, G)
    seed = zlib.crc32((name + dtype).encode())
    cands = candidates_for((N, C, H, W, K, R, S), dtype, st, pd, dl, G, layout, xb)
    assert cands, "no candidate for %s" % name
    failures = []
    if dtype == "i8":
        pr = random_int8_problem(L, N, seed)
        yref, _ = oracle.conv2d_int8_requant(pr.x, pr.w, pr.scale, st, pd, dl, G)
        for algo, cfg in cands:
            say("case", name, dtype, layout, xb, algo, cfg)
            y = run_conv(pr.x, pr.w, dtype, st, pd, dl, G, layout, xb, algo, cfg, scale=pr.scale)
            if not np.array_equal(y, yref):
                failures.append("%s/%d: %d of %d int8 outputs differ" % (algo, cfg, int((y != yref).sum()), y.size))
    else:
        pr = random_float_problem(L, N, dtype, seed)
        yref, den = oracle.conv2d(pr.x, pr.w, st, pd, dl, G)
        for algo, cfg in cands:
            say("case", name, dtype, layout, xb, algo, cfg)
            y = run_conv(pr.x, pr.w, dtype, st, pd, dl, G, layout, xb, algo, cfg)
            err = oracle.normalised_error(y, yref, den)
            if not err <= tol_for(dtype, algo):
                failures.append("%s/%d: error %.3g" % (algo, cfg, err))
    assert not failures, "; ".join(failures)


# Fused Winograd F(6x6) (config 1 of winograd_f6x6_3x3): ragged tile rows and
# columns with a ragged output-channel block; tile blocks whose rows run over
# five images; 34 tile columns (two column blocks); padding 0 and 2; 80
# channels (the last 32-channel chunk half used)
WF6 = [
    # name, N, C, H, W, K, pad
    ("wf6_c64_14x24_k40", 2, 64, 14, 24, 40, 1),
    ("wf6_c80_n5_8x8", 5, 80, 8, 8, 64, 1),
    ("wf6_c64_w200", 1, 64, 8, 200, 32, 1),
    ("wf6_c96_p0", 3, 96, 16, 16, 64, 0),
    ("wf6_c64_p2", 2, 64, 10, 16, 48, 2),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", WF6, ids=[c[0] for c in WF6])
def test_winograd_f6_fused_shapes(case, dtype):
    torch_cuda()
    name, N, C, H, W, K, pd = case
    L = Layer(name, C, K, H, W, 3, 3, 1, pd, 1, 1)
    pr = random_float_problem(L, N, dtype, zlib.crc32((name + dtype).encode()))
    yref, den = oracle.conv2d(pr.x, pr.w, 1, pd, 1, 1)
    cands = [c for c in candidates_for((N, C, H, W, K, 3, 3), dtype, 1, pd) if c[0] == "winograd_f6x6_3x3"]
    if dtype == "bf16" and pd > 1:
        # refused: a corner output's normalising sum covers one pixel per channel
        assert not cands, cands
        return
    assert ("winograd_f6x6_3x3", 1) in cands, cands
    for algo, cfg in cands:
        for prepared in (False, True):
            say("case", name, dtype, algo, cfg, "prepared" if prepared else "")
            y = run_conv(pr.x, pr.w, dtype, 1, pd, algo=algo, config_id=cfg, prepared=prepared)
            check_float("%s/%s/%d" % (name, algo, cfg), y, yref, den, dtype, algo)


def test_prepared_filter_path_matches():
    torch_cuda()
    L = Layer("p", 24, 40, 10, 12, 3, 3, 1, 1)
    pr = random_float_problem(L, 2, "bf16", 5)
    a = run_conv(pr.x, pr.w, "bf16", 1, 1, algo="implicit_gemm", config_id=0)
    b = run_conv(pr.x, pr.w, "bf16", 1, 1, algo="implicit_gemm", config_id=0, prepared=True)
    np.testing.assert_array_equal(a, b)


def test_single_conv_16to32_32x32_full():
    """Single 3x3 conv 16->32 at 32x32, fp32, every candidate, full tensor."""
    torch_cuda()
    pr = float_problem(1)
    L = pr.layer
    yref, den = oracle.conv2d(pr.x, pr.w, L.stride, L.pad, L.dil, L.groups)
    for algo, cfg in candidates_for((1, 16, 32, 32, 32, 3, 3), "f32", 1, 1):
        say("single conv", algo, cfg)
        y = run_conv(pr.x, pr.w, "f32", 1, 1, algo=algo, config_id=cfg)
        check_float("single conv %s/%d" % (algo, cfg), y, yref, den, "f32", algo)


def test_resnet3x3_256ch_deterministic():
    torch_cuda()
    pr = float_problem(3, dtype="bf16")
    a = run_conv(pr.x, pr.w, "bf16", 1, 1, algo="implicit_gemm")
    b = run_conv(pr.x, pr.w, "bf16", 1, 1, algo="implicit_gemm")
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("layer_idx", range(20), ids=[L.name for L in CONFIGS[5].layers])
def test_resnet18_int8_layer_n2_default(layer_idx):
    """int8 ResNet-18 layer, NCHW4, N=2, the default (heuristic) algorithm, bit-exact."""
    torch_cuda()
    L = CONFIGS[5].layers[layer_idx]
    small = int8_problem(5, layer_idx, n=2)
    yref, _ = oracle.conv2d_int8_requant(small.x, small.w, small.scale, L.stride, L.pad, L.dil, L.groups)
    say("resnet18 int8 full N=2", L.name)
    y = run_conv(small.x, small.w, "i8", L.stride, L.pad, L.dil, L.groups, "NCHWX", 4, scale=small.scale)
    assert np.array_equal(y, yref), "%s N=2: %d outputs differ" % (L.name, int((y != yref).sum()))


def test_fastrun_select_and_dispatch(tmp_path):
    torch = torch_cuda()
    B.fastrun_clear()
    pr = float_problem(1)
    from tests.gpu_util import to_device, from_device
    xd, wd = to_device(pr.x, "f32"), to_device(pr.w, "f32")
    say("fastrun single conv")
    best, y = B.fastrun_select(xd, wd, 1, 1)
    yref, den = oracle.conv2d(pr.x, pr.w, 1, 1)
    check_float("fastrun output", from_device(y, "f32"), yref, den, "f32", B.algo_name(best))
    desc = B.desc_for(xd, wd, 1, 1)
    hit = B.fastrun_lookup(desc)
    assert hit is not None and hit.key() == best.key()
    assert B.resolve_algo(desc, B.algo()).key() == best.key()
    path = str(tmp_path / "fr.txt")
    B.fastrun_save(path)
    B.fastrun_clear()
    assert B.fastrun_lookup(desc) is None
    B.fastrun_load(path)
    assert B.fastrun_lookup(desc).key() == best.key()
    B.fastrun_clear()
    torch.cuda.synchronize()


def test_fastrun_int8_layer_bit_exact():
    torch = torch_cuda()
    B.fastrun_clear()
    L = CONFIGS[5].layers[6]
    pr = int8_problem(5, 6, n=4)
    from tests.gpu_util import to_device, from_device
    from cnn_convolution_fwd_amd.workloads import pack_nchwx, unpack_nchwx
    xd = to_device(pack_nchwx(pr.x, 4), "i8")
    wd = to_device(pr.w, "i8")
    sd = torch.from_numpy(pr.scale).cuda()
    say("fastrun int8", L.name)
    best, y = B.fastrun_select(xd, wd, L.stride, L.pad, L.dil, L.groups, "NCHWX", channels=L.c, requant_scale=sd)
    yref, _ = oracle.conv2d_int8_requant(pr.x, pr.w, pr.scale, L.stride, L.pad, L.dil, L.groups)
    got = unpack_nchwx(from_device(y, "i8"), L.k)
    assert np.array_equal(got, yref)
    B.fastrun_clear()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fastrun_stale_workspace_nchw4_k37(dtype):
    """Fast-Run on an NCHW4 problem whose K (37) leaves padding channels, with
    a workspace full of -1.0: the gate's error normaliser must not take the
    stale values in the padding channels (a negative normaliser there once
    let every candidate pass).  The choice must pass the oracle, both as
    returned by the selection and when run again through AUTO dispatch."""
    torch = torch_cuda()
    from tests.gpu_util import output_to_host, to_device
    B.fastrun_clear()
    L = Layer("k37", 20, 37, 12, 16, 3, 3, 1, 1)
    pr = random_float_problem(L, 2, dtype, 37)
    xd = to_device(pack_nchwx(pr.x, 4), dtype)
    wd = to_device(pr.w, dtype)
    desc = B.desc_for(xd, wd, 1, 1, layout="NCHWX", channels=L.c)
    nbytes = B.fastrun_workspace_size(desc)
    ws = torch.empty(nbytes // 4 + 1, dtype=torch.float32, device="cuda").fill_(-1.0).view(torch.uint8)
    say("fastrun stale workspace", dtype)
    best, y = B.fastrun_select(xd, wd, 1, 1, layout="NCHWX", channels=L.c, workspace=ws)
    yref, den = oracle.conv2d(pr.x, pr.w, 1, 1)
    check_float("fastrun stale ws %s" % B.algo_name(best), output_to_host(y, dtype, "NCHWX", L.k), yref, den,
                dtype, B.algo_name(best))
    y2 = B.conv2d_fwd(xd, wd, 1, 1, layout="NCHWX", channels=L.c)
    check_float("auto after stale ws", output_to_host(y2, dtype, "NCHWX", L.k), yref, den, dtype,
                B.algo_name(best))
    B.fastrun_clear()


@pytest.mark.parametrize("magnitude", [1e3, 1e-6], ids=["x1e3", "x1e-6"])
def test_bf16_magnitudes_every_candidate(magnitude):
    """bf16 inputs and weights far from unit scale, every candidate (Winograd
    included: its fp16 operands are scaled into range by powers of two),
    against the oracle within the bf16 bound.  Unscaled, 1e3 would overflow
    fp16 in F(6x6)'s transform and 1e-6 would be an fp16 subnormal."""
    torch_cuda()
    L = Layer("mag", 64, 40, 20, 24, 3, 3, 1, 1)
    pr = random_float_problem(L, 2, "bf16", 77)
    from cnn_convolution_fwd_amd.workloads import round_to_bf16
    x = round_to_bf16(pr.x * np.float32(magnitude))
    w = round_to_bf16(pr.w * np.float32(magnitude ** 0.5))
    yref, den = oracle.conv2d(x, w, 1, 1)
    cands = candidates_for((2, 64, 20, 24, 40, 3, 3), "bf16", 1, 1)
    assert any(a.startswith("winograd") for a, _ in cands)
    failures = []
    for algo, cfg in cands:
        say("magnitude", magnitude, algo, cfg)
        y = run_conv(x, w, "bf16", 1, 1, algo=algo, config_id=cfg)
        err = oracle.normalised_error(y, yref, den)
        if not err <= tol_for("bf16", algo):
            failures.append("%s/%d: error %.3g" % (algo, cfg, err))
    assert not failures, "; ".join(failures)
