"""FLOP / byte conventions against the closed forms the pages print (CPU only).

Momenta talk, section "優化1：Bottleneck": a 3x3 256->256 conv at 56x56 is
about 3.7 GFLOP and 8.8 MB; the 1x1 -> 3x3 -> 1x1 bottleneck is about 0.43
GFLOP and 9.9 MB (fp32, N=1).  Section "基本背景": a 1000^3 GEMM is 2 GFLOP
and 12 MB; a 1000x1000 matrix-vector product is 2 MFLOP and about 4 MB.
Blog "卷积总结": the naive conv of its example layer runs ~85.16 M inner
iterations, ~170 MFLOP.  MegEngine inference article, section "Winograd":
F(2x2,3x3) and F(6x6,3x3) cut multiplies 2.25x and 5.06x.
"""
from cnn_convolution_fwd_amd.roofline import bound, conv_bytes, conv_flops, gemm_flops_bytes, winograd_flops
from cnn_convolution_fwd_amd.workloads import CONFIGS, resnet18_layers


def test_plain_3x3_layer():
    f = conv_flops(1, 256, 56, 56, 256, 3, 3, 1, 1)
    b = conv_bytes(1, 256, 56, 56, 256, 3, 3, 1, 1, esize=4)
    assert f == 3_699_376_128 and round(f / 1e9, 1) == 3.7
    assert b == 8_781_824 and round(b / 1e6, 1) == 8.8


def test_bottleneck_block():
    layers = [(256, 64, 1, 0), (64, 64, 3, 1), (64, 256, 1, 0)]
    f = sum(conv_flops(1, c, 56, 56, k, r, r, 1, p) for c, k, r, p in layers)
    b = sum(conv_bytes(1, c, 56, 56, k, r, r, 1, p, esize=4) for c, k, r, p in layers)
    assert f == 436_731_904 and round(f / 1e9, 2) == 0.44  # "about 0.43G"
    assert b == 9_912_320 and round(b / 1e6, 1) == 9.9
    # ~10x fewer FLOPs, slightly more bytes: intensity collapses
    assert 8 < conv_flops(1, 256, 56, 56, 256, 3, 3, 1, 1) / f < 9


def test_gemm_and_gemv():
    f, b = gemm_flops_bytes(1000, 1000, 1000)
    assert (f, b) == (2_000_000_000, 12_000_000)
    assert round(f / b) == 167  # the talk rounds this to "about 200"
    f, b = gemm_flops_bytes(1000, 1, 1000)
    assert f == 2_000_000 and abs(b - 4e6) / 4e6 < 0.01 and round(f / b, 1) == 0.5


def test_blog_first_layer_count():
    # a 3 -> 64 valid 3x3 conv at 224x224 has exactly the quoted iteration count
    f = conv_flops(1, 3, 224, 224, 64, 3, 3)
    assert f // 2 == 85_162_752 and round(f / 1e6) == 170


def test_headline_layer_roofline():
    L = CONFIGS[3].layers[0]
    f = conv_flops(32, L.c, L.h, L.w, L.k, L.r, L.s, L.stride, L.pad)
    b = conv_bytes(32, L.c, L.h, L.w, L.k, L.r, L.s, L.stride, L.pad, esize=2)
    assert round(f / 1e9, 2) == 118.38
    assert round(b / 1e6, 1) == 103.9
    assert bound(f, b, "bf16")[0] == "mfma"
    dw = CONFIGS[2].layers[1]
    f = conv_flops(64, dw.c, dw.h, dw.w, dw.k, 3, 3, 1, 1, 1, dw.groups)
    b = conv_bytes(64, dw.c, dw.h, dw.w, dw.k, 3, 3, 1, 1, 1, dw.groups, esize=4)
    assert round(b / 1e6, 1) == 205.5 and bound(f, b, "f32")[0] == "hbm"


def test_resnet18_int8_totals():
    macs = sum(conv_flops(1, L.c, L.h, L.w, L.k, L.r, L.s, L.stride, L.pad) for L in resnet18_layers()) // 2
    assert round(macs / 1e9, 4) == 1.8136
    assert len(resnet18_layers()) == 20


def test_winograd_product_counts():
    # F(2x2,3x3): 16 products per 2x2 tile instead of 36 -> 2.25x on a 56x56 map
    d = conv_flops(1, 1, 56, 56, 1, 3, 3, 1, 1)
    assert winograd_flops(1, 1, 56, 56, 1, 2) == 2 * 16 * 28 * 28
    assert d / winograd_flops(1, 1, 56, 56, 1, 2) == 2.25
    # F(6x6,3x3): 64 instead of 324 per tile (5.0625x), but 56 is not a
    # multiple of 6: ceil(56/6)^2 = 100 tiles cover 60x60 outputs -> 4.41x
    assert winograd_flops(1, 1, 56, 56, 1, 6) == 2 * 64 * 100
    assert abs(d / winograd_flops(1, 1, 56, 56, 1, 6) - 4.41) < 0.01
    assert conv_flops(1, 1, 60, 60, 1, 3, 3, 1, 1) / winograd_flops(1, 1, 60, 60, 1, 6) == 324 / 64
    # the headline layer: 52.6 GFLOP (F(2x2)) and 26.8 GFLOP (F(6x6)) at N=32, C=K=256
    assert round(winograd_flops(32, 256, 56, 56, 256, 2) / 1e9, 1) == 52.6
    assert round(winograd_flops(32, 256, 56, 56, 256, 6) / 1e9, 1) == 26.8
