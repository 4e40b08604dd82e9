"""Algorithmic FLOPs, bytes and roofline bounds of a convolution layer.

Conventions (Momenta talk "Paper Reading | 讓深度學習更高效運行的兩個視角",
sections "基本背景" and "兩個視角：計算量和訪存量" and its Q&A): a multiply-add
counts as 2 FLOPs; the memory traffic of a layer is the size of all its
inputs, its parameters and its outputs, each counted once (caches ignored);
arithmetic intensity = FLOPs / bytes; a kernel is bound by compute when its
intensity exceeds the ridge point peak_flops / bandwidth, else by memory.
Throughput is quoted in direct-equivalent FLOPs for every algorithm (Winograd
layers are credited with the FLOPs of direct convolution); a kernel's roofline
fraction uses the FLOPs its algorithm performs (``layer_algo_flops``).

Peaks are AMD's published MI355X figures (dense, no sparsity).
"""
from __future__ import annotations

PEAK = {
    "hbm_bytes_per_s": 8.0e12,
    "bf16": 2.5e15, "f16": 2.5e15, "fp8": 5.0e15, "i8": 5.0e15, "f32": 157.3e12, "f64": 78.6e12,
}
ESIZE = {"f32": 4, "bf16": 2, "i8": 1, "f64": 8}


def out_hw(h, w, r, s, stride=1, pad=0, dil=1):
    sh, sw = (stride, stride) if isinstance(stride, int) else stride
    ph, pw = (pad, pad) if isinstance(pad, int) else pad
    dh, dw = (dil, dil) if isinstance(dil, int) else dil
    return (h + 2 * ph - dh * (r - 1) - 1) // sh + 1, (w + 2 * pw - dw * (s - 1) - 1) // sw + 1


def conv_flops(n, c, h, w, k, r, s, stride=1, pad=0, dil=1, groups=1) -> int:
    oh, ow = out_hw(h, w, r, s, stride, pad, dil)
    return 2 * n * k * (c // groups) * r * s * oh * ow


def conv_bytes(n, c, h, w, k, r, s, stride=1, pad=0, dil=1, groups=1, esize=4, esize_out=None) -> int:
    oh, ow = out_hw(h, w, r, s, stride, pad, dil)
    eo = esize if esize_out is None else esize_out
    return esize * (n * c * h * w + k * (c // groups) * r * s) + eo * n * k * oh * ow


def layer_flops(L, n) -> int:
    return conv_flops(n, L.c, L.h, L.w, L.k, L.r, L.s, L.stride, L.pad, L.dil, L.groups)


def layer_bytes(L, n, dtype) -> int:
    return conv_bytes(n, L.c, L.h, L.w, L.k, L.r, L.s, L.stride, L.pad, L.dil, L.groups, ESIZE[dtype])


def winograd_flops(n, c, h, w, k, m, pad=1, groups=1) -> int:
    """FLOPs of Winograd F(m x m, 3 x 3)'s element-wise products, the part the
    matrix cores execute: every output tile of m x m (edge tiles included,
    cropped afterwards) takes alpha^2 = (m + 2)^2 products per (input channel,
    output channel) pair, 2 FLOPs each (MegEngine inference article, section
    "Winograd": 16 instead of 36 multiplies for F(2x2,3x3))."""
    oh, ow = out_hw(h, w, 3, 3, 1, pad, 1)
    tiles = n * (-(-oh // m)) * (-(-ow // m))
    return 2 * (m + 2) ** 2 * tiles * k * (c // groups)


def layer_algo_flops(L, n, algo_name: str) -> int:
    """FLOPs the named algorithm performs for the layer: Winograd's
    element-wise products for the Winograd families, the direct count for
    every other family (implicit GEMM, direct, pointwise perform exactly it)."""
    if algo_name.startswith("winograd_f2x2"):
        return winograd_flops(n, L.c, L.h, L.w, L.k, 2, L.pad, L.groups)
    if algo_name.startswith("winograd_f6x6"):
        return winograd_flops(n, L.c, L.h, L.w, L.k, 6, L.pad, L.groups)
    return layer_flops(L, n)


def block_flops(n, c, h, w, mid, k) -> int:
    """Direct FLOPs of a bottleneck block: 1x1 c->mid, 3x3 pad 1 mid->mid, 1x1 mid->k."""
    px = n * h * w
    return 2 * px * (c * mid + mid * mid * 9 + mid * k)


def block_algo_flops(n, c, h, w, mid, k, rows_per_tile=4) -> int:
    """FLOPs the fused block kernel performs: the first 1x1 also runs on the
    two halo rows of every band of ``rows_per_tile`` output rows (Momenta
    talk, section "Operator的粒度": the tiles' overlap is recomputed)."""
    bands = -(-h // rows_per_tile)
    rows1 = bands * (rows_per_tile + 2)
    return 2 * n * w * (rows1 * c * mid + h * (mid * mid * 9 + mid * k))


def block_bytes(n, c, h, w, mid, k, esize) -> int:
    """Algorithmic bytes of the fused block: x read once, y written once, the
    three weight tensors once (no intermediate tensor)."""
    return esize * (n * c * h * w + n * k * h * w + mid * c + mid * mid * 9 + k * mid)


def gemm_flops_bytes(m, n, k, esize=4):
    """C = A(m x k) B(k x n): 2mnk FLOPs; A, B and C each moved once."""
    return 2 * m * n * k, esize * (m * k + k * n + m * n)


def bound(flops, nbytes, dtype):
    """('mfma' or 'hbm', attainable FLOP/s) on the MI355X roofline."""
    ai = flops / nbytes
    compute = PEAK[dtype]
    memory = ai * PEAK["hbm_bytes_per_s"]
    return ("mfma", compute) if compute <= memory else ("hbm", memory)
