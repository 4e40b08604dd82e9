"""Seeded synthetic workloads for the convolution benchmarks and tests.

This module holds no convolution arithmetic: it defines the layer shapes of
the five benchmark configurations, draws their seeded inputs on the host with
numpy, and packs / unpacks the NCHWx activation layout.  Both the GPU tests
and the CPU oracle are fed from here, so the two sides always see identical
bits.

Sources of the shapes (the pages' workloads; no dataset or trained weight is
used -- every value is a seeded draw):
  * ResNet 3x3 256-channel layer at 56x56 and the 1x1 -> 3x3 -> 1x1
    bottleneck: talk "Paper Reading | 讓深度學習更高效運行的兩個視角", section
    "優化1：Bottleneck".
  * MobileNet-style stem, depthwise 3x3 and pointwise 1x1: same talk, section
    "優化2：Depthwise卷積".
  * int8 ResNet-18 conv stack: the MegEngine Beta article ("推理：高效原生 int8
    实现" and the ARM inference section) quotes int8 ResNet results; the
    twenty conv shapes are the public ResNet-18 architecture at 224x224.

Seeds: numpy ``default_rng(1000 * config + tensor_id + 10 * layer)`` with
tensor ids x=1, w=2, scale=3.  bf16 values are the round-to-nearest-even
bf16 of the fp32 draw; consumers get the rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------- layer shapes


@dataclass(frozen=True)
class Layer:
    name: str
    c: int
    k: int
    h: int
    w: int
    r: int
    s: int
    stride: int = 1
    pad: int = 0
    dil: int = 1
    groups: int = 1

    def out_hw(self) -> Tuple[int, int]:
        oh = (self.h + 2 * self.pad - self.dil * (self.r - 1) - 1) // self.stride + 1
        ow = (self.w + 2 * self.pad - self.dil * (self.s - 1) - 1) // self.stride + 1
        return oh, ow


def resnet18_layers() -> List[Layer]:
    """The twenty conv layers of ResNet-18 at a 224x224 input, in network order."""
    L = []
    L.append(Layer("conv1_7x7s2", 3, 64, 224, 224, 7, 7, 2, 3))
    for i in range(4):
        L.append(Layer("layer1_%d_3x3" % i, 64, 64, 56, 56, 3, 3, 1, 1))
    L.append(Layer("layer2_0_3x3s2", 64, 128, 56, 56, 3, 3, 2, 1))
    L.append(Layer("layer2_0_3x3", 128, 128, 28, 28, 3, 3, 1, 1))
    L.append(Layer("layer2_0_down1x1s2", 64, 128, 56, 56, 1, 1, 2, 0))
    L.append(Layer("layer2_1_3x3a", 128, 128, 28, 28, 3, 3, 1, 1))
    L.append(Layer("layer2_1_3x3b", 128, 128, 28, 28, 3, 3, 1, 1))
    L.append(Layer("layer3_0_3x3s2", 128, 256, 28, 28, 3, 3, 2, 1))
    L.append(Layer("layer3_0_3x3", 256, 256, 14, 14, 3, 3, 1, 1))
    L.append(Layer("layer3_0_down1x1s2", 128, 256, 28, 28, 1, 1, 2, 0))
    L.append(Layer("layer3_1_3x3a", 256, 256, 14, 14, 3, 3, 1, 1))
    L.append(Layer("layer3_1_3x3b", 256, 256, 14, 14, 3, 3, 1, 1))
    L.append(Layer("layer4_0_3x3s2", 256, 512, 14, 14, 3, 3, 2, 1))
    L.append(Layer("layer4_0_3x3", 512, 512, 7, 7, 3, 3, 1, 1))
    L.append(Layer("layer4_0_down1x1s2", 256, 512, 14, 14, 1, 1, 2, 0))
    L.append(Layer("layer4_1_3x3a", 512, 512, 7, 7, 3, 3, 1, 1))
    L.append(Layer("layer4_1_3x3b", 512, 512, 7, 7, 3, 3, 1, 1))
    return L


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    n: int
    layers: Tuple[Layer, ...]
    dtypes: Tuple[str, ...]
    layout: str = "NCHW"
    x_block: Optional[int] = None
    batch_sweep: Tuple[int, ...] = field(default_factory=tuple)


CONFIGS = {
    1: Config(1, "single_conv_16to32_32x32", 1,
              (Layer("conv3x3", 16, 32, 32, 32, 3, 3, 1, 1),), ("f32",)),
    2: Config(2, "mobilenet_stem_dw_pw", 64,
              (Layer("stem3x3s2", 3, 32, 224, 224, 3, 3, 2, 1),
               Layer("dw3x3", 32, 32, 112, 112, 3, 3, 1, 1, groups=32),
               Layer("pw1x1", 32, 64, 112, 112, 1, 1, 1, 0)),
              ("f32", "bf16"), batch_sweep=(1, 2, 4, 8, 16, 32, 64)),
    3: Config(3, "resnet_3x3_256_56x56", 32,
              (Layer("conv3x3_256", 256, 256, 56, 56, 3, 3, 1, 1),), ("bf16", "f32")),
    4: Config(4, "bottleneck_vs_plain_56x56", 32,
              (Layer("reduce1x1_256to64", 256, 64, 56, 56, 1, 1, 1, 0),
               Layer("conv3x3_64", 64, 64, 56, 56, 3, 3, 1, 1),
               Layer("expand1x1_64to256", 64, 256, 56, 56, 1, 1, 1, 0),
               Layer("plain3x3_256", 256, 256, 56, 56, 3, 3, 1, 1)), ("bf16",)),
    5: Config(5, "resnet18_int8_nchw4", 64, tuple(resnet18_layers()), ("i8",),
              layout="NCHWX", x_block=4),
}

# ------------------------------------------------------------------ bf16 bits


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """The fp32 value of each bf16 bit pattern (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 array holding the bf16-rounded values of ``x``."""
    return bf16_to_f32(bf16_bits(x))

# ------------------------------------------------------------- NCHWx layout


def pack_nchwx(x: np.ndarray, xb: int) -> np.ndarray:
    """[N, C, H, W] -> [N, ceil(C/xb), H, W, xb]; channels past C are zero.

    Element (n, c, h, w) goes to [n][c // xb][h][w][c % xb].
    """
    N, C, H, W = x.shape
    cb = -(-C // xb)
    out = np.zeros((N, cb * xb, H, W), dtype=x.dtype)
    out[:, :C] = x
    return np.ascontiguousarray(out.reshape(N, cb, xb, H, W).transpose(0, 1, 3, 4, 2))


def unpack_nchwx(xp: np.ndarray, c: int) -> np.ndarray:
    """[N, CB, H, W, xb] -> [N, c, H, W] (drops the padded channels)."""
    N, CB, H, W, xb = xp.shape
    full = xp.transpose(0, 1, 4, 2, 3).reshape(N, CB * xb, H, W)
    return np.ascontiguousarray(full[:, :c])

def to_nhwc(x: np.ndarray) -> np.ndarray:
    """[N, C, H, W] -> [N, H, W, C]: element (n, c, h, w) goes to [n][h][w][c]."""
    return np.ascontiguousarray(x.transpose(0, 2, 3, 1))


def from_nhwc(x: np.ndarray) -> np.ndarray:
    """[N, H, W, C] -> [N, C, H, W]."""
    return np.ascontiguousarray(x.transpose(0, 3, 1, 2))

def pack_int4(v: np.ndarray) -> np.ndarray:
    """Signed 4-bit values (-8 .. 7), flattened, two per byte: value i in byte
    i // 2, low nibble for even i, high nibble for odd i (uint8 array)."""
    v = np.asarray(v).reshape(-1).astype(np.int16)
    if v.size and (v.min() < -8 or v.max() > 7):
        raise ValueError("4-bit values must lie in -8 .. 7")
    u = (v & 0xF).astype(np.uint8)
    if u.size % 2:
        u = np.concatenate([u, np.zeros(1, np.uint8)])
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray, count: int) -> np.ndarray:
    """Inverse of pack_int4: int8 array of the first ``count`` values."""
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    v = np.empty(p.size * 2, np.int16)
    v[0::2], v[1::2] = lo, hi
    v = np.where(v >= 8, v - 16, v)
    return v[:count].astype(np.int8)

# --------------------------------------------------------------- generators


def rng_for(config: int, tensor_id: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(1000 * config + tensor_id + 10 * layer)


@dataclass
class FloatProblem:
    """fp32 or bf16 problem: ``x``/``w`` hold the exact values (bf16 already rounded)."""
    layer: Layer
    n: int
    dtype: str
    x: np.ndarray  # float32 [N, C, H, W]
    w: np.ndarray  # float32 [K, C/G, R, S]


@dataclass
class Int8Problem:
    layer: Layer
    n: int
    x: np.ndarray      # int8 [N, C, H, W]
    w: np.ndarray      # int8 [K, C/G, R, S]
    scale: np.ndarray  # float32 [K]


def _finish_float(x: np.ndarray, w: np.ndarray, dtype: str):
    x = x.astype(np.float32)
    w = w.astype(np.float32)
    if dtype == "bf16":
        x, w = round_to_bf16(x), round_to_bf16(w)
    elif dtype != "f32":
        raise ValueError(dtype)
    return x, w


def float_problem(config: int, layer_idx: int = 0, n: Optional[int] = None,
                  dtype: Optional[str] = None) -> FloatProblem:
    """Inputs of float configs 1-4 (per layer; each layer is drawn standalone)."""
    cfg = CONFIGS[config]
    L = cfg.layers[layer_idx]
    n = cfg.n if n is None else n
    dtype = cfg.dtypes[0] if dtype is None else dtype
    fan_in = (L.c // L.groups) * L.r * L.s
    rx = rng_for(config, 1, layer_idx)
    rw = rng_for(config, 2, layer_idx)
    xs = (n, L.c, L.h, L.w)
    ws = (L.k, L.c // L.groups, L.r, L.s)
    if config in (1, 2):
        x = rx.uniform(-1.0, 1.0, size=xs)
        w = rw.uniform(-1.0, 1.0, size=ws) / np.sqrt(fan_in)
    elif config in (3, 4):
        x = rx.standard_normal(size=xs, dtype=np.float32)
        w = rw.standard_normal(size=ws, dtype=np.float32) * np.float32(np.sqrt(2.0 / fan_in))
    else:
        raise ValueError("config %d is not a float config" % config)
    x, w = _finish_float(x, w, dtype)
    return FloatProblem(L, n, dtype, x, w)


@dataclass
class BlockProblem:
    """Inputs of a bottleneck block: x [N, C, H, W], w1 [M, C, 1, 1], w2 [M, M, 3, 3], w3 [K, M, 1, 1]."""
    n: int
    x: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    w3: np.ndarray


def bottleneck_block_problem(n: Optional[int] = None, dtype: str = "bf16") -> BlockProblem:
    """The 56x56 bottleneck (1x1 256->64, 3x3 64->64, 1x1 64->256) as one block:
    x and each weight drawn exactly as its layer's standalone problem."""
    ps = [float_problem(4, i, n=n, dtype=dtype) for i in range(3)]
    return BlockProblem(ps[0].n, ps[0].x, ps[0].w, ps[1].w, ps[2].w)


def random_block_problem(n: int, c: int, h: int, w: int, mid: int, k: int, seed: int,
                         dtype: str = "bf16") -> BlockProblem:
    """Ad-hoc block shapes: x ~ N(0, 1), each weight ~ N(0, 2 / fan_in) (bf16-exact for bf16)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, c, h, w))
    w1 = rng.standard_normal((mid, c, 1, 1)) * np.sqrt(2.0 / c)
    w2 = rng.standard_normal((mid, mid, 3, 3)) * np.sqrt(2.0 / (mid * 9))
    w3 = rng.standard_normal((k, mid, 1, 1)) * np.sqrt(2.0 / mid)
    x, w1 = _finish_float(x, w1, dtype)
    _, w2 = _finish_float(x, w2, dtype)
    _, w3 = _finish_float(x, w3, dtype)
    return BlockProblem(n, x, w1, w2, w3)


def random_float_problem(layer: Layer, n: int, dtype: str, seed: int) -> FloatProblem:
    """Uniform[-1,1] input, Uniform[-1,1]/sqrt(fan_in) weights for ad-hoc shapes."""
    rng = np.random.default_rng(seed)
    fan_in = (layer.c // layer.groups) * layer.r * layer.s
    x = rng.uniform(-1.0, 1.0, size=(n, layer.c, layer.h, layer.w))
    w = rng.uniform(-1.0, 1.0, size=(layer.k, layer.c // layer.groups, layer.r, layer.s)) / np.sqrt(fan_in)
    x, w = _finish_float(x, w, dtype)
    return FloatProblem(layer, n, dtype, x, w)

# int8: symmetric per-output-channel weights, activations uniform on -127..127
_VAR_U127 = (255.0 ** 2 - 1.0) / 12.0  # variance of the discrete uniform on -127..127


def quantise_weights(wf: np.ndarray) -> np.ndarray:
    """Symmetric per-output-channel int8: w_q = clamp(rne(w / (max|w[k]| / 127)), -127, 127)."""
    K = wf.shape[0]
    amax = np.abs(wf.reshape(K, -1)).max(axis=1)
    amax = np.where(amax > 0, amax, 1.0)
    sw = amax / 127.0
    q = np.rint(wf / sw.reshape((K,) + (1,) * (wf.ndim - 1)))
    return np.clip(q, -127, 127).astype(np.int8)


def int8_problem_for(layer: Layer, n: int, config: int, layer_idx: int) -> Int8Problem:
    rx = rng_for(config, 1, layer_idx)
    rw = rng_for(config, 2, layer_idx)
    rs = rng_for(config, 3, layer_idx)
    fan_in = (layer.c // layer.groups) * layer.r * layer.s
    x = rx.integers(-127, 128, size=(n, layer.c, layer.h, layer.w), dtype=np.int8)
    wf = rw.standard_normal(size=(layer.k, layer.c // layer.groups, layer.r, layer.s)) * np.sqrt(2.0 / fan_in)
    wq = quantise_weights(wf)
    sumsq = (wq.reshape(layer.k, -1).astype(np.float64) ** 2).sum(axis=1)
    sigma = np.sqrt(_VAR_U127 * np.maximum(sumsq, 1.0))
    u = rs.uniform(0.5, 2.0, size=layer.k)
    scale = (u * 127.0 / (4.0 * sigma)).astype(np.float32)
    return Int8Problem(layer, n, x, wq, scale)


def int8_problem(config: int = 5, layer_idx: int = 0, n: Optional[int] = None) -> Int8Problem:
    cfg = CONFIGS[config]
    L = cfg.layers[layer_idx]
    return int8_problem_for(L, cfg.n if n is None else n, config, layer_idx)


def random_int8_problem(layer: Layer, n: int, seed: int) -> Int8Problem:
    rng = np.random.default_rng(seed)
    x = rng.integers(-127, 128, size=(n, layer.c, layer.h, layer.w), dtype=np.int8)
    w = rng.integers(-127, 128, size=(layer.k, layer.c // layer.groups, layer.r, layer.s), dtype=np.int8)
    fan = (layer.c // layer.groups) * layer.r * layer.s
    scale = (rng.uniform(0.5, 2.0, size=layer.k) * 127.0 / (4.0 * np.sqrt(_VAR_U127 * _VAR_U127 * fan))).astype(np.float32)
    return Int8Problem(layer, n, x, w, scale)


# ------------------------------------------------------- fused-epilogue inputs


@dataclass
class EpilogueInputs:
    """bias [K] and residual (logical NCHW, the output's shape) of a fused epilogue."""
    bias: np.ndarray      # float32 (fp32 / bf16 problems) or int32 (int8)
    residual: np.ndarray  # float32 holding bf16-exact values for bf16, int8 for int8


def epilogue_inputs(out_shape, dtype: str, seed: int) -> EpilogueInputs:
    """Seeded bias and residual for an output of ``out_shape`` = (N, K, OH, OW).

    float: bias ~ U[-1, 1] (bf16-rounded for bf16), residual ~ U[-1, 1];
    int8: bias ~ U{-4096..4096} (int32, added to the accumulator), residual ~
    U{-127..127} (in the output's quantised scale).
    """
    rng = np.random.default_rng(seed)
    K = out_shape[1]
    if dtype == "i8":
        bias = rng.integers(-4096, 4097, size=K, dtype=np.int64).astype(np.int32)
        res = rng.integers(-127, 128, size=out_shape, dtype=np.int8)
        return EpilogueInputs(bias, res)
    bias = rng.uniform(-1.0, 1.0, size=K).astype(np.float32)
    res = rng.uniform(-1.0, 1.0, size=out_shape).astype(np.float32)
    if dtype == "bf16":
        bias, res = round_to_bf16(bias), round_to_bf16(res)
    return EpilogueInputs(bias, res)
