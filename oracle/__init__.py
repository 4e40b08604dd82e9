"""CPU oracle for forward 2-D convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never imports, links
or calls it, and it shares no code with the GPU path: the arithmetic lives in
``oracle.c`` (plain C, fp64 / int64 loop nest, OpenMP over output planes),
compiled on its own with gcc.  This module only marshals numpy arrays.

What is computed and why is documented in ``oracle.c``: the plain
cross-correlation of the naive loop nest in the blog post "卷积总结"
(section "最原始的卷积实现"), generalised with batch, stride, zero padding,
dilation and groups, plus the int8 requantisation reading
``clamp(rne(fp32(acc) * scale[k]), -127, 127)``.

Layouts: the oracle works on logical NCHW only.  Packing to and from NCHWx is
plain numpy marshalling in ``cnn_convolution_fwd_amd/workloads.py``
(pinned by ``tests/test_layout_np.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c99", "-Wall", "-Wextra", "-Werror"]

def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` (or a copy of it) into a shared library with gcc."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def _pair(v):
    if isinstance(v, (tuple, list)):
        assert len(v) == 2
        return int(v[0]), int(v[1])
    return int(v), int(v)


class Oracle:
    """numpy front end over one build of ``oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int)
        vp = ctypes.c_void_p
        lib.oracle_output_size.argtypes = [ctypes.c_int] * 5
        lib.oracle_output_size.restype = ctypes.c_int
        lib.oracle_check.argtypes = [i32p]
        lib.oracle_check.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_conv2d_f64.argtypes = [vp, vp, i32p, vp, vp]
        lib.oracle_conv2d_f64.restype = ctypes.c_int
        lib.oracle_conv2d_i8.argtypes = [vp, vp, i32p, vp]
        lib.oracle_conv2d_i8.restype = ctypes.c_int
        lib.oracle_requant_one.argtypes = [ctypes.c_int64, ctypes.c_float]
        lib.oracle_requant_one.restype = ctypes.c_int8
        lib.oracle_requant_i8.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_long, vp]
        lib.oracle_requant_i8.restype = ctypes.c_int
        lib.oracle_conv2d_f64_points.argtypes = [vp, vp, i32p, ctypes.c_long, vp, vp, vp]
        lib.oracle_conv2d_f64_points.restype = ctypes.c_int
        lib.oracle_conv2d_i8_points.argtypes = [vp, vp, i32p, ctypes.c_long, vp, vp]
        lib.oracle_conv2d_i8_points.restype = ctypes.c_int
        lib.oracle_epilogue_f64.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long]
        lib.oracle_epilogue_f64.restype = ctypes.c_int
        lib.oracle_requant_epi_one.argtypes = [ctypes.c_int64, ctypes.c_float, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int8, ctypes.c_int]
        lib.oracle_requant_epi_one.restype = ctypes.c_int8
        lib.oracle_requant_epi_i8.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long,
                                              vp]
        lib.oracle_requant_epi_i8.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def _params(self, x_shape, w_shape, stride, padding, dilation, groups):
        N, C, H, W = (int(d) for d in x_shape)
        K, Cg, R, S = (int(d) for d in w_shape)
        sh, sw = _pair(stride)
        ph, pw = _pair(padding)
        dh, dw = _pair(dilation)
        G = int(groups)
        if G <= 0 or C % G or Cg * G != C:
            raise ValueError("weight shape %s does not match C=%d, groups=%d" % (w_shape, C, G))
        p = (ctypes.c_int * 14)(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, G)
        if self.lib.oracle_check(p) != 0:
            raise ValueError("invalid convolution problem %s" % (list(p),))
        OH = self.output_size(H, R, sh, ph, dh)
        OW = self.output_size(W, S, sw, pw, dw)
        return p, (N, K, OH, OW)

    def output_size(self, n_in: int, k: int, stride: int = 1, pad: int = 0, dil: int = 1) -> int:
        """floor((in + 2 pad - dil (k - 1) - 1) / stride) + 1, or 0 if it does not fit."""
        return int(self.lib.oracle_output_size(int(n_in), int(k), int(stride), int(pad), int(dil)))

    def max_threads(self) -> int:
        """OpenMP threads the oracle will use (OMP_NUM_THREADS, else all cores)."""
        return int(self.lib.oracle_max_threads())

    def conv2d(self, x, w, stride=1, padding=0, dilation=1, groups=1):
        """fp64 convolution of NCHW ``x`` with KCRS ``w``.

        Inputs of any real float dtype are widened exactly to float64.
        Returns ``(y, den)``, both float64 [N, K, OH, OW], where ``den`` is the
        sum of |x * w| over each output's terms.
        """
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        p, oshape = self._params(x.shape, w.shape, stride, padding, dilation, groups)
        y = np.empty(oshape, dtype=np.float64)
        den = np.empty(oshape, dtype=np.float64)
        if self.lib.oracle_conv2d_f64(x.ctypes.data, w.ctypes.data, p, y.ctypes.data, den.ctypes.data):
            raise RuntimeError("oracle_conv2d_f64 failed")
        return y, den

    def conv2d_int8(self, x, w, stride=1, padding=0, dilation=1, groups=1):
        """Exact int64 accumulators of the int8 convolution (NCHW ``x``, KCRS ``w``)."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        if x.dtype != np.int8 or w.dtype != np.int8:
            raise TypeError("conv2d_int8 takes int8 arrays")
        p, oshape = self._params(x.shape, w.shape, stride, padding, dilation, groups)
        acc = np.empty(oshape, dtype=np.int64)
        if self.lib.oracle_conv2d_i8(x.ctypes.data, w.ctypes.data, p, acc.ctypes.data):
            raise RuntimeError("oracle_conv2d_i8 failed")
        return acc

    def requant(self, acc, scale):
        """int8 outputs clamp(rne(fp32(acc) * scale[k]), -127, 127) of [N, K, ...] accumulators."""
        acc = np.ascontiguousarray(acc, dtype=np.int64)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        N, K = acc.shape[0], acc.shape[1]
        if scale.shape != (K,):
            raise ValueError("scale must have shape [K]")
        hw = int(np.prod(acc.shape[2:], dtype=np.int64)) if acc.ndim > 2 else 1
        y = np.empty(acc.shape, dtype=np.int8)
        if self.lib.oracle_requant_i8(acc.ctypes.data, scale.ctypes.data, N, K, hw, y.ctypes.data):
            raise OverflowError("an accumulator does not fit in int32")
        return y

    def requant_one(self, acc: int, scale: float) -> int:
        """The requantisation rule for a single accumulator value (int32 range)."""
        if not (-2**31 <= int(acc) < 2**31):
            raise OverflowError("accumulator outside int32")
        return int(self.lib.oracle_requant_one(int(acc), float(np.float32(scale))))

    def conv2d_int8_requant(self, x, w, scale, stride=1, padding=0, dilation=1, groups=1):
        """int8 convolution followed by the requantisation rule; returns (y_int8, acc_int64)."""
        acc = self.conv2d_int8(x, w, stride, padding, dilation, groups)
        return self.requant(acc, scale), acc

    # ---- fused epilogue (reading in oracle.c): bias, then residual, then ReLU

    def epilogue(self, y, den, bias=None, residual=None, relu=False):
        """(y', den') = the fused epilogue applied to fp64 conv outputs [N, K, ...].

        y' = act(y + bias[k] + residual); den' = den + |bias[k]| + |residual|.
        """
        y = np.array(y, dtype=np.float64, order="C")
        den = np.array(den, dtype=np.float64, order="C")
        N, K = y.shape[0], y.shape[1]
        hw = int(np.prod(y.shape[2:], dtype=np.int64)) if y.ndim > 2 else 1
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
        r = None if residual is None else np.ascontiguousarray(residual, dtype=np.float64)
        if b is not None and b.shape != (K,):
            raise ValueError("bias must have shape [K]")
        if r is not None and r.shape != y.shape:
            raise ValueError("residual must have the output's shape")
        self.lib.oracle_epilogue_f64(y.ctypes.data, den.ctypes.data, None if b is None else b.ctypes.data,
                                     None if r is None else r.ctypes.data, int(bool(relu)), N, K, hw)
        return y, den

    def conv2d_fused(self, x, w, bias=None, residual=None, relu=False, stride=1, padding=0, dilation=1, groups=1):
        """fp64 (y, den') of conv followed by the fused epilogue."""
        y, den = self.conv2d(x, w, stride, padding, dilation, groups)
        return self.epilogue(y, den, bias, residual, relu)

    # ---- bottleneck block (Momenta talk, sections "優化1：Bottleneck" and
    # "Operator的粒度"): three convolutions chained, each with its epilogue

    def bottleneck(self, x, w1, w2, w3, b1=None, b2=None, b3=None, residual=None, relu=(False, False, False)):
        """fp64 (y, den) of a bottleneck block on NCHW ``x``.

        t1 = act1(conv(x, w1) + b1)            1x1, C -> M
        t2 = act2(conv(t1, w2, pad 1) + b2)    3x3, zero padding 1, M -> M
        y  = act3(conv(t2, w3) + b3 + residual) 1x1, M -> K
        all stride 1, act = ReLU where ``relu`` says so, nothing rounded in
        between.  ``den`` is the chain's error normaliser: each stage's
        normaliser passed through the next convolution with |w|, plus |bias|
        (and |residual| at the end).  A relative rounding of size eps at any
        stage (a stored intermediate, an accumulation) moves y by at most
        about eps * den, since |t_i| <= den_i and ReLU does not enlarge
        differences.
        """
        r1, r2, r3 = relu
        t1, d1 = self.conv2d_fused(x, w1, b1, None, r1)
        y2, _ = self.conv2d(t1, w2, 1, 1)
        d2, _ = self.conv2d(d1, np.abs(np.asarray(w2, dtype=np.float64)), 1, 1)
        t2, d2 = self.epilogue(y2, d2, b2, None, r2)
        y3, _ = self.conv2d(t2, w3)
        d3, _ = self.conv2d(d2, np.abs(np.asarray(w3, dtype=np.float64)))
        return self.epilogue(y3, d3, b3, residual, r3)

    def requant_epi(self, acc, scale, bias=None, residual=None, relu=False):
        """int8 outputs of the fused int8 epilogue over [N, K, ...] accumulators."""
        acc = np.ascontiguousarray(acc, dtype=np.int64)
        scale = np.ascontiguousarray(scale, dtype=np.float32)
        N, K = acc.shape[0], acc.shape[1]
        hw = int(np.prod(acc.shape[2:], dtype=np.int64)) if acc.ndim > 2 else 1
        if scale.shape != (K,):
            raise ValueError("scale must have shape [K]")
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.int32)
        r = None if residual is None else np.ascontiguousarray(residual, dtype=np.int8)
        if b is not None and b.shape != (K,):
            raise ValueError("bias must have shape [K]")
        if r is not None and r.shape != acc.shape:
            raise ValueError("residual must have the output's shape")
        y = np.empty(acc.shape, dtype=np.int8)
        if self.lib.oracle_requant_epi_i8(acc.ctypes.data, scale.ctypes.data, None if b is None else b.ctypes.data,
                                          None if r is None else r.ctypes.data, int(bool(relu)), N, K, hw,
                                          y.ctypes.data):
            raise OverflowError("an accumulator plus its bias does not fit in int32")
        return y

    def requant_epi_one(self, acc: int, scale: float, bias: int = 0, residual=None, relu: bool = False) -> int:
        """The fused int8 epilogue for a single accumulator value."""
        if not (-2**31 <= int(acc) + int(bias) < 2**31):
            raise OverflowError("accumulator plus bias outside int32")
        return int(self.lib.oracle_requant_epi_one(int(acc), float(np.float32(scale)), int(bias),
                                                   int(residual is not None),
                                                   int(residual) if residual is not None else 0, int(bool(relu))))

    def conv2d_int8_requant_fused(self, x, w, scale, bias=None, residual=None, relu=False, stride=1, padding=0,
                                  dilation=1, groups=1):
        """int8 conv followed by the fused int8 epilogue; returns (y_int8, acc_int64)."""
        acc = self.conv2d_int8(x, w, stride, padding, dilation, groups)
        return self.requant_epi(acc, scale, bias, residual, relu), acc

    @staticmethod
    def _points_idx(idx):
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        if idx.ndim != 2 or idx.shape[1] != 4:
            raise ValueError("idx must be [npts, 4] of (n, k, oh, ow)")
        return idx

    def conv2d_points(self, x, w, idx, stride=1, padding=0, dilation=1, groups=1):
        """fp64 values (y, den) of selected outputs idx[:, (n, k, oh, ow)]."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        idx = self._points_idx(idx)
        p, _ = self._params(x.shape, w.shape, stride, padding, dilation, groups)
        y = np.empty(len(idx), dtype=np.float64)
        den = np.empty(len(idx), dtype=np.float64)
        if self.lib.oracle_conv2d_f64_points(x.ctypes.data, w.ctypes.data, p, len(idx),
                                             idx.ctypes.data, y.ctypes.data, den.ctypes.data):
            raise ValueError("oracle_conv2d_f64_points: index out of range")
        return y, den

    def conv2d_int8_points(self, x, w, idx, stride=1, padding=0, dilation=1, groups=1):
        """Exact int64 accumulators of selected outputs idx[:, (n, k, oh, ow)]."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        if x.dtype != np.int8 or w.dtype != np.int8:
            raise TypeError("conv2d_int8_points takes int8 arrays")
        idx = self._points_idx(idx)
        p, _ = self._params(x.shape, w.shape, stride, padding, dilation, groups)
        acc = np.empty(len(idx), dtype=np.int64)
        if self.lib.oracle_conv2d_i8_points(x.ctypes.data, w.ctypes.data, p, len(idx),
                                            idx.ctypes.data, acc.ctypes.data):
            raise ValueError("oracle_conv2d_i8_points: index out of range")
        return acc


_default = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` in this directory (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def output_size(*a, **k):
    return default().output_size(*a, **k)


def max_threads():
    return default().max_threads()


def conv2d(*a, **k):
    return default().conv2d(*a, **k)


def conv2d_int8(*a, **k):
    return default().conv2d_int8(*a, **k)


def requant(*a, **k):
    return default().requant(*a, **k)


def requant_one(*a, **k):
    return default().requant_one(*a, **k)


def conv2d_int8_requant(*a, **k):
    return default().conv2d_int8_requant(*a, **k)


def conv2d_points(*a, **k):
    return default().conv2d_points(*a, **k)


def conv2d_int8_points(*a, **k):
    return default().conv2d_int8_points(*a, **k)


def epilogue(*a, **k):
    return default().epilogue(*a, **k)


def conv2d_fused(*a, **k):
    return default().conv2d_fused(*a, **k)


def bottleneck(*a, **k):
    return default().bottleneck(*a, **k)


def requant_epi(*a, **k):
    return default().requant_epi(*a, **k)


def requant_epi_one(*a, **k):
    return default().requant_epi_one(*a, **k)


def conv2d_int8_requant_fused(*a, **k):
    return default().conv2d_int8_requant_fused(*a, **k)


def normalised_error(y_hat, y, den):
    """Pass/fail metric of the float parity tests: max_i |y_hat_i - y_i| / den_i.

    ``den_i`` is the sum of |x * w| over output i's terms (as returned by
    ``conv2d``).  Each output's deviation is divided by its own ``den_i``.
    Outputs with ``den_i == 0`` have only zero terms, so the exact result is 0:
    they are left out of the maximum and must be exactly zero, else the error
    is +inf.  Any NaN or infinity in ``y_hat`` also gives +inf.  With every
    ``den_i == 0`` (and ``y_hat`` all zero) the error is 0.
    """
    y_hat = np.asarray(y_hat, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    if y_hat.shape != y.shape or y.shape != den.shape:
        raise ValueError("shapes differ: %s, %s, %s" % (y_hat.shape, y.shape, den.shape))
    if not np.all(np.isfinite(y_hat)):
        return float("inf")
    zero = den == 0
    if np.any(y_hat[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    nz = ~zero
    return float(np.max(np.abs(y_hat[nz] - y[nz]) / den[nz]))
