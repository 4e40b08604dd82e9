"""ctypes binding of libcfwd.so (include/cfwd.h), same names as the C ABI.

Argument marshalling only: every step of the convolution runs in the HIP
library.  torch is used for device memory and streams (``data_ptr()`` and
``torch.cuda.current_stream().cuda_stream``).  If the library has not been
built, loading fails loudly -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple, Union

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcfwd.so")

# enums (mirror include/cfwd.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_NO_CANDIDATE, ERR_HIP, ERR_CACHE_IO = range(7)
LAYOUT_NCHW, LAYOUT_NCHWX, LAYOUT_NHWC = 0, 1, 2
_LAYOUTS = {"NCHW": LAYOUT_NCHW, "NCHWX": LAYOUT_NCHWX, "NHWC": LAYOUT_NHWC}
F32, BF16, I8 = 0, 1, 2
ALGO_AUTO, ALGO_IMPLICIT_GEMM, ALGO_WINOGRAD_F2X2_3X3, ALGO_WINOGRAD_F6X6_3X3, ALGO_DIRECT, ALGO_POINTWISE = range(6)

ALGO_NAMES = {
    "auto": ALGO_AUTO, "implicit_gemm": ALGO_IMPLICIT_GEMM, "winograd_f2x2_3x3": ALGO_WINOGRAD_F2X2_3X3,
    "winograd_f6x6_3x3": ALGO_WINOGRAD_F6X6_3X3, "direct": ALGO_DIRECT, "pointwise": ALGO_POINTWISE,
}

EXPORTED = [
    "cfwd_version", "cfwd_output_dims", "cfwd_resolve_algo", "cfwd_list_candidates", "cfwd_filter_size",
    "cfwd_prepare_filter", "cfwd_workspace_size", "cfwd_scratch_size", "cfwd_conv2d_fwd", "cfwd_fastrun_select",
    "cfwd_fastrun_workspace_size", "cfwd_fastrun_lookup", "cfwd_fastrun_load", "cfwd_fastrun_save",
    "cfwd_fastrun_clear", "cfwd_fastrun_choose", "cfwd_status_string", "cfwd_last_error", "cfwd_algo_name",
    "cfwd_conv2d_fwd_noalloc", "cfwd_conv2d_fwd_ex", "cfwd_fastrun_allow_inexact_int8",
    "cfwd_bottleneck_check", "cfwd_bottleneck_filter_size", "cfwd_bottleneck_prepare", "cfwd_bottleneck_fwd",
    "cfwd_convert_layout", "cfwd_unpack_int4",
]
ACT_NONE, ACT_RELU = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # CFWD_NOALLOC_SCRATCH_BYTES


class ConvDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n", "c", "h", "w", "k", "r", "s", "stride_h", "stride_w", "pad_h",
                                            "pad_w", "dil_h", "dil_w", "groups")] + \
               [("layout", ctypes.c_int), ("x", ctypes.c_int), ("dtype", ctypes.c_int)]


class Epilogue(ctypes.Structure):
    """cfwd_epilogue: bias [K] (fp32, or int32 for int8), residual (y's shape / layout / dtype), activation."""
    _fields_ = [("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p), ("act", ctypes.c_int)]


class BottleneckDesc(ctypes.Structure):
    """cfwd_bottleneck_desc: x [N, C, H, W], inner channels ``mid``, output channels ``k``."""
    _fields_ = [(n, ctypes.c_int) for n in ("n", "c", "h", "w", "mid", "k")] + [("dtype", ctypes.c_int)]


class BottleneckEpilogue(ctypes.Structure):
    """cfwd_bottleneck_epilogue: fp32 biases b1 [mid], b2 [mid], b3 [K], bf16 residual, ReLU after each stage."""
    _fields_ = [("b1", ctypes.c_void_p), ("b2", ctypes.c_void_p), ("b3", ctypes.c_void_p),
                ("residual", ctypes.c_void_p), ("relu1", ctypes.c_int), ("relu2", ctypes.c_int),
                ("relu3", ctypes.c_int)]


class Algo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("config_id", ctypes.c_int), ("median_ms", ctypes.c_float)]

    def __repr__(self):
        return "Algo(%s, ms=%.4g)" % (algo_name(self), self.median_ms)

    def key(self) -> Tuple[int, int]:
        return (self.kind, self.config_id)


class CfwdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_lib().cfwd_status_string(status).decode(), msg))
        self.status = status


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libcfwd.so is not built (run python -m cnn_convolution_fwd_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        dp = P(ConvDesc)
        lib.cfwd_version.restype = ctypes.c_char_p
        lib.cfwd_status_string.restype = ctypes.c_char_p
        lib.cfwd_status_string.argtypes = [ctypes.c_int]
        lib.cfwd_last_error.restype = ctypes.c_char_p
        lib.cfwd_algo_name.restype = ctypes.c_char_p
        lib.cfwd_algo_name.argtypes = [Algo]
        sigs = {
            "cfwd_output_dims": [dp, P(ctypes.c_int), P(ctypes.c_int)],
            "cfwd_resolve_algo": [dp, Algo, P(Algo)],
            "cfwd_list_candidates": [dp, P(Algo), ctypes.c_int, P(ctypes.c_int)],
            "cfwd_filter_size": [dp, Algo, P(sz)],
            "cfwd_prepare_filter": [dp, Algo, vp, vp, sz, vp],
            "cfwd_workspace_size": [dp, Algo, P(sz)],
            "cfwd_scratch_size": [dp, Algo, P(sz)],
            "cfwd_conv2d_fwd": [dp, Algo, vp, vp, vp, vp, vp, vp, sz, vp],
            "cfwd_conv2d_fwd_noalloc": [dp, Algo, vp, vp, vp, vp, vp, vp],
            "cfwd_conv2d_fwd_ex": [dp, Algo, vp, vp, vp, vp, P(Epilogue), vp, vp, sz, vp],
            "cfwd_fastrun_select": [dp, vp, vp, vp, vp, vp, sz, vp, P(Algo)],
            "cfwd_fastrun_workspace_size": [dp, P(sz)],
            "cfwd_fastrun_lookup": [dp, P(Algo)],
            "cfwd_fastrun_load": [ctypes.c_char_p],
            "cfwd_fastrun_save": [ctypes.c_char_p],
            "cfwd_fastrun_clear": [],
            "cfwd_fastrun_allow_inexact_int8": [ctypes.c_int],
            "cfwd_bottleneck_check": [P(BottleneckDesc)],
            "cfwd_unpack_int4": [vp, vp, ctypes.c_longlong, vp],
            "cfwd_convert_layout": [ctypes.c_int] * 4 + [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int,
                                                         ctypes.c_int, vp, vp],
            "cfwd_bottleneck_filter_size": [P(BottleneckDesc), P(sz)],
            "cfwd_bottleneck_prepare": [P(BottleneckDesc), vp, vp, sz, vp],
            "cfwd_bottleneck_fwd": [P(BottleneckDesc), vp, vp, vp, vp, P(BottleneckEpilogue), vp, vp],
            "cfwd_fastrun_choose": [P(Algo), P(ctypes.c_float), ctypes.c_int, ctypes.c_int, P(ctypes.c_int),
                                    P(ctypes.c_int)],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _check(status: int):
    if status != OK:
        raise CfwdError(status, _lib().cfwd_last_error().decode())


# ------------------------------------------------------------ descriptors

def _pair(v) -> Tuple[int, int]:
    if isinstance(v, (tuple, list)):
        return int(v[0]), int(v[1])
    return int(v), int(v)


def make_desc(n, c, h, w, k, r, s, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", x_block=None,
              dtype="f32") -> ConvDesc:
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    lay = _LAYOUTS[layout.upper()]
    dt = {"f32": F32, "fp32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16, "i8": I8, "int8": I8}[dtype]
    return ConvDesc(n, c, h, w, k, r, s, sh, sw, ph, pw, dh, dw, groups, lay, int(x_block or 0), dt)


def algo(kind: Union[str, int] = "auto", config_id: int = -1) -> Algo:
    if isinstance(kind, str):
        kind = ALGO_NAMES[kind]
    return Algo(kind, config_id, 0.0)


def algo_name(a: Algo) -> str:
    return _lib().cfwd_algo_name(a).decode()


def version() -> str:
    return _lib().cfwd_version().decode()


def output_dims(desc: ConvDesc) -> Tuple[int, int]:
    oh, ow = ctypes.c_int(), ctypes.c_int()
    _check(_lib().cfwd_output_dims(ctypes.byref(desc), ctypes.byref(oh), ctypes.byref(ow)))
    return oh.value, ow.value


def resolve_algo(desc: ConvDesc, a: Algo) -> Algo:
    out = Algo()
    _check(_lib().cfwd_resolve_algo(ctypes.byref(desc), a, ctypes.byref(out)))
    return out


def list_candidates(desc: ConvDesc) -> List[Algo]:
    n = ctypes.c_int()
    _check(_lib().cfwd_list_candidates(ctypes.byref(desc), None, 0, ctypes.byref(n)))
    arr = (Algo * max(1, n.value))()
    _check(_lib().cfwd_list_candidates(ctypes.byref(desc), arr, n.value, ctypes.byref(n)))
    return [arr[i] for i in range(n.value)]


def filter_size(desc: ConvDesc, a: Algo) -> int:
    b = ctypes.c_size_t()
    _check(_lib().cfwd_filter_size(ctypes.byref(desc), a, ctypes.byref(b)))
    return b.value


def workspace_size(desc: ConvDesc, a: Algo) -> int:
    b = ctypes.c_size_t()
    _check(_lib().cfwd_workspace_size(ctypes.byref(desc), a, ctypes.byref(b)))
    return b.value


def scratch_size(desc: ConvDesc, a: Algo) -> int:
    b = ctypes.c_size_t()
    _check(_lib().cfwd_scratch_size(ctypes.byref(desc), a, ctypes.byref(b)))
    return b.value


def fastrun_workspace_size(desc: ConvDesc) -> int:
    b = ctypes.c_size_t()
    _check(_lib().cfwd_fastrun_workspace_size(ctypes.byref(desc), ctypes.byref(b)))
    return b.value


def fastrun_lookup(desc: ConvDesc) -> Optional[Algo]:
    out = Algo()
    st = _lib().cfwd_fastrun_lookup(ctypes.byref(desc), ctypes.byref(out))
    return out if st == OK else None


def fastrun_load(path: str):
    _check(_lib().cfwd_fastrun_load(path.encode()))


def fastrun_save(path: str):
    _check(_lib().cfwd_fastrun_save(path.encode()))


def fastrun_clear():
    _check(_lib().cfwd_fastrun_clear())


def fastrun_allow_inexact_int8(allow: bool):
    """Let int8 candidates that may differ by 1 from the exact result (int8 Winograd F(2x2)) join Fast-Run."""
    _check(_lib().cfwd_fastrun_allow_inexact_int8(1 if allow else 0))


def fastrun_choose(cands: Sequence[Algo], times: Sequence[Sequence[float]], gate_ok: Sequence[bool]) -> int:
    n = len(cands)
    reps = len(times[0]) if n else 1
    ca = (Algo * max(1, n))(*cands)
    ta = (ctypes.c_float * max(1, n * reps))(*[float(v) for row in times for v in row])
    ok = (ctypes.c_int * max(1, n))(*[int(bool(v)) for v in gate_ok])
    chosen = ctypes.c_int()
    _check(_lib().cfwd_fastrun_choose(ca, ta, n, reps, ok, ctypes.byref(chosen)))
    return chosen.value


# ---------------------------------------------------------- raw-pointer calls

def conv2d_fwd_raw(desc: ConvDesc, a: Algo, x: int, w: int, w_prepared: int, scale: int, y: int, ws: int,
                   ws_bytes: int, stream: int) -> int:
    """cfwd_conv2d_fwd with integer device pointers; returns the status."""
    return _lib().cfwd_conv2d_fwd(ctypes.byref(desc), a, x or None, w or None, w_prepared or None, scale or None,
                                  y or None, ws or None, ws_bytes, stream or None)


def epilogue_of(bias: int = 0, residual: int = 0, relu: bool = False) -> Optional[Epilogue]:
    """cfwd_epilogue from device pointers, or None when there is nothing to fuse."""
    if not bias and not residual and not relu:
        return None
    return Epilogue(bias or None, residual or None, ACT_RELU if relu else ACT_NONE)


def conv2d_fwd_ex_raw(desc: ConvDesc, a: Algo, x: int, w: int, w_prepared: int, scale: int, ep: Optional[Epilogue],
                      y: int, ws: int, ws_bytes: int, stream: int) -> int:
    """cfwd_conv2d_fwd_ex with integer device pointers; returns the status."""
    return _lib().cfwd_conv2d_fwd_ex(ctypes.byref(desc), a, x or None, w or None, w_prepared or None, scale or None,
                                     ctypes.byref(ep) if ep is not None else None, y or None, ws or None, ws_bytes,
                                     stream or None)


def conv2d_fwd_noalloc_raw(desc: ConvDesc, a: Algo, x: int, w: int, w_prepared: int, scale: int, y: int,
                           stream: int) -> int:
    """cfwd_conv2d_fwd_noalloc with integer device pointers; returns the status."""
    return _lib().cfwd_conv2d_fwd_noalloc(ctypes.byref(desc), a, x or None, w or None, w_prepared or None,
                                          scale or None, y or None, stream or None)


def prepare_filter_raw(desc: ConvDesc, a: Algo, w: int, wp: int, nbytes: int, stream: int) -> int:
    return _lib().cfwd_prepare_filter(ctypes.byref(desc), a, w or None, wp or None, nbytes, stream or None)


# ---------------------------------------------------------- torch front end

def _torch():
    import torch
    return torch


_DT = {"torch.float32": "f32", "torch.bfloat16": "bf16", "torch.int8": "i8"}


def _dtype_of(t) -> str:
    key = str(t.dtype)
    if key not in _DT:
        raise TypeError("unsupported dtype %s (float32, bfloat16 or int8)" % t.dtype)
    return _DT[key]


def desc_for(x, w, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", channels=None) -> ConvDesc:
    """Descriptor for activations ``x`` (NCHW [N,C,H,W], NHWC [N,H,W,C] or NCHWX [N,CB,H,W,X]) and KCRS ``w``."""
    if layout.upper() == "NCHW":
        if x.dim() != 4:
            raise ValueError("NCHW activations must be 4-D")
        n, c, h, wd = x.shape
        xb = 0
    elif layout.upper() == "NHWC":
        if x.dim() != 4:
            raise ValueError("NHWC activations must be 4-D")
        n, h, wd, c = x.shape
        xb = 0
    else:
        if x.dim() != 5:
            raise ValueError("NCHWX activations must be 5-D [N, C/x, H, W, x]")
        n, cb, h, wd, xb = x.shape
        c = channels if channels is not None else cb * xb
        if not (cb - 1) * xb < c <= cb * xb:
            raise ValueError("channels=%d does not match %d blocks of %d" % (c, cb, xb))
    k, cg, r, s = w.shape
    if cg * groups != c:
        raise ValueError("weights [K, C/G, R, S] = %s do not match C=%d, groups=%d" % (tuple(w.shape), c, groups))
    return make_desc(n, c, h, wd, k, r, s, stride, padding, dilation, groups, layout, xb, _dtype_of(x))


def _out_shape(desc: ConvDesc):
    oh, ow = output_dims(desc)
    if desc.layout == LAYOUT_NCHW:
        return (desc.n, desc.k, oh, ow)
    if desc.layout == LAYOUT_NHWC:
        return (desc.n, oh, ow, desc.k)
    return (desc.n, -(-desc.k // desc.x), oh, ow, desc.x)


def _stream():
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _check_dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def prepare_filter(w, desc: ConvDesc, a: Algo):
    """Prepared filter of algorithm ``a`` as a uint8 device tensor (None if it reads KCRS)."""
    torch = _torch()
    a = resolve_algo(desc, a)
    nbytes = filter_size(desc, a)
    if nbytes == 0:
        return None
    _check_dev(w)
    wp = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check(prepare_filter_raw(desc, a, w.data_ptr(), wp.data_ptr(), nbytes, _stream()))
    return wp


def conv2d_fwd(x, w, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", channels=None, algo_kind="auto",
               config_id=-1, requant_scale=None, out=None, w_prepared=None, workspace=None, bias=None, residual=None,
               relu=False):
    """y = conv(x, w) on the current stream.  Tensors on the GPU, contiguous.

    ``algo_kind`` is one of auto, implicit_gemm, winograd_f2x2_3x3,
    winograd_f6x6_3x3, direct, pointwise; ``requant_scale`` (float32 [K]) is
    required for int8.  ``w_prepared`` is the output of ``prepare_filter`` for
    the same resolved algorithm.  ``bias`` (float32 [K], int32 for int8),
    ``residual`` (shaped like the output) and ``relu`` are the fused epilogue.
    """
    torch = _torch()
    _check_dev(x, w, requant_scale, out, w_prepared, workspace, bias, residual)
    desc = desc_for(x, w, stride, padding, dilation, groups, layout, channels)
    a = resolve_algo(desc, algo(algo_kind, config_id))
    if out is None:
        out = torch.empty(_out_shape(desc), dtype=x.dtype, device=x.device)
    ws_bytes = workspace_size(desc, a) if w_prepared is None else scratch_size(desc, a)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    ep = epilogue_of(bias.data_ptr() if bias is not None else 0,
                     residual.data_ptr() if residual is not None else 0, relu)
    st = conv2d_fwd_ex_raw(desc, a, x.data_ptr(), w.data_ptr(),
                           w_prepared.data_ptr() if w_prepared is not None else 0,
                           requant_scale.data_ptr() if requant_scale is not None else 0, ep, out.data_ptr(),
                           workspace.data_ptr() if workspace is not None else 0, ws_bytes, _stream())
    _check(st)
    return out


def fastrun_select(x, w, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", channels=None,
                   requant_scale=None, out=None, workspace=None) -> Tuple[Algo, object]:
    """Run the Fast-Run selection for this problem; returns (best algo, output).

    ``workspace`` (uint8 device tensor of at least ``fastrun_workspace_size``
    bytes) is allocated here when not given.
    """
    torch = _torch()
    _check_dev(x, w, requant_scale, out, workspace)
    desc = desc_for(x, w, stride, padding, dilation, groups, layout, channels)
    if out is None:
        out = torch.empty(_out_shape(desc), dtype=x.dtype, device=x.device)
    nbytes = fastrun_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    best = Algo()
    _check(_lib().cfwd_fastrun_select(ctypes.byref(desc), x.data_ptr(), w.data_ptr(),
                                      requant_scale.data_ptr() if requant_scale is not None else None,
                                      out.data_ptr(), workspace.data_ptr(), nbytes, _stream(),
                                      ctypes.byref(best)))
    return best, out


class LayerPlan:
    """One conv layer set up the way an inference step runs it.

    ``algo="auto"``: unless the map already holds the problem, the Fast-Run
    selection phase runs once on (x, w) and records its choice in the map;
    launches then pass AUTO, so the library dispatches from the map
    (execution phase).  Otherwise the named family
    (and config, "family/cfg") is resolved once and passed explicitly.  The
    filter is prepared once (constant weights) and the algorithm's scratch is
    allocated once; ``prepare_ms`` is the prepare step's device time.
    """

    def __init__(self, x, w, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", channels=None,
                 requant_scale=None, algo_spec="auto", bias=None, relu=False):
        torch = _torch()
        _check_dev(x, w, requant_scale, bias)
        self.w, self.scale = w, requant_scale
        self.bias, self.relu = bias, relu  # fused epilogue (a residual is given per launch)
        self.desc = desc_for(x, w, stride, padding, dilation, groups, layout, channels)
        self.out_shape = _out_shape(self.desc)
        self.dtype, self.device = x.dtype, x.device
        if algo_spec == "auto":
            # a problem already in the map (an earlier layer of the same shape,
            # or a map loaded from a file) is dispatched from it unsearched
            best = fastrun_lookup(self.desc)
            if best is None:
                best, _ = fastrun_select(x, w, stride, padding, dilation, groups, layout, channels,
                                         requant_scale=requant_scale)
            self.chosen = resolve_algo(self.desc, algo())
            if self.chosen.key() != best.key():
                raise RuntimeError("AUTO resolves to %s, Fast-Run chose %s" % (algo_name(self.chosen),
                                                                               algo_name(best)))
            self.chosen.median_ms = best.median_ms
            self.algo_arg = algo()
        else:
            fam, _, cid = algo_spec.partition("/")
            self.chosen = resolve_algo(self.desc, algo(fam, int(cid) if cid else -1))
            self.algo_arg = self.chosen
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        self.wp = prepare_filter(w, self.desc, self.chosen)
        e1.record()
        torch.cuda.synchronize()
        self.prepare_ms = e0.elapsed_time(e1) if self.wp is not None else 0.0
        self.scratch_bytes = scratch_size(self.desc, self.chosen)
        self.scratch = torch.empty(max(self.scratch_bytes, 16), dtype=torch.uint8, device=x.device)

    @property
    def name(self) -> str:
        return algo_name(self.chosen)

    def new_output(self):
        return _torch().empty(self.out_shape, dtype=self.dtype, device=self.device)

    def launch_raw(self, x_ptr: int, y_ptr: int, stream: int, residual_ptr: int = 0) -> int:
        """Enqueue the layer on ``stream`` with raw device pointers; returns the status."""
        ep = epilogue_of(self.bias.data_ptr() if self.bias is not None else 0, residual_ptr, self.relu)
        return conv2d_fwd_ex_raw(self.desc, self.algo_arg, x_ptr, self.w.data_ptr(),
                                 self.wp.data_ptr() if self.wp is not None else 0,
                                 self.scale.data_ptr() if self.scale is not None else 0, ep, y_ptr,
                                 self.scratch.data_ptr() if self.scratch_bytes else 0, self.scratch_bytes, stream)

    def __call__(self, x, out=None, residual=None):
        """y = conv(x) (+ the fused epilogue) on the current stream (x shaped and typed like the set-up input)."""
        _check_dev(x, out, residual)
        if out is None:
            out = self.new_output()
        _check(self.launch_raw(x.data_ptr(), out.data_ptr(), _stream(),
                               residual.data_ptr() if residual is not None else 0))
        return out


# ------------------------------------------------------- fused bottleneck block

_DTYPE_CODES = {"f32": F32, "fp32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16, "i8": I8, "int8": I8}


def bottleneck_desc(n, c, h, w, mid, k, dtype="bf16") -> BottleneckDesc:
    return BottleneckDesc(n, c, h, w, mid, k, _DTYPE_CODES[dtype] if isinstance(dtype, str) else dtype)


def bottleneck_check(desc: BottleneckDesc) -> None:
    """Raise CfwdError (UNSUPPORTED with the reason) unless the fused kernel runs this block."""
    _check(_lib().cfwd_bottleneck_check(ctypes.byref(desc)))


def bottleneck_filter_size(desc: BottleneckDesc) -> int:
    b = ctypes.c_size_t()
    _check(_lib().cfwd_bottleneck_filter_size(ctypes.byref(desc), ctypes.byref(b)))
    return b.value


def bottleneck_desc_for(x, w1, w3) -> BottleneckDesc:
    n, c, h, wd = x.shape
    return bottleneck_desc(n, c, h, wd, w1.shape[0], w3.shape[0], _dtype_of(x))


def bottleneck_prepare(w2, desc: BottleneckDesc):
    """Prepared 3x3 weights of the block (uint8 device tensor)."""
    torch = _torch()
    _check_dev(w2)
    nbytes = bottleneck_filter_size(desc)
    wp = torch.empty(nbytes, dtype=torch.uint8, device=w2.device)
    _check(_lib().cfwd_bottleneck_prepare(ctypes.byref(desc), w2.data_ptr(), wp.data_ptr(), nbytes, _stream()))
    return wp


def bottleneck_fwd_raw(desc: BottleneckDesc, x: int, w1: int, w2p: int, w3: int, ep, y: int, stream) -> int:
    """cfwd_bottleneck_fwd with integer device pointers; returns the status."""
    return _lib().cfwd_bottleneck_fwd(ctypes.byref(desc), x, w1, w2p, w3, ctypes.byref(ep) if ep is not None else None,
                                      y, stream)


def bottleneck_fwd(x, w1, w2_prepared, w3, b1=None, b2=None, b3=None, residual=None, relu=(False, False, False),
                   out=None):
    """y = the fused bottleneck block of NCHW ``x`` on the current stream (see cfwd.h)."""
    torch = _torch()
    _check_dev(x, w1, w2_prepared, w3, b1, b2, b3, residual, out)
    desc = bottleneck_desc_for(x, w1, w3)
    if out is None:
        out = torch.empty((desc.n, desc.k, desc.h, desc.w), dtype=x.dtype, device=x.device)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    ep = BottleneckEpilogue(ptr(b1), ptr(b2), ptr(b3), ptr(residual), int(bool(relu[0])), int(bool(relu[1])),
                            int(bool(relu[2])))
    _check(bottleneck_fwd_raw(desc, x.data_ptr(), w1.data_ptr(), w2_prepared.data_ptr(), w3.data_ptr(), ep,
                              out.data_ptr(), _stream()))
    return out


# ------------------------------------------------------- layout conversion

def convert_layout(t, src_layout: str, dst_layout: str, dst_x: int = 0, channels: Optional[int] = None, out=None):
    """Copy activations between NCHW [N,C,H,W], NHWC [N,H,W,C] and NCHWX [N,CB,H,W,X] (cfwd_convert_layout)."""
    torch = _torch()
    _check_dev(t, out)
    sl, dl = src_layout.upper(), dst_layout.upper()
    if sl == "NCHW":
        n, c, h, w = t.shape
        sx = 0
    elif sl == "NHWC":
        n, h, w, c = t.shape
        sx = 0
    else:
        n, cb, h, w, sx = t.shape
        c = channels if channels is not None else cb * sx
    shape = {"NCHW": (n, c, h, w), "NHWC": (n, h, w, c)}.get(dl) or (n, -(-c // dst_x), h, w, dst_x)
    if out is None:
        out = torch.empty(shape, dtype=t.dtype, device=t.device)
    _check(_lib().cfwd_convert_layout(n, c, h, w, _DTYPE_CODES[_dtype_of(t)], _LAYOUTS[sl], sx, t.data_ptr(),
                                      _LAYOUTS[dl], int(dst_x), out.data_ptr(), _stream()))
    return out


# ------------------------------------------------------- 4-bit weights

def unpack_int4(packed, count: int, out=None):
    """int8 tensor of ``count`` signed 4-bit values packed two per byte, low nibble first (cfwd_unpack_int4)."""
    torch = _torch()
    _check_dev(packed, out)
    if out is None:
        out = torch.empty(count, dtype=torch.int8, device=packed.device)
    _check(_lib().cfwd_unpack_int4(packed.data_ptr(), out.data_ptr(), int(count), _stream()))
    return out
