"""The C ABI on the host, without a GPU: the library loads, exports every
entry point include/cfwd.h declares, validates descriptors, sizes buffers,
lists candidates and applies the Fast-Run choice rule."""
import os
import re

import pytest

from cnn_convolution_fwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "cfwd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cfwd_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.library()
    declared = header_functions()
    assert len(declared) >= 18
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTED)


def test_version():
    assert B.version().startswith("cfwd ")


@pytest.mark.parametrize("H,R,s,p,d,expected", [(56, 3, 1, 1, 1, 56), (224, 7, 2, 3, 1, 112), (224, 3, 2, 1, 1, 112),
                                                 (56, 1, 2, 0, 1, 28), (4, 2, 2, 0, 1, 2), (7, 3, 1, 0, 3, 1)])
def test_output_dims(H, R, s, p, d, expected):
    desc = B.make_desc(1, 4, H, H, 4, R, R, s, p, d)
    assert B.output_dims(desc) == (expected, expected)


@pytest.mark.parametrize("kw", [dict(n=0), dict(c=0), dict(k=-1), dict(r=0), dict(stride=0), dict(dilation=0),
                                dict(padding=-1), dict(groups=4), dict(h=2, r=5)])
def test_invalid_descriptors(kw):
    base = dict(n=1, c=6, h=8, w=8, k=6, r=3, s=3, stride=1, padding=1, dilation=1, groups=1)
    base.update(kw)
    if "r" in kw:
        base["s"] = kw["r"]
    if "h" in kw:
        base["w"] = kw["h"]
        base["padding"] = 0
    desc = B.make_desc(**base)
    with pytest.raises(B.CfwdError) as e:
        B.output_dims(desc)
    assert e.value.status == B.ERR_INVALID_ARG


def test_bad_layout_block():
    desc = B.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, 1, 1, "NCHWX", 3, "i8")
    with pytest.raises(B.CfwdError) as e:
        B.output_dims(desc)
    assert e.value.status == B.ERR_INVALID_ARG


def test_too_large_image_unsupported():
    desc = B.make_desc(1, 1 << 16, 1 << 8, 1 << 8, 4, 1, 1)
    with pytest.raises(B.CfwdError) as e:
        B.output_dims(desc)
    assert e.value.status == B.ERR_UNSUPPORTED


def test_auto_heuristic_preferences():
    dw = B.make_desc(64, 32, 112, 112, 32, 3, 3, 1, 1, 1, 32, dtype="f32")
    assert B.algo_name(B.resolve_algo(dw, B.algo())).startswith("direct")
    dense = B.make_desc(32, 256, 56, 56, 256, 3, 3, 1, 1, 1, 1, dtype="bf16")
    assert B.algo_name(B.resolve_algo(dense, B.algo())).startswith("implicit_gemm")
    # Winograd is never chosen without measurement
    for kind in ("winograd_f2x2_3x3", "winograd_f6x6_3x3"):
        assert not B.algo_name(B.resolve_algo(dense, B.algo())).startswith(kind)


def test_candidates_order_and_validity():
    desc = B.make_desc(32, 256, 56, 56, 256, 3, 3, 1, 1, 1, 1, dtype="bf16")
    c = B.list_candidates(desc)
    rank = {B.ALGO_IMPLICIT_GEMM: 0, B.ALGO_POINTWISE: 1, B.ALGO_DIRECT: 2, B.ALGO_WINOGRAD_F2X2_3X3: 3,
            B.ALGO_WINOGRAD_F6X6_3X3: 4}
    keys = [(rank[a.kind], a.config_id) for a in c]
    assert keys == sorted(keys)
    for a in c:
        assert B.resolve_algo(desc, a).key() == a.key()


def test_winograd_refuses_unsupported_problems():
    for desc in (B.make_desc(1, 8, 8, 8, 8, 3, 3, 2, 1, dtype="f32"),       # stride 2
                 B.make_desc(1, 8, 8, 8, 8, 5, 5, 1, 2, dtype="f32"),       # 5x5
                 B.make_desc(1, 8, 8, 8, 8, 3, 3, 2, 1, dtype="i8"),        # int8 stride 2
                 B.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, 1, 2, dtype="f32")):  # groups
        for kind in ("winograd_f2x2_3x3", "winograd_f6x6_3x3"):
            with pytest.raises(B.CfwdError) as e:
                B.resolve_algo(desc, B.algo(kind))
            assert e.value.status == B.ERR_UNSUPPORTED
    # int8: F(2x2) three-launch form only (F(6x6) transforms are not exact in fp16)
    i8 = B.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, dtype="i8")
    with pytest.raises(B.CfwdError) as e:
        B.resolve_algo(i8, B.algo("winograd_f6x6_3x3"))
    assert e.value.status == B.ERR_UNSUPPORTED
    for cfg in (1, 2):
        with pytest.raises(B.CfwdError):
            B.resolve_algo(i8, B.algo("winograd_f2x2_3x3", cfg))


@pytest.mark.parametrize("layout,xb", [("NCHW", None), ("NCHWX", 4), ("NCHWX", 8)])
def test_int8_winograd_is_opt_in(layout, xb):
    """int8 Winograd F(2x2) runs when named, and joins the candidate list only
    after cfwd_fastrun_allow_inexact_int8(1); AUTO never picks it unmeasured."""
    desc = B.make_desc(2, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, layout, xb, "i8")
    a = B.resolve_algo(desc, B.algo("winograd_f2x2_3x3"))
    assert (a.kind, a.config_id) == (B.ALGO_WINOGRAD_F2X2_3X3, 0)
    # prepared filter: 16 positions x 1 K block of 64 x 2 chunks of 32 channels x 64 x 64 bytes
    assert B.filter_size(desc, a) == 16 * 1 * 2 * 64 * 64
    # scratch: 16 positions x 2 chunks x 2 * 28 * 28 tiles (padded to 64) x 64 bytes, no maxima area
    tiles = (2 * 28 * 28 + 63) // 64 * 64
    assert B.scratch_size(desc, a) == 16 * 2 * tiles * 64
    kinds = lambda: [x.kind for x in B.list_candidates(desc)]  # noqa: E731
    try:
        assert B.ALGO_WINOGRAD_F2X2_3X3 not in kinds()
        B.fastrun_allow_inexact_int8(True)
        assert B.ALGO_WINOGRAD_F2X2_3X3 in kinds()
        assert B.fastrun_workspace_size(desc) >= B.workspace_size(desc, a)
    finally:
        B.fastrun_allow_inexact_int8(False)
    assert B.ALGO_WINOGRAD_F2X2_3X3 not in kinds()
    assert B.resolve_algo(desc, B.algo()).kind != B.ALGO_WINOGRAD_F2X2_3X3


def test_filter_and_workspace_sizes():
    desc = B.make_desc(32, 256, 56, 56, 256, 3, 3, 1, 1, 1, 1, dtype="bf16")
    a = B.algo("implicit_gemm", 0)
    # 256 K (2 tiles of 128) x 8 chunks of 32 channels x 9 taps x 128 x 64 bytes
    assert B.filter_size(desc, a) == 2 * 8 * 9 * 128 * 64
    assert B.workspace_size(desc, a) == B.filter_size(desc, a)
    assert B.filter_size(desc, B.algo("direct", 0)) == 0
    assert B.fastrun_workspace_size(desc) > 3 * 32 * 256 * 56 * 56 * 2


def test_conv_rejects_bad_pointers_without_touching_the_gpu():
    desc = B.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, dtype="f32")
    a = B.algo("direct", 0)
    assert B.conv2d_fwd_raw(desc, a, 0, 0x1000, 0, 0, 0x2000, 0, 0, 0) == B.ERR_INVALID_ARG   # x NULL
    assert B.conv2d_fwd_raw(desc, a, 0x1004, 0x1000, 0, 0, 0x2000, 0, 0, 0) == B.ERR_INVALID_ARG  # misaligned
    assert B.conv2d_fwd_raw(desc, a, 0x1000, 0x1000, 0, 0x3000, 0x2000, 0, 0, 0) == B.ERR_INVALID_ARG  # scale on f32
    d8 = B.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, dtype="i8")
    assert B.conv2d_fwd_raw(d8, a, 0x1000, 0x1000, 0, 0, 0x2000, 0, 0, 0) == B.ERR_INVALID_ARG  # int8 without scale
    ig = B.algo("implicit_gemm", 0)
    assert B.conv2d_fwd_raw(desc, ig, 0x1000, 0x1000, 0, 0, 0x2000, 0, 0, 0) == B.ERR_WORKSPACE
    assert "workspace" in B.library().cfwd_last_error().decode()


def test_fastrun_choose_rule():
    ig0, ig1, dr = B.algo("implicit_gemm", 0), B.algo("implicit_gemm", 1), B.algo("direct", 0)
    # median, not mean: one outlier does not decide
    assert B.fastrun_choose([ig0, ig1], [[1, 1, 1, 1, 9], [0.9, 0.9, 0.9, 0.9, 0.9]], [1, 1]) == 1
    # within 1%: the earlier candidate keeps the choice
    assert B.fastrun_choose([ig0, ig1], [[1.0] * 5, [0.995] * 5], [1, 1]) == 0
    assert B.fastrun_choose([ig0, ig1], [[1.0] * 5, [0.985] * 5], [1, 1]) == 1
    # a failed accuracy gate excludes the fastest
    assert B.fastrun_choose([ig0, dr], [[1.0] * 5, [0.1] * 5], [1, 0]) == 0
    assert B.fastrun_choose([ig0, dr], [[1.0] * 5, [0.1] * 5], [0, 0]) == -1


def test_fastrun_map_file_handling(tmp_path):
    B.fastrun_clear()
    missing = str(tmp_path / "missing.txt")
    B.fastrun_load(missing)  # ignored
    bad = tmp_path / "bad.txt"
    bad.write_text("not a map\nfoo\tbar\n")
    B.fastrun_load(str(bad))  # ignored
    corrupt = tmp_path / "corrupt.txt"
    corrupt.write_text("cfwd-fastrun 1\nx|1|kset|1,2\t9\t0\t1.0\nshort line\n")
    B.fastrun_load(str(corrupt))
    out = str(tmp_path / "out.txt")
    B.fastrun_save(out)
    assert open(out).read().startswith("cfwd-fastrun 1\n")
    with pytest.raises(B.CfwdError) as e:
        B.fastrun_save(str(tmp_path / "no_dir" / "x.txt"))
    assert e.value.status == B.ERR_CACHE_IO
    # without a GPU there is no device to key the map by: lookups miss
    desc = B.make_desc(1, 8, 8, 8, 8, 3, 3, 1, 1, dtype="f32")
    assert B.fastrun_lookup(desc) is None


def test_bottleneck_block_checks_on_the_host():
    ok = B.bottleneck_desc(32, 256, 56, 56, 64, 256)
    B.bottleneck_check(ok)
    assert B.bottleneck_filter_size(ok) == 9 * 64 * 64 * 2
    for bad in (B.bottleneck_desc(32, 256, 56, 56, 64, 256, "f32"),   # dtype
                B.bottleneck_desc(32, 256, 56, 56, 128, 256),         # inner channels
                B.bottleneck_desc(32, 250, 56, 56, 64, 256),          # C % 32
                B.bottleneck_desc(32, 256, 56, 56, 64, 250),          # K % 32
                B.bottleneck_desc(32, 256, 56, 60, 64, 256),          # W % 8
                B.bottleneck_desc(32, 256, 56, 72, 64, 256)):         # W > 64
        with pytest.raises(B.CfwdError) as e:
            B.bottleneck_check(bad)
        assert e.value.status == B.ERR_UNSUPPORTED
    with pytest.raises(B.CfwdError) as e:
        B.bottleneck_check(B.bottleneck_desc(0, 256, 56, 56, 64, 256))
    assert e.value.status == B.ERR_UNSUPPORTED
    # argument validation happens before anything is enqueued
    d = B.bottleneck_desc(1, 32, 8, 8, 64, 32)
    ep = B.BottleneckEpilogue()
    assert B.bottleneck_fwd_raw(d, 0, 16, 16, 16, ep, 4096, None) == B.ERR_INVALID_ARG       # NULL x
    assert B.bottleneck_fwd_raw(d, 8, 16, 16, 16, ep, 1 << 20, None) == B.ERR_INVALID_ARG   # misaligned x
    assert B.bottleneck_fwd_raw(d, 4096, 16, 16, 16, ep, 4096 + 512, None) == B.ERR_INVALID_ARG  # y overlaps x
    ep_bad = B.BottleneckEpilogue(2, None, None, None, 0, 0, 0)
    assert B.bottleneck_fwd_raw(d, 4096, 16, 16, 16, ep_bad, 1 << 20, None) == B.ERR_INVALID_ARG  # bias alignment
    ep_res = B.BottleneckEpilogue(None, None, None, (1 << 20) + 256, 0, 0, 0)
    assert B.bottleneck_fwd_raw(d, 4096, 16, 16, 16, ep_res, 1 << 20, None) == B.ERR_INVALID_ARG  # residual overlaps y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nhwc_routes_to_its_own_configs(dtype):
    desc = B.make_desc(32, 256, 56, 56, 256, 3, 3, 1, 1, 1, 1, "NHWC", None, dtype)
    cands = B.list_candidates(desc)
    assert len(cands) == 1 and all(a.kind == B.ALGO_IMPLICIT_GEMM for a in cands)
    nhwc_cfg = cands[0].config_id
    assert B.resolve_algo(desc, B.algo()).key() == cands[0].key()
    assert B.resolve_algo(desc, B.algo("implicit_gemm")).key() == cands[0].key()
    # weights [K][R][S][C] (C already a whole chunk)
    assert B.filter_size(desc, cands[0]) == 256 * 9 * 256 * (4 if dtype == "f32" else 2)
    for kind in ("direct", "pointwise", "winograd_f2x2_3x3", "winograd_f6x6_3x3"):
        with pytest.raises(B.CfwdError):
            B.resolve_algo(desc, B.algo(kind))
    with pytest.raises(B.CfwdError):
        B.resolve_algo(desc, B.algo("implicit_gemm", 0))
    # the NHWC config does not take NCHW problems
    nchw = B.make_desc(32, 256, 56, 56, 256, 3, 3, 1, 1, 1, 1, "NCHW", None, dtype)
    with pytest.raises(B.CfwdError):
        B.resolve_algo(nchw, B.algo("implicit_gemm", nhwc_cfg))
    # outside the NHWC kernel's scope there is no algorithm, AUTO included
    for bad in (B.make_desc(1, 6, 8, 8, 8, 3, 3, 1, 1, 1, 1, "NHWC", None, dtype),       # C % 8 (bf16), C % 4 (fp32)
                B.make_desc(1, 16, 8, 8, 16, 3, 3, 1, 1, 1, 2, "NHWC", None, dtype),     # groups
                B.make_desc(1, 16, 8, 8, 16, 3, 3, 1, 1, 1, 1, "NHWC", None, "i8")):     # int8
        assert B.list_candidates(bad) == []
        with pytest.raises(B.CfwdError) as e:
            B.resolve_algo(bad, B.algo())
        assert e.value.status == B.ERR_UNSUPPORTED


def test_convert_layout_validation_on_the_host():
    lib = B.library()
    args = (2, 8, 4, 4, B.BF16)
    assert lib.cfwd_convert_layout(*args, 7, 0, 4096, B.LAYOUT_NHWC, 0, 1 << 20, None) == B.ERR_INVALID_ARG  # layout
    assert lib.cfwd_convert_layout(*args, B.LAYOUT_NCHWX, 3, 4096, B.LAYOUT_NHWC, 0, 1 << 20, None) == B.ERR_INVALID_ARG
    assert lib.cfwd_convert_layout(*args, B.LAYOUT_NCHW, 0, None, B.LAYOUT_NHWC, 0, 1 << 20, None) == B.ERR_INVALID_ARG
    assert lib.cfwd_convert_layout(*args, B.LAYOUT_NCHW, 0, 4096, B.LAYOUT_NHWC, 0, 4096 + 64, None) == B.ERR_INVALID_ARG
    assert lib.cfwd_convert_layout(*args, B.LAYOUT_NCHW, 0, 4097, B.LAYOUT_NHWC, 0, 1 << 20, None) == B.ERR_INVALID_ARG
    assert lib.cfwd_convert_layout(0, 8, 4, 4, B.BF16, B.LAYOUT_NCHW, 0, 4096, B.LAYOUT_NHWC, 0, 1 << 20,
                                   None) == B.ERR_INVALID_ARG


def test_unpack_int4_validation_on_the_host():
    lib = B.library()
    assert lib.cfwd_unpack_int4(None, 4096, 10, None) == B.ERR_INVALID_ARG                # NULL
    assert lib.cfwd_unpack_int4(4096, 8192, 0, None) == B.ERR_INVALID_ARG                 # count
    assert lib.cfwd_unpack_int4(4104, 8192, 10, None) == B.ERR_INVALID_ARG                # misaligned
    assert lib.cfwd_unpack_int4(4096, 4096 + 16, 64, None) == B.ERR_INVALID_ARG           # overlap


def test_cfwd_log_reports_failures(tmp_path):
    """CFWD_LOG=1 prints each failure's reason to stderr (environment read once per process)."""
    import subprocess
    import sys as _sys
    code = ("from cnn_convolution_fwd_amd import binding as B\n"
            "d = B.make_desc(1, 8, 8, 8, 8, 3, 3, 2, 1, dtype='f32')\n"
            "try:\n    B.resolve_algo(d, B.algo('winograd_f2x2_3x3'))\nexcept B.CfwdError:\n    pass\n")
    env = dict(os.environ, CFWD_LOG="1")
    r = subprocess.run([_sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert "cfwd: winograd" in r.stderr
    env["CFWD_LOG"] = "0"
    r = subprocess.run([_sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert "cfwd:" not in r.stderr
