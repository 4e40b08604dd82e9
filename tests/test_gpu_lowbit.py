"""GPU parity of the 4-bit weight path (cfwd_unpack_int4): unpacking is
bit-exact against the numpy unpacking pinned in test_layout_np.py, and a
convolution with unpacked 4-bit weights is bit-identical to the oracle's
exact int8 convolution with the same values (the int8 path's bar).

MegEngine CPU-inference article, section "结论": lower-bit quantisation is
named as a next step; gfx950 has no int4 matrix operands, so the weights are
widened to int8 once, when loaded.
"""
import sys

import numpy as np
import pytest

import oracle
from cnn_convolution_fwd_amd import binding as B
from cnn_convolution_fwd_amd.workloads import CONFIGS, int8_problem, pack_int4, pack_nchwx, unpack_int4, unpack_nchwx
from tests.gpu_util import from_device, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("count", [1, 2, 31, 32, 33, 64, 1000001])
def test_unpack_int4_exact(count):
    torch = torch_cuda()
    v = np.random.default_rng(count).integers(-8, 8, count)
    p = pack_int4(v)
    pd = torch.from_numpy(np.concatenate([p, np.zeros(16, np.uint8)])).cuda()  # room for the vector loads' alignment
    say("unpack", count)
    out = from_device(B.unpack_int4(pd, count), "i8")
    np.testing.assert_array_equal(out, unpack_int4(p, count))
    np.testing.assert_array_equal(out, v.astype(np.int8))


@pytest.mark.parametrize("layer_idx", [1, 5, 7, 16])
def test_conv_with_4bit_weights(layer_idx):
    """ResNet-18 int8 layer (NCHW4, N=2) with its weights narrowed to 4 bits:
    the default algorithm on the unpacked weights equals the oracle exactly."""
    torch = torch_cuda()
    L = CONFIGS[5].layers[layer_idx]
    pr = int8_problem(5, layer_idx, n=2)
    w4 = np.clip(np.rint(pr.w.astype(np.float64) / 16.0), -8, 7).astype(np.int8)  # 4-bit grid, same channel scales
    scale = (pr.scale * 16.0).astype(np.float32)
    packed = pack_int4(w4)
    pd = torch.from_numpy(np.concatenate([packed, np.zeros(16, np.uint8)])).cuda()
    wd = B.unpack_int4(pd, w4.size).view(w4.shape)
    xd = to_device(pack_nchwx(pr.x, 4), "i8")
    sd = torch.from_numpy(scale).cuda()
    say("4-bit weights", L.name)
    y = B.conv2d_fwd(xd, wd, L.stride, L.pad, L.dil, L.groups, "NCHWX", channels=L.c, requant_scale=sd)
    got = unpack_nchwx(from_device(y, "i8"), L.k)
    ref, _ = oracle.conv2d_int8_requant(pr.x, w4, scale, L.stride, L.pad, L.dil, L.groups)
    assert np.array_equal(got, ref), "%d of %d outputs differ" % (int((got != ref).sum()), got.size)
