"""Helpers shared by the GPU parity tests: move seeded numpy problems to the
device, run the HIP library through its C ABI, and bring results back."""
import functools

import numpy as np
import pytest

import oracle

from cnn_convolution_fwd_amd import binding as B
from cnn_convolution_fwd_amd.workloads import bf16_bits, bf16_to_f32, pack_nchwx, unpack_nchwx

TOL = {"f32": 1e-5, "bf16": 1e-2}
TOL_WINOGRAD = {"f32": 1e-3, "bf16": 1e-2}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_device(arr, dtype):
    """numpy float32 (bf16-exact for bf16) / int8 array -> torch device tensor."""
    torch = torch_cuda()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    if dtype == "bf16":
        bits = bf16_bits(arr).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.bfloat16)
    if dtype == "i8":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int8)).cuda()
    raise ValueError(dtype)


def from_device(t, dtype):
    torch = torch_cuda()
    torch.cuda.synchronize()
    if dtype == "bf16":
        return bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float32)
    return t.cpu().numpy()


def run_conv(x, w, dtype, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", xb=None, algo="auto",
             config_id=-1, scale=None, prepared=False):
    """Run the GPU convolution on logical-NCHW numpy inputs; returns logical-NCHW numpy output."""
    torch = torch_cuda()
    C = x.shape[1]
    xin = pack_nchwx(x, xb) if layout == "NCHWX" else x
    xd = to_device(xin, dtype)
    wd = to_device(w, dtype)
    sd = torch.from_numpy(np.ascontiguousarray(scale, dtype=np.float32)).cuda() if scale is not None else None
    wp = None
    if prepared:
        desc = B.desc_for(xd, wd, stride, padding, dilation, groups, layout, channels=C)
        wp = B.prepare_filter(wd, desc, B.algo(algo, config_id))
    y = B.conv2d_fwd(xd, wd, stride, padding, dilation, groups, layout, channels=C, algo_kind=algo,
                     config_id=config_id, requant_scale=sd, w_prepared=wp)
    out = from_device(y, dtype)
    if layout == "NCHWX":
        K = w.shape[0]
        # channels past K in the last block must have been written as 0
        full = out.transpose(0, 1, 4, 2, 3).reshape(out.shape[0], -1, out.shape[2], out.shape[3])
        assert np.all(full[:, K:] == 0), "padded output channels are not zero"
        out = unpack_nchwx(out, K)
    return out


def candidates_for(shape, dtype, stride=1, padding=0, dilation=1, groups=1, layout="NCHW", xb=None):
    N, C, H, W, K, R, S = shape
    d = B.make_desc(N, C, H, W, K, R, S, stride, padding, dilation, groups, layout, xb, dtype)
    return [(B.algo_name(a).split("/")[0], a.config_id) for a in B.list_candidates(d)]


def output_to_host(y, dtype, layout, K):
    """Device output -> logical-NCHW numpy; NCHWX channels past K must be 0."""
    out = from_device(y, dtype)
    if layout == "NCHWX":
        full = out.transpose(0, 1, 4, 2, 3).reshape(out.shape[0], -1, out.shape[2], out.shape[3])
        assert np.all(full[:, K:] == 0), "padded output channels are not zero"
        out = unpack_nchwx(out, K)
    return out


@functools.lru_cache(maxsize=4)
def float_reference(config, layer_idx, n, dtype):
    """(problem, y, den) of a float workload layer at batch n: the whole tensor from the oracle."""
    from cnn_convolution_fwd_amd.workloads import float_problem
    pr = float_problem(config, layer_idx, n=n, dtype=dtype)
    L = pr.layer
    y, den = oracle.conv2d(pr.x, pr.w, L.stride, L.pad, L.dil, L.groups)
    return pr, y, den


@functools.lru_cache(maxsize=4)
def int8_reference(config, layer_idx, n):
    """(problem, y) of an int8 workload layer at batch n: the whole tensor from the oracle."""
    from cnn_convolution_fwd_amd.workloads import int8_problem
    pr = int8_problem(config, layer_idx, n=n)
    L = pr.layer
    y, _ = oracle.conv2d_int8_requant(pr.x, pr.w, pr.scale, L.stride, L.pad, L.dil, L.groups)
    return pr, y
