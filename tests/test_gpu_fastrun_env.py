"""Fast-Run's environment flags on the GPU (each read once per process, so
each case runs in a child process): CFWD_FASTRUN_CACHE loads a saved map
before the first AUTO call; CFWD_FASTRUN_MODE=off makes AUTO ignore it."""
import os
import subprocess
import sys

import pytest

from cnn_convolution_fwd_amd import binding as B
from cnn_convolution_fwd_amd.workloads import Layer, random_float_problem
from tests.gpu_util import to_device, torch_cuda

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = ("import torch\n"
         "from cnn_convolution_fwd_amd import binding as B\n"
         "torch.cuda.init()\n"
         "d = B.make_desc(2, 32, 12, 12, 48, 3, 3, 1, 1, 1, 1, 'NCHW', None, 'f32')\n"
         "print('AUTO', B.algo_name(B.resolve_algo(d, B.algo())))\n")


def child(**env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, "-c", CHILD], env=e, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    return [l.split()[1] for l in r.stdout.splitlines() if l.startswith("AUTO")][0]


def test_cache_file_and_mode_off(tmp_path):
    torch = torch_cuda()
    B.fastrun_clear()
    pr = random_float_problem(Layer("env", 32, 48, 12, 12, 3, 3, 1, 1, 1, 1), 2, "f32", 3)
    xd, wd = to_device(pr.x, "f32"), to_device(pr.w, "f32")
    best, _ = B.fastrun_select(xd, wd, 1, 1)
    path = str(tmp_path / "map.txt")
    B.fastrun_save(path)
    B.fastrun_clear()
    torch.cuda.synchronize()
    # point the entry at a candidate the fixed preference never picks for a
    # dense 3x3 layer (the generic direct kernel), so the three cases differ
    lines = open(path).read().splitlines()
    assert lines[0] == "cfwd-fastrun 1" and len(lines) == 2, lines
    key, kind, cfg, ms = lines[1].split("\t")
    open(path, "w").write("%s\n%s\t%d\t0\t%s\n" % (lines[0], key, B.ALGO_DIRECT, ms))
    fixed = child()                                           # no map: the fixed preference
    cached = child(CFWD_FASTRUN_CACHE=path)                   # the map file's entry
    off = child(CFWD_FASTRUN_CACHE=path, CFWD_FASTRUN_MODE="off")
    print("selected", B.algo_name(best), "fixed", fixed, "cached", cached, "off", off, flush=True)
    assert fixed.startswith("implicit_gemm")
    assert cached == "direct/0"
    assert off == fixed
