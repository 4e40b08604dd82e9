"""Build libcfwd.so (the HIP library behind include/cfwd.h) for gfx950.

Every source under csrc/ is compiled with hipcc into csrc/../_build/*.o, in
parallel, then linked into cnn_convolution_fwd_amd/libcfwd.so.  Runs on a
machine without a GPU (hipcc cross-compiles).  Usage:

    python -m cnn_convolution_fwd_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC_DIR = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcfwd.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


COMMON = [
    "-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH,
    # packed fp32 ALU forms are kept out of generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    "-I", INCLUDE, "-I", SRC_DIR,
]


# Per-source extra flags.  The stem kernels (gather form and the int8 NCHW4
# stem) and the persistent int8 kernel are bound by vector ALU issue; keeping
# MFMA results in ordinary VGPRs instead of accumulation registers removes the
# register moves around their epilogues (about a tenth of their vector
# instructions) without raising register use (in the persistent kernel it
# lowers it: two of its 3x3 variants fall under 256 registers, and the
# epilogue variants of its widest tile spill less).
EXTRA = {
    "k_lowc.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "k_stem_i8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "k_igemm_i8_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(SRC_DIR, f) for f in os.listdir(SRC_DIR)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (src, r.stdout, r.stderr))
    if r.stderr.strip() and verbose:
        print(r.stderr, file=sys.stderr)
    return obj


def _stale(src: str) -> bool:
    """True when src's object is missing or older than src or any header."""
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    headers = [os.path.join(SRC_DIR, f) for f in os.listdir(SRC_DIR) if f.endswith(".h")]
    headers.append(os.path.join(INCLUDE, "cfwd.h"))
    return any(os.path.getmtime(f) > t for f in [src, *headers, os.path.abspath(__file__)])


def build(jobs: int = 0, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (only stale ones when ``incremental``) and link
    libcfwd.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    if incremental:
        stale = [s for s in srcs if _stale(s)]
        if stale:
            with cf.ThreadPoolExecutor(max_workers=jobs or min(len(stale), 16)) as ex:
                list(ex.map(lambda s: _compile(s, verbose), stale))
        objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
        return _link(objs, verbose)
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    return _link(objs, verbose)


def _link(objs, verbose: bool) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--incremental", action="store_true", help="recompile only sources newer than their objects")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.incremental))


if __name__ == "__main__":
    main()
