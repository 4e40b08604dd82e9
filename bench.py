#!/usr/bin/env python3
"""Benchmark: forward convolution of the ResNet 3x3 256-channel layer at 56x56.

One step = one forward convolution of the whole batch (N=32, C=K=256,
56x56, 3x3, stride 1, pad 1, bf16 in / fp32 accumulate / bf16 out, NCHW)
through the C ABI with AUTO dispatch: the Fast-Run selection phase runs once
during set-up (untimed), every timed step dispatches from the Fast-Run map
(execution phase) with the filter prepared once, as inference does with
constant weights.  Inputs are seeded synthetic data (x ~ N(0,1),
w ~ N(0, 2/fan_in)), already resident in HBM; the timed loop rotates over
enough input/output buffer sets (> 512 MB, twice the 256 MB Infinity Cache)
that no step reads its input from the cache a previous step filled.

Prints ONE JSON line with the throughput, the roofline of the dominant kernel
(HIP events around every launch, on the stream the kernel runs on) and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--dtype bf16|f32] [--algo auto|implicit_gemm/<cfg>|...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv TFLOP/s (int8 TOP/s) + % MFMA/HBM roofline, ResNet 3x3 256ch@56x56"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--algo", default="auto", help="auto (Fast-Run) or family[/config], e.g. implicit_gemm/1")
    ap.add_argument("--sets", type=int, default=0, help="rotated buffer sets (0: enough for > 512 MB)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle CPU work at most")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (batch sharding is described in "
              "DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from cnn_convolution_fwd_amd import binding as B
    from cnn_convolution_fwd_amd.roofline import PEAK, layer_bytes, layer_flops
    from cnn_convolution_fwd_amd.workloads import CONFIGS, bf16_bits, float_problem

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg = CONFIGS[3]
    L = cfg.layers[0]
    N = cfg.n
    pr = float_problem(3, dtype=a.dtype)

    def to_dev(arr):
        if a.dtype == "bf16":
            return torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)

    x0 = to_dev(pr.x)
    w = to_dev(pr.w)
    esize = 2 if a.dtype == "bf16" else 4
    set_bytes = (x0.numel() + N * L.k * L.h * L.w) * esize
    nsets = a.sets or max(2, -(-512 * 2**20 // set_bytes) + 1)
    xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
    desc = B.desc_for(x0, w, L.stride, L.pad, L.dil, L.groups)
    oh, ow = B.output_dims(desc)
    ys = [torch.empty((N, L.k, oh, ow), dtype=x0.dtype, device=dev) for _ in range(nsets)]

    # Fast-Run selection (untimed set-up), then the execution phase dispatches from the map.
    if a.algo == "auto":
        B.fastrun_clear()
        best, _ = B.fastrun_select(x0, w, L.stride, L.pad, L.dil, L.groups, out=ys[0])
        chosen = B.resolve_algo(desc, B.algo())
        assert chosen.key() == best.key()
        algo_arg = B.algo()  # AUTO: dispatch from the Fast-Run map
    else:
        fam, _, cid = a.algo.partition("/")
        chosen = B.resolve_algo(desc, B.algo(fam, int(cid) if cid else -1))
        algo_arg = chosen
    wp = B.prepare_filter(w, desc, chosen)
    wp_ptr = wp.data_ptr() if wp is not None else 0
    sbytes = B.scratch_size(desc, chosen)  # Winograd: transformed-input tiles
    scratch = torch.empty(max(sbytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(i):
        st = B.conv2d_fwd_raw(desc, algo_arg, xs[i % nsets].data_ptr(), w.data_ptr(), wp_ptr, 0,
                              ys[i % nsets].data_ptr(), scratch.data_ptr() if sbytes else 0, sbytes, sptr)
        if st != 0:
            raise RuntimeError(B.library().cfwd_last_error().decode())

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(a.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    per_launch = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kernel_ms = sum(per_launch) / len(per_launch)
    ms_per_step = total_ms / a.steps

    # warm (same buffers every step) secondary figure
    for i in range(3):
        step(0)
    torch.cuda.synchronize()
    wb = torch.cuda.Event(enable_timing=True)
    we = torch.cuda.Event(enable_timing=True)
    wb.record(stream)
    for i in range(a.steps):
        step(0)
    we.record(stream)
    torch.cuda.synchronize()
    warm_ms = wb.elapsed_time(we) / a.steps

    flops = layer_flops(L, N)
    nbytes = layer_bytes(L, N, a.dtype)
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK[a.dtype]
    achieved = flops / (kernel_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,2/fan_in) weights)",
        "config": {
            "workload": "resnet_3x3_256ch_56x56_n32", "n": N, "c": L.c, "k": L.k, "h": L.h, "w": L.w,
            "r": L.r, "s": L.s, "stride": L.stride, "pad": L.pad, "layout": "NCHW",
            "algo": B.algo_name(chosen), "dispatch": "fastrun_map" if a.algo == "auto" else "fixed",
            "rotated_buffer_sets": nsets, "gflop_per_step": round(flops / 1e9, 3),
            "mb_per_step": round(nbytes / 1e6, 2), "warm_ms_per_step": round(warm_ms, 5),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak / 1e12,
            "unit": "TFLOP/s",
            "frac": round(achieved * 1e12 / peak, 4),
            "traffic": None,
            "kernel_avg_ms": round(kernel_ms, 5),
        },
    }

    if not a.no_cpu:
        import oracle
        # bounded sample of the same workload: whole images, as many as the budget allows
        t0 = time.perf_counter()
        oracle.conv2d(pr.x[:1], pr.w, L.stride, L.pad, L.dil, L.groups)
        t1 = time.perf_counter() - t0
        nimg = 1
        if 2 * t1 < a.cpu_budget:
            nimg = max(1, min(N, int(a.cpu_budget / t1) - 1))
            if nimg > 1:
                t0 = time.perf_counter()
                oracle.conv2d(pr.x[:nimg], pr.w, L.stride, L.pad, L.dil, L.groups)
                t1 = time.perf_counter() - t0
        sflops = layer_flops(L, nimg)
        out["cpu_baseline"] = {
            "value": round(sflops / t1 / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": "%d of %d images (%.2f GFLOP, fp64 loop nest, %.1f s)" % (nimg, N, sflops / 1e9, t1),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
