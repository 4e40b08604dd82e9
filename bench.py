#!/usr/bin/env python3
"""Benchmark of the forward-convolution library on one GPU.

One step = one forward pass of every conv layer of the chosen workload over
one batch, each layer dispatched through the C ABI.  The default workload is
the ResNet 3x3 256-channel layer at 56x56 (N=32, C=K=256, stride 1, pad 1,
bf16 in / fp32 accumulate / bf16 out, NCHW).  With ``--algo auto`` (the
default) the Fast-Run selection phase runs once per layer during set-up
(untimed) and every timed step dispatches from the Fast-Run map (execution
phase), with filters prepared once, as inference does with constant weights.

Inputs are seeded synthetic data (the distributions of each workload, drawn
by ``cnn_convolution_fwd_amd.workloads``) already resident in HBM; the timed
loop rotates over enough input/output buffer sets (> 512 MB, twice the 256 MB
Infinity Cache) that no step reads its input from the cache a previous step
filled.

Before the W warm-up steps, the same launches run untimed for about a third of
a second (at least ``--settle`` seconds), so that the timed steps see the
clock the GPU holds under sustained load rather than one still ramping up
from idle (this matters for a fixed ``--algo``, where no Fast-Run search has
run first).

Prints ONE JSON line: whole-step throughput (direct-equivalent FLOPs), the
roofline of the dominant kernel (HIP events around every launch, on the
stream the kernel runs on; FLOPs its algorithm performs, so Winograd is held
to its own element-wise products), the filter prepare time (once per layer,
outside the step), the shader clock and board power sampled while the same
steps run, and the CPU oracle timed on a bounded sample of the same workload
(threads used, host CPU model).

    python bench.py [--workload NAME] [--n N] [--dtype bf16|f32|i8] [--algo auto|family[/cfg]]
                    [--steps K] [--warmup W] [--layers I,J] [--fastrun-load F] [--fastrun-save F]
    python bench.py --copy-calibration    # plain 1 GiB device copy, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "conv TFLOP/s (int8 TOP/s) + % MFMA/HBM roofline, ResNet 3x3 256ch@56x56"

# name -> (benchmark configuration, layer indices, dtypes (first = default))
WORKLOADS = {
    "resnet_3x3_256ch_56x56": (3, [0], ("bf16", "f32")),
    "single_conv_16to32_32x32": (1, [0], ("f32",)),
    "mobilenet_stem_dw_pw": (2, [0, 1, 2], ("f32", "bf16")),
    "mobilenet_stem3x3s2_3to32_224": (2, [0], ("f32", "bf16")),
    "mobilenet_dw3x3_32ch_112": (2, [1], ("f32", "bf16")),
    "mobilenet_pw1x1_32to64_112": (2, [2], ("f32", "bf16")),
    "bottleneck_1x1_3x3_1x1_56x56": (4, [0, 1, 2], ("bf16",)),
    "plain_3x3_256_56x56": (4, [3], ("bf16",)),
    "resnet18_int8_nchw4": (5, list(range(20)), ("i8",)),
}
ALIASES = {
    "resnet3x3": "resnet_3x3_256ch_56x56", "single": "single_conv_16to32_32x32",
    "mobilenet": "mobilenet_stem_dw_pw", "stem": "mobilenet_stem3x3s2_3to32_224",
    "depthwise": "mobilenet_dw3x3_32ch_112", "pointwise": "mobilenet_pw1x1_32to64_112",
    "bottleneck": "bottleneck_1x1_3x3_1x1_56x56", "plain": "plain_3x3_256_56x56",
    "resnet18_int8": "resnet18_int8_nchw4",
}
# (config, layer) pairs whose output takes the skip connection: the second
# 3x3 of each ResNet-18 basic block, the bottleneck's expanding 1x1
RESIDUAL_LAYERS = {(5, 2), (5, 4), (5, 9), (5, 14), (5, 19), (4, 2)}
ROTATE_BYTES = 512 * 2**20
MAX_SETS = 256


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="resnet3x3", help="one of %s" % ", ".join(list(ALIASES) + list(WORKLOADS)))
    ap.add_argument("--n", type=int, default=0, help="batch size (0: the workload's own)")
    ap.add_argument("--dtype", default="", choices=["", "bf16", "f32", "i8"])
    ap.add_argument("--algo", default="auto", help="auto (Fast-Run) or family[/config], e.g. implicit_gemm/7")
    ap.add_argument("--settle", type=float, default=0.3, help="seconds of untimed launches before the warm-up steps")
    ap.add_argument("--sets", type=int, default=0, help="rotated buffer sets (0: enough for > 512 MB)")
    ap.add_argument("--telemetry-window", type=float, default=0.5,
                    help="seconds of further untimed steps while clock and power are sampled")
    ap.add_argument("--epilogue", default="none", choices=["none", "fused", "unfused"],
                    help="bias + ReLU after every layer (plus the residual on ResNet block-closing layers): fused "
                         "into the convolution, or as separate elementwise passes after it")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle CPU work at most")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--layers", default="", help="comma-separated layer indices of the workload to run (default: all)")
    ap.add_argument("--fastrun-load", default="", help="Fast-Run map file to load before set-up (its problems are not "
                    "searched again)")
    ap.add_argument("--fastrun-save", default="", help="write the Fast-Run map to this file after set-up")
    ap.add_argument("--layout", default="", choices=["", "nhwc"],
                    help="float workloads: run the layers on NHWC activations (the NHWC implicit GEMM)")
    ap.add_argument("--block", default="layers", choices=["layers", "fused"],
                    help="bottleneck workload: its three layers one by one, or the fused block kernel")
    ap.add_argument("--allow-inexact-int8", action="store_true",
                    help="let Fast-Run time int8 Winograd F(2x2) (outputs within 1 of the exact ones)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device copy of 1 GiB instead (scales HBM byte counters)")
    return ap.parse_args()


def sources_digest(names) -> str:
    """sha256 (16 hex digits) over the named kernel source files, in the given order."""
    d = os.path.join(ROOT, "cnn_convolution_fwd_amd", "csrc")
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, dtype: str, algo: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when there is none, when it was taken for another
    algorithm, or when the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (workload, dtype))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
    try:
        if kv.get("algo") != algo or kv["sources_sha256"] != sources_digest(kv["sources"].split()):
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, OSError, ValueError):
        return None


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    nbytes = 2**30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": round(ms, 4),
                      "gb_per_s": round(2 * nbytes / ms / 1e6, 1)}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (images are independent, so the "
              "path would shard along the batch with replicated weights and no collective); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.copy_calibration:
        copy_calibration()
        return

    from cnn_convolution_fwd_amd import binding as B
    from cnn_convolution_fwd_amd import telemetry
    from cnn_convolution_fwd_amd.roofline import (PEAK, block_algo_flops, block_bytes, block_flops, bound,
                                                   layer_algo_flops, layer_bytes, layer_flops)
    from cnn_convolution_fwd_amd.workloads import (CONFIGS, bf16_bits, epilogue_inputs, float_problem, int8_problem, to_nhwc,
                                                    pack_nchwx)

    base = ALIASES.get(a.workload, a.workload)
    if base not in WORKLOADS:
        print("unknown workload %s" % a.workload, file=sys.stderr)
        sys.exit(2)
    cfg_idx, layer_ids, dtypes = WORKLOADS[base]
    if a.layers:
        pick = [int(v) for v in a.layers.split(",")]
        if not pick or any(li not in layer_ids for li in pick):
            print("workload %s has layers %s" % (base, layer_ids), file=sys.stderr)
            sys.exit(2)
        layer_ids = pick
    cfg = CONFIGS[cfg_idx]
    dtype = a.dtype or dtypes[0]
    if dtype not in dtypes:
        print("workload %s runs in %s" % (base, "/".join(dtypes)), file=sys.stderr)
        sys.exit(2)
    if a.block == "fused" and (base != "bottleneck_1x1_3x3_1x1_56x56" or a.layers or a.epilogue == "unfused"):
        print("--block fused runs the whole bottleneck workload (no --layers, epilogue none or fused)",
              file=sys.stderr)
        sys.exit(2)
    if a.epilogue == "unfused" and dtype == "i8":
        print("an unfused int8 epilogue would need the int32 accumulators; use --epilogue fused", file=sys.stderr)
        sys.exit(2)
    N = a.n or cfg.n
    workload = "%s_n%d" % (base, N) + ("_layers%s" % "-".join(str(li) for li in layer_ids) if a.layers else "")
    dev = torch.device("cuda:0")
    int8 = dtype == "i8"
    layout = "NCHWX" if int8 else "NCHW"
    if a.layout == "nhwc":
        if int8 or a.block == "fused":
            print("--layout nhwc runs float layers (fp32 / bf16) one by one", file=sys.stderr)
            sys.exit(2)
        layout = "NHWC"
        workload += "_nhwc"
    act = to_nhwc if layout == "NHWC" else (lambda v: v)

    def to_dev(arr):
        if dtype == "bf16":
            return torch.from_numpy(bf16_bits(arr).view(np.int16)).to(dev).view(torch.bfloat16)
        if int8:
            return torch.from_numpy(np.ascontiguousarray(arr, np.int8)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)

    if a.fastrun_load:
        B.fastrun_load(a.fastrun_load)
    if a.allow_inexact_int8:
        B.fastrun_allow_inexact_int8(True)
    # ---- per-layer set-up: inputs, algorithm (Fast-Run), prepared filter, scratch.
    # LayerPlan is the same sequence of library calls the parity tests run.
    layers = []
    if a.block == "fused":
        # the three layers as one fused block: x and weights drawn as each
        # layer's standalone problem, the epilogues those layers would take
        prs = [float_problem(cfg_idx, li, n=N, dtype=dtype) for li in layer_ids]
        Ls = [cfg.layers[li] for li in layer_ids]
        x0 = to_dev(prs[0].x)
        w1, w2, w3 = (to_dev(p.w) for p in prs)
        desc = B.bottleneck_desc_for(x0, w1, w3)
        B.bottleneck_check(desc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        w2p = B.bottleneck_prepare(w2, desc)
        e1.record()
        torch.cuda.synchronize()
        biases, relus, res0 = [None] * 3, [False] * 3, None
        if a.epilogue == "fused":
            for j, (li, L) in enumerate(zip(layer_ids, Ls)):
                epi = epilogue_inputs((N, L.k, L.h, L.w), dtype, 7000 + li)
                biases[j] = torch.from_numpy(epi.bias).to(dev)
                relus[j] = True
                if (cfg_idx, li) in RESIDUAL_LAYERS:
                    res0 = to_dev(epi.residual)
        blk = dict(block=True, Ls=Ls, prs=prs, x0=x0, w=(w1, w2p, w3), desc=desc, biases=biases, relus=relus,
                   res0=res0, y0=torch.empty((N, Ls[2].k, Ls[2].h, Ls[2].w), dtype=x0.dtype, device=dev),
                   prepare_ms=e0.elapsed_time(e1))
        layers.append(blk)
    for li in (layer_ids if a.block == "layers" else []):
        L = cfg.layers[li]
        if int8:
            pr = int8_problem(cfg_idx, li, n=N)
            x0 = to_dev(pack_nchwx(pr.x, cfg.x_block))
            scale = torch.from_numpy(pr.scale).to(dev)
        else:
            pr = float_problem(cfg_idx, li, n=N, dtype=dtype)
            x0 = to_dev(act(pr.x))
            scale = None
        w = to_dev(pr.w)
        # epilogue of this layer: bias, ReLU (not on downsample shortcuts), and
        # the skip connection on the layers that close a residual block
        bias = res0 = None
        relu = False
        if a.epilogue != "none":
            oh, ow = L.out_hw()
            epi = epilogue_inputs((N, L.k, oh, ow), dtype, 7000 + li)
            bias = torch.from_numpy(epi.bias).to(dev)
            relu = "down" not in L.name
            if (cfg_idx, li) in RESIDUAL_LAYERS:
                res0 = to_dev(pack_nchwx(epi.residual, cfg.x_block) if int8 else act(epi.residual))
        fused = a.epilogue == "fused"
        plan = B.LayerPlan(x0, w, L.stride, L.pad, L.dil, L.groups, layout, channels=L.c, requant_scale=scale,
                           algo_spec=a.algo, bias=bias if fused else None, relu=relu and fused)
        layers.append(dict(L=L, pr=pr, x0=x0, y0=plan.new_output(), plan=plan, bias=bias, res0=res0, relu=relu))

    if a.fastrun_save:
        B.fastrun_save(a.fastrun_save)

    # every layer rotates over its own buffer sets, > 512 MB per layer, so a
    # layer timed alone (per-kernel figures) cannot read from the cache either
    for l in layers:
        set_bytes = l["x0"].numel() * l["x0"].element_size() + l["y0"].numel() * l["y0"].element_size()
        ns = a.sets or min(MAX_SETS, max(2, -(-ROTATE_BYTES // set_bytes) + 1))
        l["nsets"] = ns
        l["xs"] = [l["x0"]] + [l["x0"].clone() for _ in range(ns - 1)]
        l["ys"] = [l["y0"]] + [torch.empty_like(l["y0"]) for _ in range(ns - 1)]
        l["rs"] = None if l["res0"] is None else [l["res0"]] + [l["res0"].clone() for _ in range(ns - 1)]
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def launch(l, i):
        ns = l["nsets"]
        y = l["ys"][i % ns]
        res = l["rs"][i % ns] if l["rs"] is not None else None
        fused = a.epilogue == "fused"
        if l.get("block"):
            w1, w2p, w3 = l["w"]
            ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
            r = l["relus"]
            ep = B.BottleneckEpilogue(*(ptr(b) for b in l["biases"]), ptr(res), int(r[0]), int(r[1]), int(r[2]))
            st = B.bottleneck_fwd_raw(l["desc"], l["xs"][i % ns].data_ptr(), w1.data_ptr(), w2p.data_ptr(),
                                      w3.data_ptr(), ep, y.data_ptr(), sptr)
            if st != 0:
                raise RuntimeError(B.library().cfwd_last_error().decode())
            return
        st = l["plan"].launch_raw(l["xs"][i % ns].data_ptr(), y.data_ptr(), sptr,
                                  res.data_ptr() if (fused and res is not None) else 0)
        if st != 0:
            raise RuntimeError(B.library().cfwd_last_error().decode())
        if a.epilogue == "unfused":  # the same epilogue as elementwise passes over y
            y.add_(l["bias"].view((1, 1, 1, -1) if layout == "NHWC" else (1, -1, 1, 1)).to(y.dtype))
            if res is not None:
                y.add_(res)
            if l["relu"]:
                y.relu_()

    sampler = telemetry.Sampler(torch.cuda.current_device())
    t_end = time.perf_counter() + a.settle
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            for l in layers:
                launch(l, i)
            i += 1
        torch.cuda.synchronize()
    for i in range(a.warmup):
        for l in layers:
            launch(l, i)
    torch.cuda.synchronize()

    nl = len(layers)

    def timed(fn, reps):
        """ms per rep of ``fn(i)`` over ``reps`` reps, bracketed by one event pair on the stream."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the timed region: whole steps (every layer), nothing else on the stream
    ms_per_step = timed(lambda i: [launch(l, i) for l in layers], a.steps)
    # per-kernel durations: each layer's launches back to back, same rotation
    if nl == 1:
        layer_avg = [ms_per_step]
    else:
        layer_avg = [timed(lambda i, l=l: launch(l, i), a.steps) for l in layers]

    # clock and power under the same load: keep launching whole steps for a
    # while after the timed region, sampled only while those launches run
    sampler.start()
    t_end = time.perf_counter() + a.telemetry_window
    i = 0
    batch = max(8, int(20.0 / max(ms_per_step, 1e-3)))  # ~20 ms of steps between synchronisations
    while time.perf_counter() < t_end:
        for _ in range(batch):
            for l in layers:
                launch(l, i)
            i += 1
        torch.cuda.synchronize()
    gpu_telemetry = sampler.stop()

    # warm (same buffers every step) secondary figure
    for _ in range(3):
        for l in layers:
            launch(l, 0)
    warm_ms = timed(lambda i: [launch(l, 0) for l in layers], a.steps)

    peak_key = "i8" if int8 else dtype
    unit = "TOP/s" if int8 else "TFLOP/s"
    total_flops = 0
    per_layer = []
    for l, t in zip(layers, layer_avg):
        if l.get("block"):
            L1, L3 = l["Ls"][0], l["Ls"][2]
            dims = (N, L1.c, L1.h, L1.w, L1.k, L3.k)
            L = type(L1)("bottleneck_block", L1.c, L3.k, L1.h, L1.w, 1, 1, 1, 0, 1, 1)
            name = "bottleneck_fused"
            fl, afl = block_flops(*dims), block_algo_flops(*dims)
            by = block_bytes(*dims, 2)
            l["plan"] = type("P", (), {"name": name, "prepare_ms": l["prepare_ms"]})()
        else:
            L = l["L"]
            name = l["plan"].name
            fl = layer_flops(L, N)               # direct-equivalent (the metric)
            afl = layer_algo_flops(L, N, name)   # what the chosen algorithm performs
            by = layer_bytes(L, N, dtype)
        kind, _ = bound(afl, by, peak_key)
        total_flops += fl
        if kind == "hbm":
            ach, pk, u = by / (t * 1e-3) / 1e9, PEAK["hbm_bytes_per_s"] / 1e9, "GB/s"
        else:
            ach, pk, u = afl / (t * 1e-3) / 1e12, PEAK[peak_key] / 1e12, unit
        per_layer.append(dict(name=L.name, algo=name, ms=round(t, 5), bound=kind, achieved=round(ach, 2), peak=pk,
                              unit=u, frac=round(ach / pk, 4), flops=fl, algo_flops=afl, bytes=by,
                              prepare_ms=round(l["plan"].prepare_ms, 5)))
    dom = max(range(nl), key=lambda j: layer_avg[j])
    d = per_layer[dom]
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded draws with each workload's distributions; no dataset, no trained weights)",
        "config": {
            "workload": workload, "n": N, "layers": nl, "layout": layout,
            "algo": "+".join(sorted({p["algo"] for p in per_layer})),
            "dispatch": "fastrun_map" if a.algo == "auto" else "fixed",
            "fastrun_map_loaded": os.path.basename(a.fastrun_load) or None,
            "inexact_int8_allowed": bool(a.allow_inexact_int8), "rotated_buffer_sets": max(l["nsets"] for l in layers),
            "gflop_per_step": round(total_flops / 1e9, 3),
            "mb_per_step": round(sum(p["bytes"] for p in per_layer) / 1e6, 2),
            "warm_ms_per_step": round(warm_ms, 5),
            "filter_prepare_ms": round(sum(p["prepare_ms"] for p in per_layer), 5),
            "epilogue": a.epilogue,
            "block": a.block,
        },
        "gpu_telemetry": gpu_telemetry,
        "roofline": {
            "bound": d["bound"],
            "achieved": d["achieved"],
            "peak": d["peak"],
            "unit": d["unit"],
            "frac": d["frac"],
            "traffic": stored_traffic(workload, dtype, d["algo"]),
            "kernel": "%s (%s)" % (d["name"], d["algo"]),
            "kernel_avg_ms": d["ms"],
            "algorithmic_bytes": d["bytes"],
            "algorithmic_flops": d["algo_flops"],
            "direct_equivalent_flops": d["flops"],
        },
    }
    if nl > 1:
        out["layers"] = [{k: p[k] for k in ("name", "algo", "ms", "bound", "achieved", "unit", "frac", "prepare_ms")}
                         for p in per_layer]

    if not a.no_cpu:
        import oracle

        def run_oracle(nimg):
            t0 = time.perf_counter()
            for l in layers:
                if l.get("block"):
                    p0, p1, p2 = l["prs"]
                    oracle.bottleneck(p0.x[:nimg], p0.w, p1.w, p2.w)
                    continue
                L, pr = l["L"], l["pr"]
                if int8:
                    oracle.conv2d_int8_requant(pr.x[:nimg], pr.w, pr.scale, L.stride, L.pad, L.dil, L.groups)
                else:
                    oracle.conv2d(pr.x[:nimg], pr.w, L.stride, L.pad, L.dil, L.groups)
            return time.perf_counter() - t0

        # bounded sample of the same workload: whole images through every layer of the step
        nimg = 1
        t1 = run_oracle(1)
        if 2 * t1 < a.cpu_budget:
            nimg = max(1, min(N, int(a.cpu_budget / t1) - 1))
            if nimg > 1:
                t1 = run_oracle(nimg)
        sflops = sum(block_flops(nimg, l["Ls"][0].c, l["Ls"][0].h, l["Ls"][0].w, l["Ls"][0].k, l["Ls"][2].k)
                     if l.get("block") else layer_flops(l["L"], nimg) for l in layers)
        out["cpu_baseline"] = {
            "value": round(sflops / t1 / 1e12, 6),
            "unit": unit,
            "cores": oracle.max_threads(),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": telemetry.cpu_model(),
            "kind": "oracle",
            "sample": "%d of %d images through %d layer(s) (%.2f G%s, %s loop nest, %.1f s)" % (
                nimg, N, nl, sflops / 1e9, "OP" if int8 else "FLOP", "int64" if int8 else "fp64", t1),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
