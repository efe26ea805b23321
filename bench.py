#!/usr/bin/env python3
"""Benchmark of the fused conv2d + folded BN + SiLU operator on one MI355X.

One step = one fused call over the whole layer (one batch of seeded synthetic
input, already resident in HBM).  The headline workload is the bf16 1x1
pointwise layer (N=8, 256 -> 256 channels, 80x80); ``--workload`` picks
another of the five.  Input/output buffer sets are rotated so that the
working set of consecutive steps exceeds twice the 256 MB Infinity Cache and
every step streams from HBM.

Prints ONE JSON line with the metric (TFLOP/s), the roofline of the dominant
kernel measured with HIP events on the stream the kernel runs on, the HBM
traffic counted by rocprofv3 (when the committed counter record matches the
current kernel sources), and the CPU oracle timed on a bounded sample of the
same workload on the host cores.  ``--layers`` adds the same per-layer
figures for all five workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_F32_TFLOPS = 157.3    # fp32 MFMA
MALL_BYTES = 256 << 20     # Infinity Cache


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "conv_bn_silu_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def roofline_bound(wl) -> str:
    peak_flops = (MFMA_F32_TFLOPS if wl.dtype == 0 else MFMA_BF16_TFLOPS) * 1e12
    return "mfma" if wl.flops / peak_flops > wl.algorithmic_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"


def measure_layer(key: str, steps: int, warmup: int, variant: str = "auto") -> dict:
    import torch
    from conv_bn_silu_amd import binding as B, synth
    wl = synth.WORKLOADS[key]
    inp = synth.make_inputs(wl)
    dev = torch.device("cuda", 0)
    if wl.dtype == synth.DTYPE_BF16:
        x0 = torch.from_numpy(inp.x_bits.view("int16")).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(inp.w_bits.view("int16")).view(torch.bfloat16).to(dev)
    else:
        x0 = torch.from_numpy(inp.x).to(dev)
        w = torch.from_numpy(inp.w).to(dev)
    sc = torch.from_numpy(inp.scale).to(dev)
    bi = torch.from_numpy(inp.bias).to(dev)
    per_set = wl.algorithmic_bytes
    sets = max(2, math.ceil(2 * MALL_BYTES / per_set))
    xs = [x0] + [x0.clone() for _ in range(sets - 1)]
    ys = [torch.empty((wl.N, wl.C_out, wl.OH, wl.OW), dtype=x0.dtype, device=dev) for _ in range(sets)]
    lib = B.default_library()
    v = B.VARIANTS[variant]
    if v == 0:
        v = B.select_variant(wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad, wl.dtype)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    geo = (wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad, wl.dtype)

    def step(i):
        lib.run_ptr(v, xs[i % sets].data_ptr(), w.data_ptr(), sc.data_ptr(), bi.data_ptr(),
                    ys[i % sets].data_ptr(), *geo, sp)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Whole-job wall clock over exactly `steps` steps.
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-launch kernel duration: HIP events recorded on the launch stream
    # around each launch.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    kern = sum(durs) / len(durs)
    bound = roofline_bound(wl)
    if bound == "hbm":
        achieved, peak, unit = wl.algorithmic_bytes / kern / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        peak = MFMA_F32_TFLOPS if wl.dtype == 0 else MFMA_BF16_TFLOPS
        achieved, unit = wl.flops / kern / 1e12, "TFLOP/s"
    return {
        "key": key, "wl": wl, "variant": B.variant_name(v), "sets": sets,
        "ms_per_step": wall / steps * 1e3, "tflops": wl.flops / (wall / steps) / 1e12,
        "kernel_us_mean": kern * 1e6, "kernel_us_median": durs[len(durs) // 2] * 1e6,
        "kernel_us_min": durs[0] * 1e6,
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4)},
        "hbm_gbs_alg": wl.algorithmic_bytes / kern / 1e9,
        "tflops_kernel": wl.flops / kern / 1e12,
    }


def traffic_for(key: str, wl) -> dict | None:
    """HBM bytes per launch from the committed rocprofv3 counter record, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_digest") != kernel_sources_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(key: str, min_seconds: float = 10.0, max_reps: int = 5) -> dict:
    """The oracle (unfused fp64 three-pass sequence, as it stands) on the host
    cores, over the whole workload, repeated until ~min_seconds have passed."""
    import oracle
    from conv_bn_silu_amd import synth
    wl = synth.WORKLOADS[key]
    inp = synth.make_inputs(wl)
    o = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1
    reps, t_total = 0, 0.0
    while reps < max_reps and (reps == 0 or t_total < min_seconds):
        t0 = time.perf_counter()
        o.forward(inp.x, inp.w, inp.scale, inp.bias, wl.stride, wl.pad, nthreads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": round(wl.flops * reps / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole workload {wl.name} ({wl.flops / 1e9:.2f} GFLOP) x{reps}, fp64 three passes, "
                      f"{t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", help="c1..c5 (default c2, the bf16 1x1 layer)")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--layers", action="store_true", help="also measure all five layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this operator's path has no multi-GPU part "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    if not os.path.exists(os.path.join(ROOT, "conv_bn_silu_amd", "libconv_bn_silu.so")):
        from conv_bn_silu_amd import build as _b
        _b.build()
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    from conv_bn_silu_amd import synth
    r = measure_layer(args.workload, args.steps, args.warmup, args.variant)
    wl = r["wl"]
    roof = dict(r["roofline"])
    roof["traffic"] = traffic_for(args.workload, wl)
    out = {
        "metric": "fused conv+BN+SiLU TFLOP/s and % of bf16 MFMA or HBM roofline per layer",
        "value": round(r["tflops"], 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == synth.DTYPE_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": wl.N, "C_in": wl.C_in, "H": wl.H, "W": wl.W, "C_out": wl.C_out,
                   "KH": wl.KH, "KW": wl.KW, "stride": wl.stride, "pad": wl.pad, "variant": r["variant"],
                   "rotated_buffer_sets": r["sets"], "kernel_us_mean": round(r["kernel_us_mean"], 3),
                   "kernel_us_median": round(r["kernel_us_median"], 3),
                   "algorithmic_bytes": wl.algorithmic_bytes, "flops": wl.flops},
        "roofline": roof,
    }
    if args.layers:
        layers = {}
        for key in sorted(synth.WORKLOADS):
            q = r if key == args.workload else measure_layer(key, max(20, args.steps // 2), args.warmup)
            layers[q["wl"].name] = {"variant": q["variant"], "kernel_us": round(q["kernel_us_mean"], 3),
                                    "tflops": round(q["tflops_kernel"], 3),
                                    "hbm_gbs_algorithmic": round(q["hbm_gbs_alg"], 1),
                                    "bound": q["roofline"]["bound"], "frac": q["roofline"]["frac"]}
        out["layers"] = layers
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
