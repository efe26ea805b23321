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
same workload on the host cores.

The line also carries "ceilings": the rate a plain 1 GiB device copy reaches
on the same GPU (the practical ceiling of the streaming layers; per layer,
"frac_of_copy" sets the layer's algorithmic GB/s against it).

Extra figures (each adds a key to the same line):
  --layers    the fused operator on all five workloads (per layer: time, TFLOP/s,
              algorithmic GB/s, the bound and its fraction, and both the
              fraction of the matrix peak and of the HBM peak)
  --unfused   the three-kernel sequence conv -> t1 -> BN -> t2 -> SiLU -> y
              beside the fused call, per workload
  --variants  every variant that supports each workload, and whether the
              automatic dispatch picked the fastest
Progress goes to stderr; stdout carries only the JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_F32_TFLOPS = 157.3    # fp32 MFMA
MALL_BYTES = 256 << 20     # Infinity Cache
METRIC = "fused conv+BN+SiLU TFLOP/s and % of bf16 MFMA or HBM roofline per layer"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "conv_bn_silu_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def roofline_bound(wl) -> str:
    peak_flops = (MFMA_F32_TFLOPS if wl.dtype == 0 else MFMA_BF16_TFLOPS) * 1e12
    return "mfma" if wl.flops / peak_flops > wl.algorithmic_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"


def roofline(wl, seconds: float) -> dict:
    bound = roofline_bound(wl)
    if bound == "hbm":
        achieved, peak, unit = wl.algorithmic_bytes / seconds / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        peak = MFMA_F32_TFLOPS if wl.dtype == 0 else MFMA_BF16_TFLOPS
        achieved, unit = wl.flops / seconds / 1e12, "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4)}


class Layer:
    """Device buffers of one workload: `sets` rotated copies of x and y (so
    consecutive steps do not hit in the Infinity Cache), one w/scale/bias."""

    def __init__(self, key: str, extra_outputs: int = 0):
        import torch
        from conv_bn_silu_amd import synth
        self.wl = wl = synth.WORKLOADS[key]
        inp = synth.make_inputs(wl)
        dev = torch.device("cuda", 0)
        if wl.dtype == synth.DTYPE_BF16:
            x0 = torch.from_numpy(inp.x_bits.view("int16")).view(torch.bfloat16).to(dev)
            self.w = torch.from_numpy(inp.w_bits.view("int16")).view(torch.bfloat16).to(dev)
        else:
            x0 = torch.from_numpy(inp.x).to(dev)
            self.w = torch.from_numpy(inp.w).to(dev)
        self.sc = torch.from_numpy(inp.scale).to(dev)
        self.bi = torch.from_numpy(inp.bias).to(dev)
        per_set = wl.algorithmic_bytes * (1 + extra_outputs)
        self.sets = max(2, math.ceil(2 * MALL_BYTES / per_set))
        self.xs = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        shape = (wl.N, wl.C_out, wl.OH, wl.OW)
        self.ys = [[torch.empty(shape, dtype=x0.dtype, device=dev) for _ in range(1 + extra_outputs)]
                   for _ in range(self.sets)]
        self.geo = (wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad, wl.dtype)


def time_steps(step, steps: int, warmup: int, stream) -> dict:
    """Wall clock over exactly `steps` steps, then HIP events on the launch
    stream: one pair around each launch (per-launch kernel duration) and one
    pair around the whole region."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    issued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for i in range(steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    return {"wall_s": wall, "host_issue_s": issued, "launch_mean_s": sum(durs) / len(durs),
            "launch_median_s": durs[len(durs) // 2],
            "launch_min_s": durs[0], "region_per_step_s": r0.elapsed_time(r1) * 1e-3 / steps}


def measure_fused(key: str, steps: int, warmup: int, variant: str = "auto", layer: Layer | None = None) -> dict:
    import torch
    from conv_bn_silu_amd import binding as B
    L = layer or Layer(key)
    wl = L.wl
    lib = B.default_library()
    v = B.VARIANTS[variant]
    if v == 0:
        v = B.select_variant(*L.geo)
    stream = torch.cuda.current_stream(torch.device("cuda", 0))
    sp = stream.cuda_stream

    # Arguments bound once per buffer set, and the C entry point called
    # directly: at tens of microseconds per launch the Python side must stay
    # well ahead of the GPU, or the timing measures the host.
    fn, handle = B.lib.conv_bn_silu_run_variant, lib.handle
    args = [(handle, v, L.xs[j].data_ptr(), L.w.data_ptr(), L.sc.data_ptr(), L.bi.data_ptr(),
             L.ys[j][0].data_ptr(), *L.geo, sp) for j in range(L.sets)]

    def step(i):
        rc = fn(*args[i % L.sets])
        if rc:
            lib.run_ptr(*args[i % L.sets][1:])  # raises with the status and HIP error

    t = time_steps(step, steps, warmup, stream)
    # Average launch duration: HIP events around the whole back-to-back
    # region on the launch stream, divided by the launch count.  (The
    # per-launch event pairs are reported too; the event packets between
    # launches make them read slightly longer.)
    kern = t["region_per_step_s"]
    return {"key": key, "wl": wl, "variant": B.variant_name(v), "sets": L.sets,
            "ms_per_step": t["wall_s"] / steps * 1e3, "tflops": wl.flops / (t["wall_s"] / steps) / 1e12,
            "kernel_us_mean": kern * 1e6, "host_issue_us_per_step": t["host_issue_s"] / steps * 1e6,
            "launch_events_us_mean": t["launch_mean_s"] * 1e6,
            "launch_events_us_median": t["launch_median_s"] * 1e6,
            "kernel_us_min": t["launch_min_s"] * 1e6, "region_us_per_step": t["region_per_step_s"] * 1e6,
            "roofline": roofline(wl, kern), "hbm_gbs_alg": wl.algorithmic_bytes / kern / 1e9,
            "tflops_kernel": wl.flops / kern / 1e12}


def measure_unfused(key: str, steps: int, warmup: int) -> dict:
    """conv -> t1, BN -> t2, SiLU -> y, all three intermediates in HBM."""
    import torch
    from conv_bn_silu_amd import binding as B
    L = Layer(key, extra_outputs=2)
    lib = B.default_library()
    stream = torch.cuda.current_stream(torch.device("cuda", 0))
    sp = stream.cuda_stream

    fn, handle = B.lib.conv_bn_silu_run_unfused, lib.handle
    args = [(handle, L.xs[j].data_ptr(), L.w.data_ptr(), L.sc.data_ptr(), L.bi.data_ptr(),
             L.ys[j][1].data_ptr(), L.ys[j][2].data_ptr(), L.ys[j][0].data_ptr(), *L.geo, sp)
            for j in range(L.sets)]

    def step(i):
        rc = fn(*args[i % L.sets])
        if rc:
            lib.run_unfused_ptr(*args[i % L.sets][1:])  # raises with the status and HIP error

    t = time_steps(step, steps, warmup, stream)
    return {"us_per_step": t["region_per_step_s"] * 1e6, "wall_us_per_step": t["wall_s"] / steps * 1e6}


def traffic_for(wl) -> dict | None:
    """HBM bytes per launch from the committed rocprofv3 counter record, if it
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_sources_digest") != kernel_sources_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(key: str, min_seconds: float = 12.0, max_reps: int = 200) -> dict:
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
            "sample": f"whole workload {wl.name} ({wl.flops / 1e9:.2f} GFLOP) x{reps}, fp64 conv, BN and "
                      f"SiLU passes, {t_total:.1f} s on {threads} threads"}


def copy_ceiling(mib: int = 1024, reps: int = 20) -> dict:
    """The HBM rate a plain device-to-device copy of `mib` MiB reaches on
    this GPU (read + write bytes over the time of `reps` back-to-back
    copies, HIP events on the copying stream): the practical ceiling for
    the streaming layers, reported beside the 8 TB/s peak."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * n / sec / 1e9, 1), "copy_bytes_each_way": n,
            "what": "torch device-to-device copy, read + write bytes per second"}


def copy_calibration(mib: int, reps: int) -> None:
    """A plain device-to-device copy of a known size, for scaling the HBM
    byte counters (run under rocprofv3 --pmc)."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", help="c1..c5 (default c2, the bf16 1x1 layer)")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--layers", action="store_true", help="also measure all five layers")
    ap.add_argument("--unfused", action="store_true", help="also time the three-kernel sequence per layer")
    ap.add_argument("--variants", action="store_true", help="also time every supporting variant per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration)")
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
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return
    from conv_bn_silu_amd import binding as B, synth
    log(f"[bench] {args.workload} variant {args.variant}: {args.warmup} warmup + {args.steps} steps")
    r = measure_fused(args.workload, args.steps, args.warmup, args.variant)
    wl = r["wl"]
    log(f"[bench] {wl.name}: {r['kernel_us_mean']:.2f} us/launch ({r['variant']})")
    roof = dict(r["roofline"])
    roof["traffic"] = traffic_for(wl)
    out = {
        "metric": METRIC,
        "value": round(r["tflops"], 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == synth.DTYPE_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": wl.N, "C_in": wl.C_in, "H": wl.H, "W": wl.W, "C_out": wl.C_out,
                   "KH": wl.KH, "KW": wl.KW, "stride": wl.stride, "pad": wl.pad, "variant": r["variant"],
                   "rotated_buffer_sets": r["sets"], "kernel_us_mean": round(r["kernel_us_mean"], 3),
                   "host_issue_us_per_step": round(r["host_issue_us_per_step"], 3),
                   "launch_events_us_mean": round(r["launch_events_us_mean"], 3),
                   "launch_events_us_median": round(r["launch_events_us_median"], 3),
                   "algorithmic_bytes": wl.algorithmic_bytes, "flops": wl.flops},
        "roofline": roof,
    }
    ceil = copy_ceiling()
    log(f"[bench] copy ceiling: {ceil['copy_gbs']:.0f} GB/s")
    out["ceilings"] = ceil
    sub_steps = max(20, args.steps // 2)
    if args.layers or args.unfused or args.variants:
        layers = {}
        for key in sorted(synth.WORKLOADS):
            q = r if key == args.workload and args.variant == "auto" else None
            if args.layers or args.unfused:
                q = q or measure_fused(key, sub_steps, args.warmup)
            ent = {}
            if q is not None:
                ent = {"variant": q["variant"], "kernel_us": round(q["kernel_us_mean"], 3),
                       "tflops": round(q["tflops_kernel"], 3),
                       "hbm_gbs_algorithmic": round(q["hbm_gbs_alg"], 1),
                       "bound": q["roofline"]["bound"], "frac": q["roofline"]["frac"],
                       "mfma_frac": round(q["tflops_kernel"] / (MFMA_F32_TFLOPS if q["wl"].dtype == 0
                                                                 else MFMA_BF16_TFLOPS), 4),
                       "hbm_frac": round(q["hbm_gbs_alg"] / HBM_PEAK_GBS, 4),
                       "frac_of_copy": round(q["hbm_gbs_alg"] / ceil["copy_gbs"], 4),
                       "kernel_us_median_launch": round(q["launch_events_us_median"], 3)}
                log(f"[bench] layer {key}: {q['kernel_us_mean']:.2f} us ({q['variant']})")
            if args.unfused:
                u = measure_unfused(key, sub_steps, args.warmup)
                ent["unfused_us_per_step"] = round(u["us_per_step"], 3)
                ent["fused_us_per_step"] = round(q["region_us_per_step"], 3)
                ent["fused_speedup"] = round(u["us_per_step"] / q["region_us_per_step"], 3)
                log(f"[bench] layer {key}: unfused {u['us_per_step']:.2f} us/step")
            if args.variants:
                wlk = synth.WORKLOADS[key]
                geo = (wlk.N, wlk.C_in, wlk.H, wlk.W, wlk.C_out, wlk.KH, wlk.KW, wlk.stride, wlk.pad, wlk.dtype)
                L = Layer(key)
                times = {}
                for name, v in B.VARIANTS.items():
                    if v == 0 or not B.variant_supports(v, *geo):
                        continue
                    # the scalar variant is very slow on the large layers: fewer steps
                    n_st = sub_steps if name != "scalar" else 5
                    times[name] = round(measure_fused(key, n_st, min(args.warmup, 3), name, L)
                                        ["kernel_us_mean"], 3)
                    log(f"[bench] layer {key} variant {name}: {times[name]:.2f} us")
                picked = B.variant_name(B.select_variant(*geo))
                ent["variants_us"] = times
                ent["auto_picks"] = picked
                ent["auto_is_fastest"] = picked == min(times, key=times.get)
                del L
            layers[synth.WORKLOADS[key].name] = ent
        out["layers"] = layers
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
