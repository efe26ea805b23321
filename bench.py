#!/usr/bin/env python3
"""Benchmark of the fused conv2d + folded BN + SiLU operator on one MI355X.

One step = one fused call over a whole layer (one batch of seeded synthetic
input, already resident in HBM).  The headline is the compute-bound deep 3x3
layer (bf16, N=64, 512 -> 512 channels, 20x20), the layer the metric's
"% of bf16 MFMA" is about; every run also measures the other four layers and
reports them under "layers".  Input/output buffer sets are rotated so that
the working set of consecutive steps exceeds twice the 256 MB Infinity Cache
and every step streams from HBM.

Timing: the layer's own step repeated untimed for at least --settle-ms (the
GPU's clocks ramp up over the first tens of milliseconds of load; without
this the first layer of a short run measures the ramp), then W untimed
warm-up steps, then exactly K steps in one timed region, bracketed by
torch.cuda.synchronize() on both sides, with a HIP event pair on the launch
stream around the same K launches.  value and ms_per_step come
from the wall clock of that region; the roofline's "achieved" from the event
pair (the kernel's average launch duration), so the kernel time per step is
never above ms_per_step.

Prints ONE JSON line: the metric (TFLOP/s), the roofline of the dominant
kernel, the HBM traffic counted by rocprofv3 (when the committed counter
record matches the current kernel source), the measured ceilings (a
register-only MFMA loop and a streaming copy, both our own kernels), each
layer's figures with the unfused three-kernel sequence beside it (and, for
the HBM-bound layers, the copy kernel moving the same number of bytes), and
the CPU oracle timed on a bounded sample on the host cores.

Flags:
  --workload KEY  headline layer (default c5)
  --only          only the headline layer (no layers, ceilings or CPU
                  baseline): for profiling runs
  --variants      also time every variant that supports each layer and a
                  sweep of shapes on both sides of each dispatch threshold;
                  exits with status 3 if the automatic choice is more than 5%
                  slower than the fastest variant on any of them
Progress goes to stderr; stdout carries only the JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_F32_TFLOPS = 157.3    # fp32 MFMA
MALL_BYTES = 256 << 20     # Infinity Cache
METRIC = "fused conv+BN+SiLU TFLOP/s and % of bf16 MFMA or HBM roofline per layer"
HEADLINE = "c5"
DISPATCH_SLACK = 1.05      # AUTO may be at most 5% slower than the fastest variant

# The kernel source each variant runs (plus the shared device headers): a
# counter record stays valid while these files are unchanged.
VARIANT_SOURCES = {
    "gemm_gather": "k_gather.hip", "gemm_window": "k_window.hip", "pointwise": "k_pointwise.hip",
    "small_k": "k_stem.hip", "scalar": "k_scalar.hip", "gemm_window32": "k_window32.hip",
    "strided_rows": "k_rows.hip",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_digest(variant: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "conv_bn_silu_amd", "csrc")
    for name in (VARIANT_SOURCES[variant], "cbs_device.h", "cbs_shape.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
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
    consecutive steps do not hit in the Infinity Cache), one w/scale/bias.
    `extra_outputs` more output-sized buffers per set (t1, t2 of the
    unfused sequence)."""

    def __init__(self, wl, extra_outputs: int = 0):
        import torch
        from conv_bn_silu_amd import synth
        self.wl = wl
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
        per_set = wl.algorithmic_bytes + extra_outputs * wl.N * wl.C_out * wl.OH * wl.OW * wl.elem_bytes
        self.sets = max(2, math.ceil(2 * MALL_BYTES / per_set))
        self.xs = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        shape = (wl.N, wl.C_out, wl.OH, wl.OW)
        self.ys = [[torch.empty(shape, dtype=x0.dtype, device=dev) for _ in range(1 + extra_outputs)]
                   for _ in range(self.sets)]
        self.geo = (wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad, wl.dtype)


SETTLE_S = 0.3


def timed_region(step, steps: int, warmup: int, stream) -> dict:
    """The step repeated untimed for SETTLE_S seconds, W warm-up steps, then
    exactly `steps` steps in one region bracketed by device synchronisation,
    with a HIP event pair on the launch stream around the same launches."""
    import torch
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(32):  # batches keep the GPU loaded without a deep queue
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    issued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"wall_s": wall, "events_s": e0.elapsed_time(e1) * 1e-3, "host_issue_s": issued}


def measure_fused(wl, steps: int, warmup: int, variant: str = "auto", layer: Layer | None = None) -> dict:
    import torch
    from conv_bn_silu_amd import binding as B
    L = layer or Layer(wl)
    lib = B.default_library()
    v = B.VARIANTS[variant]
    if v == 0:
        v = B.select_variant(*L.geo)
    stream = torch.cuda.current_stream(torch.device("cuda", 0))
    sp = stream.cuda_stream
    # Arguments bound once per buffer set, and the C entry point called
    # directly: at tens of microseconds per launch the Python side must stay
    # ahead of the GPU, or the timing measures the host.
    fn, handle = B.lib.conv_bn_silu_run_variant, lib.handle
    args = [(handle, v, L.xs[j].data_ptr(), L.w.data_ptr(), L.sc.data_ptr(), L.bi.data_ptr(),
             L.ys[j][0].data_ptr(), *L.geo, sp) for j in range(L.sets)]

    def step(i):
        rc = fn(*args[i % L.sets])
        if rc:
            lib.run_ptr(*args[i % L.sets][1:])  # raises with the status and HIP error

    t = timed_region(step, steps, warmup, stream)
    kern = t["events_s"] / steps
    return {"wl": wl, "variant": B.variant_name(v), "sets": L.sets, "steps": steps,
            "wall_per_step_s": t["wall_s"] / steps, "kernel_s": kern,
            "host_issue_us_per_step": t["host_issue_s"] / steps * 1e6,
            "roofline": roofline(wl, kern), "tflops_kernel": wl.flops / kern / 1e12,
            "tflops_wall": wl.flops / (t["wall_s"] / steps) / 1e12,
            "hbm_gbs_alg": wl.algorithmic_bytes / kern / 1e9}


GRAPH_SETS = 32


def measure_graph(wl, reps: int = 20, layer: Layer | None = None) -> dict:
    """The fused call on up to GRAPH_SETS buffer sets captured once in a HIP
    graph (torch.cuda.CUDAGraph) and the graph replayed `reps` times between
    a HIP event pair: the time per launch without the host issuing each
    launch (which bounds the smallest layer when launches are issued one at
    a time).  Returns {"us_per_launch": None, "error": ...} if capture fails."""
    import torch
    from conv_bn_silu_amd import binding as B
    L = layer or Layer(wl)
    lib = B.default_library()
    v = B.select_variant(*L.geo)
    k = min(L.sets, GRAPH_SETS)
    fn, handle = B.lib.conv_bn_silu_run_variant, lib.handle

    def calls(sp):
        for j in range(k):
            rc = fn(handle, v, L.xs[j].data_ptr(), L.w.data_ptr(), L.sc.data_ptr(), L.bi.data_ptr(),
                    L.ys[j][0].data_ptr(), *L.geo, sp)
            if rc:
                raise RuntimeError(f"conv_bn_silu_run_variant returned {rc}")

    try:
        cur = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            calls(side.cuda_stream)
        cur.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls(torch.cuda.current_stream().cuda_stream)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(reps):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * k)
        del g
        return {"us_per_launch": round(us, 3), "launches_per_graph": k, "replays": reps}
    except Exception as exc:  # the line is still printed; the failure is reported in it
        torch.cuda.synchronize()
        return {"us_per_launch": None, "error": f"{type(exc).__name__}: {exc}"}


def measure_unfused(wl, steps: int, warmup: int) -> dict:
    """conv -> t1, BN -> t2, SiLU -> y, the intermediates in HBM."""
    import torch
    from conv_bn_silu_amd import binding as B
    L = Layer(wl, extra_outputs=2)
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
            lib.run_unfused_ptr(*args[i % L.sets][1:])

    t = timed_region(step, steps, warmup, stream)
    return {"us_per_step": t["events_s"] / steps * 1e6}


def traffic_for(wl, variant: str) -> dict | None:
    """HBM bytes per launch from the committed rocprofv3 counter record, if it
    was taken on the current source of the variant's kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("variant") != variant or rec.get("kernel_sources_digest") != kernel_sources_digest(variant):
        return None
    return rec


def device_info() -> dict:
    import ctypes
    from conv_bn_silu_amd import binding as B
    cu, clk, mclk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = B.lib.conv_bn_silu_bench_device_info(ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(mclk))
    if rc:
        return {}
    return {"num_cu": cu.value, "peak_clock_mhz": clk.value / 1000, "mem_clock_mhz": mclk.value / 1000}


def mfma_ceiling(num_cu: int, iters: int = 20000) -> dict:
    """Our register-only MFMA loop (k_ceiling.hip) on every compute unit:
    the matrix-core rate this GPU sustains, beside the 2.5 PFLOP/s peak."""
    import torch
    from conv_bn_silu_amd import binding as B
    n_wg = 2 * num_cu  # two workgroups (eight waves) per compute unit
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for _ in range(2):
        assert B.lib.conv_bn_silu_bench_mfma(n_wg, iters // 10, sink.data_ptr(), sp) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    assert B.lib.conv_bn_silu_bench_mfma(n_wg, iters, sink.data_ptr(), sp) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    flops = B.lib.conv_bn_silu_bench_mfma_flops(n_wg, iters)
    return {"mfma_bf16_tflops": round(flops / sec / 1e12, 1), "mfma_seconds": round(sec, 6),
            "mfma_what": f"v_mfma_f32_32x32x16_bf16 on registers, {n_wg} workgroups x 4 waves x {iters} x 8"}


def copy_ceiling(mib: int = 1024, reps: int = 10) -> dict:
    """Our 16-byte streaming copy kernel (k_ceiling.hip) over `mib` MiB:
    read + write bytes per second, the practical ceiling of the streaming
    layers."""
    import torch
    from conv_bn_silu_amd import binding as B
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for _ in range(20):
        assert B.lib.conv_bn_silu_bench_copy(a.data_ptr(), b.data_ptr(), n, sp) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        assert B.lib.conv_bn_silu_bench_copy(a.data_ptr(), b.data_ptr(), n, sp) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * n / sec / 1e9, 1), "copy_bytes_each_way": n,
            "copy_what": "copy kernel, one 16-byte load and store per lane, one 256-lane workgroup per 4 KiB, "
                         "non-temporal stores"}


def same_bytes_copy(wl, reps: int = 100) -> dict:
    """The copy kernel moving the layer's algorithmic bytes (half read, half
    written), on rotated buffer pairs as the layer's own timing uses, timed
    per launch: what a kernel of this size costs when it does nothing but
    stream its bytes, start-up and tail included."""
    import torch
    from conv_bn_silu_amd import binding as B
    n = (wl.algorithmic_bytes // 2 + 15) // 16 * 16
    sets = max(2, math.ceil(2 * MALL_BYTES / (2 * n)))
    src = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    dst = [torch.empty_like(a) for a in src]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    fn = B.lib.conv_bn_silu_bench_copy
    for i in range(max(20, reps // 2)):
        assert fn(src[i % sets].data_ptr(), dst[i % sets].data_ptr(), n, sp) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        assert fn(src[i % sets].data_ptr(), dst[i % sets].data_ptr(), n, sp) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"us": round(us, 3), "bytes_each_way": n, "sets": sets}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_passes(key: str, min_seconds: float, max_reps: int = 50) -> dict:
    """The oracle as it stands (conv, BN and SiLU passes, fp64) on one
    workload, each pass timed on its own, repeated until ~min_seconds."""
    import oracle
    from conv_bn_silu_amd import synth
    wl = synth.WORKLOADS[key]
    inp = synth.make_inputs(wl)
    o = oracle.get()
    per = {"conv": 0.0, "bn": 0.0, "silu": 0.0}
    reps = 0
    while reps < max_reps and (reps == 0 or sum(per.values()) < min_seconds):
        t0 = time.perf_counter()
        t1 = o.conv(inp.x, inp.w, wl.stride, wl.pad)
        t_a = time.perf_counter()
        t2 = o.bn(t1, inp.scale, inp.bias)
        t_b = time.perf_counter()
        o.silu(t2)
        t_c = time.perf_counter()
        per["conv"] += t_a - t0
        per["bn"] += t_b - t_a
        per["silu"] += t_c - t_b
        reps += 1
    total = sum(per.values()) / reps
    return {"workload": wl.name, "reps": reps, "seconds_per_pass": {k: round(v / reps, 4) for k, v in per.items()},
            "seconds_per_call": round(total, 4), "fp64_gflops": round(wl.flops / total / 1e9, 3)}


def cpu_baseline(key: str, gpu_tflops: float, min_seconds: float = 10.0) -> dict:
    """The oracle on the host cores: the headline workload on every thread
    OpenMP uses, then c1, c2 and c4 on one thread (in a child process with
    OMP_NUM_THREADS=1), each pass timed on its own."""
    from conv_bn_silu_amd import synth
    wl = synth.WORKLOADS[key]
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    mt = oracle_passes(key, min_seconds)
    code = ("import json, sys; sys.path.insert(0, %r); import bench; "
            "print(json.dumps({k: bench.oracle_passes(k, 0.0, 1) for k in ('c1', 'c2', 'c4')}))" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    single = None
    try:
        res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
        if res.returncode == 0:
            single = json.loads(res.stdout.strip().splitlines()[-1])
    except (subprocess.TimeoutExpired, ValueError, IndexError):
        single = None
    value = wl.flops / mt["seconds_per_call"] / 1e12
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload {wl.name} ({wl.flops / 1e9:.1f} GFLOP) x{mt['reps']}: fp64 conv, BN "
                      f"and SiLU passes, each timed, on {threads} threads",
            "cpu_model": cpu_model(), "seconds_per_pass": mt["seconds_per_pass"],
            "fp64_gflops": mt["fp64_gflops"], "gpu_over_oracle": round(gpu_tflops / value, 1),
            "single_thread": single}


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


def layer_entry(q: dict, ceil: dict) -> dict:
    wl = q["wl"]
    peak = MFMA_F32_TFLOPS if wl.dtype == 0 else MFMA_BF16_TFLOPS
    ent = {"variant": q["variant"], "kernel_us": round(q["kernel_s"] * 1e6, 3),
           "wall_us_per_step": round(q["wall_per_step_s"] * 1e6, 3),
           "tflops": round(q["tflops_kernel"], 3), "hbm_gbs_algorithmic": round(q["hbm_gbs_alg"], 1),
           "bound": q["roofline"]["bound"], "frac": q["roofline"]["frac"],
           "mfma_frac": round(q["tflops_kernel"] / peak, 4),
           "hbm_frac": round(q["hbm_gbs_alg"] / HBM_PEAK_GBS, 4),
           "flops": wl.flops, "algorithmic_bytes": wl.algorithmic_bytes}
    if "copy_gbs" in ceil:
        ent["frac_of_copy_ceiling"] = round(q["hbm_gbs_alg"] / ceil["copy_gbs"], 4)
    if "mfma_bf16_tflops" in ceil and wl.dtype == 1:
        ent["frac_of_mfma_ceiling"] = round(q["tflops_kernel"] / ceil["mfma_bf16_tflops"], 4)
    tr = traffic_for(wl, q["variant"])
    if tr:
        ent["traffic_bytes"] = tr["traffic_bytes_per_launch"]
        ent["traffic_over_algorithmic"] = tr["traffic_over_algorithmic"]
    return ent


# Shapes on both sides of each dispatch rule (N, C_in, H, W, C_out, KH, KW,
# stride, pad, dtype): the scalar kernel's size limits (fp32 and bf16), the
# 1x1 kernel's channel limit, the strided-row kernel's channel range, the
# 32x32 window kernel against the 16x16 one at small and large channel
# counts and tile fills, a 5x5 filter and a width the 32x32 kernel does not
# serve.
DISPATCH_SWEEP = [
    (1, 16, 32, 32, 32, 3, 3, 1, 1, 0), (1, 16, 48, 48, 32, 3, 3, 1, 1, 0), (1, 16, 64, 64, 32, 3, 3, 1, 1, 0),
    (1, 32, 64, 64, 64, 3, 3, 1, 1, 0), (2, 32, 64, 64, 64, 3, 3, 1, 1, 0), (2, 64, 64, 64, 64, 3, 3, 1, 1, 0),
    (4, 64, 64, 64, 128, 3, 3, 1, 1, 0), (1, 32, 48, 48, 64, 3, 3, 1, 1, 1), (1, 16, 64, 64, 64, 3, 3, 1, 1, 1),
    (8, 64, 40, 40, 128, 5, 5, 1, 2, 1), (8, 48, 40, 36, 96, 3, 3, 1, 1, 1), (8, 16, 80, 80, 64, 3, 3, 1, 1, 1),
    (1, 16, 32, 32, 32, 3, 3, 1, 1, 1), (1, 16, 48, 48, 32, 3, 3, 1, 1, 1), (1, 32, 64, 64, 64, 3, 3, 1, 1, 1),
    (8, 256, 40, 40, 256, 1, 1, 1, 0, 1), (8, 512, 40, 40, 256, 1, 1, 1, 0, 1), (8, 64, 80, 80, 128, 1, 1, 1, 0, 1),
    (16, 32, 160, 160, 64, 3, 3, 2, 1, 1), (16, 64, 160, 160, 128, 3, 3, 2, 1, 1),
    (16, 96, 80, 80, 192, 3, 3, 2, 1, 1), (16, 128, 80, 80, 256, 3, 3, 2, 1, 1),
    (32, 64, 20, 20, 256, 3, 3, 1, 1, 1), (32, 96, 20, 20, 256, 3, 3, 1, 1, 1),
    (32, 128, 20, 20, 256, 3, 3, 1, 1, 1), (32, 256, 20, 20, 256, 3, 3, 1, 1, 1),
    (32, 256, 16, 16, 256, 3, 3, 1, 1, 1), (32, 256, 24, 24, 256, 3, 3, 1, 1, 1),
    (32, 256, 40, 40, 256, 3, 3, 1, 1, 1), (16, 256, 10, 10, 512, 3, 3, 1, 1, 1),
]


DISPATCH_ROUNDS = 3


def dispatch_check(wl, steps: int, warmup: int) -> dict:
    """Every variant that supports the shape, timed DISPATCH_ROUNDS times in
    interleaved rounds (the best of them kept: the smallest shapes run at
    the host's issue rate, where single runs differ by several percent);
    AUTO's pick against the fastest."""
    from conv_bn_silu_amd import binding as B
    global SETTLE_S
    settle, SETTLE_S = SETTLE_S, min(SETTLE_S, 0.05)  # the clocks are up by now: a short settle per variant
    L = Layer(wl)
    times = {}
    macs = wl.flops // 2
    names = []
    for name, v in B.VARIANTS.items():
        if v == 0 or not B.variant_supports(v, *L.geo):
            continue
        if name == "scalar" and macs > (1 << 31):
            continue  # a minute of scalar work per call; never the fastest there
        names.append(name)
    for _ in range(DISPATCH_ROUNDS):
        for name in names:
            # the scalar kernel on a large shape: fewer steps (it is slow there)
            n_st = steps if name != "scalar" or macs <= (1 << 26) else max(3, steps // 10)
            t = round(measure_fused(wl, n_st, min(warmup, 3), name, L)["kernel_s"] * 1e6, 3)
            times[name] = min(times.get(name, t), t)
    picked = B.variant_name(B.select_variant(*L.geo))
    fastest = min(times, key=times.get)
    SETTLE_S = settle
    del L
    return {"variants_us": times, "auto_picks": picked, "fastest": fastest,
            "auto_over_fastest": round(times[picked] / times[fastest], 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, help="headline layer, c1..c5 (default c5)")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--only", action="store_true", help="only the headline layer (profiling runs)")
    ap.add_argument("--variants", action="store_true", help="also check the dispatch on a shape sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed repetitions of each layer's step before its warm-up (clock ramp)")
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
    from conv_bn_silu_amd import synth
    global SETTLE_S
    SETTLE_S = args.settle_ms / 1000.0
    wl = synth.WORKLOADS[args.workload]
    dev = device_info()
    num_cu = dev.get("num_cu", 256)
    ceil = {}
    if not args.only:
        ceil.update(copy_ceiling())
        ceil.update(mfma_ceiling(num_cu))
        log(f"[bench] ceilings: copy {ceil['copy_gbs']:.0f} GB/s, MFMA {ceil['mfma_bf16_tflops']:.0f} TFLOP/s")

    log(f"[bench] {args.workload} variant {args.variant}: {args.warmup} warmup + {args.steps} steps")
    r = measure_fused(wl, args.steps, args.warmup, args.variant)
    log(f"[bench] {wl.name}: {r['kernel_s'] * 1e6:.2f} us/launch ({r['variant']}), "
        f"{r['wall_per_step_s'] * 1e6:.2f} us/step wall")
    roof = dict(r["roofline"])
    tr = traffic_for(wl, r["variant"])
    roof["traffic"] = tr["traffic_bytes_per_launch"] if tr else None
    out = {
        "metric": METRIC,
        "value": round(r["tflops_wall"], 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["wall_per_step_s"] * 1e3, 5), "higher_is_better": True,
        "scaling": None, "vs_baseline": None, "dtype": "bf16" if wl.dtype == synth.DTYPE_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": wl.N, "C_in": wl.C_in, "H": wl.H, "W": wl.W, "C_out": wl.C_out,
                   "KH": wl.KH, "KW": wl.KW, "stride": wl.stride, "pad": wl.pad, "variant": r["variant"],
                   "rotated_buffer_sets": r["sets"], "kernel_us_mean": round(r["kernel_s"] * 1e6, 3),
                   "host_issue_us_per_step": round(r["host_issue_us_per_step"], 3),
                   "settle_ms": args.settle_ms,
                   "algorithmic_bytes": wl.algorithmic_bytes, "flops": wl.flops, **dev},
        "roofline": roof,
    }
    if not args.only:
        out["ceilings"] = ceil
        out["roofline"]["frac_of_measured_ceiling"] = round(
            r["tflops_kernel"] / ceil["mfma_bf16_tflops"] if roof["bound"] == "mfma"
            else r["hbm_gbs_alg"] / ceil["copy_gbs"], 4)
        sub_steps = max(20, args.steps // 2)
        layers = {}
        for key in sorted(synth.WORKLOADS):
            wlk = synth.WORKLOADS[key]
            Lk = None if key == args.workload and args.variant == "auto" else Layer(wlk)
            q = r if Lk is None else measure_fused(wlk, sub_steps, args.warmup, layer=Lk)
            ent = layer_entry(q, ceil)
            gr = measure_graph(wlk, layer=Lk)
            ent["graph_us_per_launch"] = gr["us_per_launch"]
            if gr.get("error"):
                ent["graph_error"] = gr["error"]
            if ent["bound"] == "hbm":
                cp = same_bytes_copy(wlk)
                ent["same_bytes_copy_us"] = cp["us"]
                ent["over_same_bytes_copy"] = round(ent["kernel_us"] / cp["us"], 4)
            u = measure_unfused(wlk, sub_steps, args.warmup)
            ent["unfused_us_per_step"] = round(u["us_per_step"], 3)
            ent["fused_speedup_over_unfused"] = round(u["us_per_step"] / (q["kernel_s"] * 1e6), 3)
            log(f"[bench] layer {key}: {ent['kernel_us']:.2f} us ({ent['variant']}, frac {ent['frac']}), "
                f"graph-replayed {ent['graph_us_per_launch']} us, same-bytes copy "
                f"{ent.get('same_bytes_copy_us', '-')} us, unfused {ent['unfused_us_per_step']:.2f} us")
            layers[wlk.name] = ent
        out["layers"] = layers
    if args.variants:
        checks = []
        shapes = [(k, synth.WORKLOADS[k]) for k in sorted(synth.WORKLOADS)]
        for i, g in enumerate(DISPATCH_SWEEP):
            seed = 7000 + i
            shapes.append((f"sweep{i}", synth.Workload(f"sweep{i}", g[9], *g[:9], "n01", seed)))
        for key, wlk in shapes:
            c = dispatch_check(wlk, max(10, args.steps // 10), args.warmup)
            c["shape"] = [wlk.N, wlk.C_in, wlk.H, wlk.W, wlk.C_out, wlk.KH, wlk.KW, wlk.stride, wlk.pad, wlk.dtype]
            c["name"] = wlk.name
            log(f"[bench] dispatch {wlk.name}: auto {c['auto_picks']}, fastest {c['fastest']}, "
                f"ratio {c['auto_over_fastest']}")
            checks.append(c)
        worst = max(c["auto_over_fastest"] for c in checks)
        out["dispatch"] = {"shapes": checks, "worst_auto_over_fastest": worst,
                           "auto_within_5pct": worst <= DISPATCH_SLACK}
    if args.no_cpu_baseline or args.only:
        out["cpu_baseline"] = None
    else:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args.workload, r["tflops_kernel"], args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if args.variants and not out["dispatch"]["auto_within_5pct"]:
        log(f"[bench] dispatch check failed: AUTO is {out['dispatch']['worst_auto_over_fastest']}x the fastest")
        sys.exit(3)


if __name__ == "__main__":
    main()
