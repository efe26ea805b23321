#!/usr/bin/env python3
"""rocprofv3 runs over bench.py, summarised into short text records under
profiles/ (run on a machine with the GPU; raw profiler output stays in
gpurun_out/).

  python3 bench_profile.py trace   [--workload c5]
      rocprofv3 --kernel-trace --stats over the bench command for the named
      workload alone (bench.py --only); writes
      profiles/kernel_trace_<workload>.md with the per-kernel durations and
      the bench's own JSON line from the same run.

  python3 bench_profile.py traffic [--workload c5]
      four counter runs, each on its own: FETCH_SIZE and WRITE_SIZE over a
      plain 1 GiB device copy (to scale the counters to bytes), then
      FETCH_SIZE and WRITE_SIZE over the bench command; writes
      profiles/traffic_<workload>.md, which bench.py reads back while the
      source of the variant's kernel is unchanged.

  python3 bench_profile.py mfma    [--workload c5]
      one counter run (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16)
      over the bench command; writes
      profiles/mfma_<workload>.md with the matrix-core busy fraction of the
      operator's kernel and the MFMA work it counted against the layer's
      algorithmic FLOP.

  python3 bench_profile.py stalls  [--workload c5]
      two counter runs over the bench command: the LDS counters
      (SQ_INSTS_LDS, SQ_LDS_BANK_CONFLICT, SQ_LDS_ADDR_CONFLICT,
      SQ_LDS_UNALIGNED_STALL, SQ_LDS_IDX_ACTIVE, SQ_WAIT_INST_LDS,
      SQ_ACTIVE_INST_LDS), then the wave-time counters (SQ_WAVE_CYCLES,
      SQ_BUSY_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_ANY,
      SQ_ACTIVE_INST_VALU, SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA); writes
      profiles/stalls_<workload>.md with the LDS bank-conflict rate (conflict
      cycles over LDS active cycles) and the shares of wave time spent
      waiting and issuing.

  python3 bench_profile.py all
      trace for c1..c5, traffic for c2..c5, mfma for c5, stalls for c2..c5:
      each rocprofv3 pass a run of its own.

This process never touches the GPU itself: rocprofv3 starts bench.py as a
child.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
RAW = os.path.join(ROOT, "gpurun_out", "rocprof")
PROFILES = os.path.join(ROOT, "profiles")  # --out overrides


def run(cmd: list[str], limit: int) -> str:
    """Run under a hard time limit, echoing the child's output as it comes
    (stderr passes straight through); returns its stdout."""
    print("[profile] " + " ".join(cmd), flush=True)
    p = subprocess.Popen(["timeout", "-s", "KILL", str(limit)] + cmd, cwd=ROOT, stdout=subprocess.PIPE, text=True)
    lines = []
    for line in p.stdout:
        lines.append(line)
        sys.stdout.write(line[:2000])
        sys.stdout.flush()
    rc = p.wait()
    out = "".join(lines)
    if rc != 0:
        # rocprofv3 itself may end with SIGSEGV after a complete run; accept
        # that only if the program's JSON line came out.
        if not (rc in (139, -11) and out.strip().endswith("}")):
            raise SystemExit(f"command failed with status {rc}")
    return out


def last_json(text: str) -> dict:
    for line in reversed(text.strip().splitlines()):
        line = line.strip()
        if line.startswith("{") and line.endswith("}"):
            return json.loads(line)
    raise SystemExit("no JSON line in the program's output")


def bench_cmd(workload: str, steps: int | None = None, extra: tuple = ()) -> list[str]:
    cmd = ["python3", "bench.py", "--only", "--workload", workload]
    if steps is not None:
        cmd += ["--steps", str(steps), "--warmup", "2"]
    return cmd + list(extra)


def read_csv(path: str) -> list[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def workload_name(key: str) -> str:
    from conv_bn_silu_amd import synth
    return synth.WORKLOADS[key].name


def do_trace(args) -> None:
    out = os.path.join(RAW, f"trace_{args.workload}")
    cmd = bench_cmd(args.workload, 100)
    prof = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", out, "-o", "run", "--"]
    stdout = run(prof + cmd, 400)
    line = last_json(stdout)
    stats = read_csv(os.path.join(out, "run_kernel_stats.csv"))
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    name = workload_name(args.workload)
    rows = []
    for r in stats[:12]:
        rows.append(f"| {r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                    f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.1f} |")
    text = [f"# Kernel trace: fused conv+BN+SiLU, workload {name}", "",
            "Command (from the repository root, on one MI355X):", "",
            "```", " ".join(prof[:-1] + ["--"] + cmd).replace(out, f"gpurun_out/rocprof/trace_{args.workload}"),
            "```", "",
            "Kernels by total time (durations in microseconds):", "",
            "| kernel | calls | avg | min | max | % time |", "|---|---|---|---|---|---|"] + rows + [
            "", "bench.py's own JSON line from the same run (kernel_us_mean: HIP events around the timed "
            "region on the launch stream, per launch; the average above also counts the warm-up "
            "launches):", "", "```json", json.dumps(line), "```", ""]
    os.makedirs(args.out, exist_ok=True)
    path = os.path.join(args.out, f"kernel_trace_{name}.md")
    with open(path, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {path}", flush=True)


def counter_by_kernel(path: str, counter: str, match, combine=lambda a, b: a + b) -> dict[str, list[float]]:
    """Per kernel name that `match` accepts: the counter's value for each of
    its dispatches, the rows of one dispatch (one per hardware instance)
    combined by `combine` (summed by default)."""
    by: dict[str, dict[str, float]] = {}
    for r in read_csv(path):
        if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
            continue
        d = by.setdefault(r["Kernel_Name"], {})
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(d))
        v = float(r["Counter_Value"])
        d[key] = combine(d[key], v) if key in d else v
    if not by:
        raise SystemExit(f"no {counter} rows in {path}")
    return {k: list(v.values()) for k, v in by.items()}


def mean(v: list[float]) -> float:
    return sum(v) / len(v)


def do_traffic(args) -> None:
    import bench
    copy_mib = 1024
    res = {}
    cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = os.path.join(RAW, f"copy_{counter.lower()}")
        c = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", out, "-o", "run", "--",
             "python3", "bench.py", "--copy-calibration", str(copy_mib), "--steps", "8"]
        run(c, 60)
        by = counter_by_kernel(os.path.join(out, "run_counter_collection.csv"), counter,
                               lambda k: "opy" in k or "elementwise" in k)
        name = max(by, key=lambda n: len(by[n]))          # the copy runs 8 times, the fill once
        kib = mean(by[name])
        res[f"copy_{counter}"] = {"kernel": name[:100], "dispatches": len(by[name]), "kib_per_dispatch": kib,
                                  "factor": (copy_mib << 20) / (kib * 1024.0)}
        cmds[f"copy_{counter}"] = " ".join(["timeout -s KILL 60"] + c).replace(out, "gpurun_out/rocprof/copy")
    dominant = None
    variant = None
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        out = os.path.join(RAW, f"{args.workload}_{counter.lower()}")
        c = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", out, "-o", "run", "--"] + \
            bench_cmd(args.workload, 20)
        variant = last_json(run(c, 60))["config"]["variant"]
        by = counter_by_kernel(os.path.join(out, "run_counter_collection.csv"), counter, lambda k: "cbs" in k)
        if dominant is None:  # the operator's kernel that fetches the most
            dominant = max(by, key=lambda n: sum(by[n]))
        res[counter] = {"kernel": dominant[:100], "dispatches": len(by[dominant]),
                        "kib_per_dispatch": mean(by[dominant]),
                        "other_kernels_kib": {k[:60]: round(mean(v), 1) for k, v in by.items() if k != dominant}}
        cmds[counter] = " ".join(["timeout -s KILL 60"] + c).replace(out, f"gpurun_out/rocprof/{args.workload}")
    from conv_bn_silu_amd import synth
    wl = synth.WORKLOADS[args.workload]
    fetch = res["FETCH_SIZE"]["kib_per_dispatch"] * 1024 * res["copy_FETCH_SIZE"]["factor"]
    write = res["WRITE_SIZE"]["kib_per_dispatch"] * 1024 * res["copy_WRITE_SIZE"]["factor"]
    rec = {"workload": wl.name, "variant": variant, "kernel": res["FETCH_SIZE"]["kernel"],
           "fetch_kib_per_dispatch_raw": round(res["FETCH_SIZE"]["kib_per_dispatch"], 1),
           "write_kib_per_dispatch_raw": round(res["WRITE_SIZE"]["kib_per_dispatch"], 1),
           "copy_bytes": copy_mib << 20,
           "fetch_factor": round(res["copy_FETCH_SIZE"]["factor"], 4),
           "write_factor": round(res["copy_WRITE_SIZE"]["factor"], 4),
           "read_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
           "traffic_bytes_per_launch": int(fetch + write),
           "algorithmic_bytes": wl.algorithmic_bytes,
           "other_kernels_fetch_kib_raw": res["FETCH_SIZE"]["other_kernels_kib"],
           "traffic_over_algorithmic": round((fetch + write) / wl.algorithmic_bytes, 4),
           "kernel_sources_digest": bench.kernel_sources_digest(variant)}
    text = [f"# HBM traffic: fused conv+BN+SiLU, workload {wl.name}", "",
            "Each counter in a run of its own (from the repository root, on one MI355X):", "",
            "```"] + [cmds[k] for k in ("copy_FETCH_SIZE", "copy_WRITE_SIZE", "FETCH_SIZE", "WRITE_SIZE")] + [
            "```", "",
            f"The copy moves {copy_mib} MiB each way per dispatch; factor = copy bytes / counter bytes "
            f"(FETCH_SIZE {rec['fetch_factor']}, WRITE_SIZE {rec['write_factor']}), applied to the "
            f"kernel's per-dispatch counter means ({res['FETCH_SIZE']['dispatches']} dispatches).", "",
            "```json", json.dumps(rec, indent=1), "```", ""]
    path = os.path.join(args.out, f"traffic_{wl.name}.md")
    os.makedirs(args.out, exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {path}: {json.dumps(rec)}", flush=True)


def do_mfma(args) -> None:
    counters = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    out = os.path.join(RAW, f"{args.workload}_mfma")
    c = ["rocprofv3", "--pmc"] + counters + ["--output-format", "csv", "-d", out, "-o", "run", "--"] + \
        bench_cmd(args.workload, 20)
    variant = last_json(run(c, 60))["config"]["variant"]
    path = os.path.join(out, "run_counter_collection.csv")
    vals = {}
    for ctr in counters:
        by = counter_by_kernel(path, ctr, lambda k: "cbs" in k)
        name = max(by, key=lambda n: sum(by[n]))
        vals[ctr] = (name, mean(by[name]), len(by[name]))
    kname = vals[counters[0]][0]
    durs = {}
    for r in read_csv(path):
        if r["Kernel_Name"] == kname and r["Counter_Name"] == counters[0]:
            durs[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    dur = mean(list(durs.values()))
    from conv_bn_silu_amd import synth
    wl = synth.WORKLOADS[args.workload]
    simds, clock = 4 * 256, 2.4e9
    busy, mops = vals[counters[0]][1], vals[counters[1]][1]
    rec = {"workload": wl.name, "variant": variant, "kernel": kname[:100], "dispatches": vals[counters[0]][2],
           "SQ_VALU_MFMA_BUSY_CYCLES": busy, "SQ_INSTS_VALU_MFMA_MOPS_BF16": mops,
           "mfma_busy_cycles_per_simd": round(busy / simds), "dispatch_duration_us": round(dur * 1e6, 3),
           "mfma_busy_pct": round(100.0 * busy / simds / (dur * clock), 2),
           "mfma_flop_counted": mops * 512, "algorithmic_flop": wl.flops,
           "counted_over_algorithmic": round(mops * 512 / wl.flops, 4),
           "kernel_sources_digest": __import__("bench").kernel_sources_digest(variant)}
    text = [f"# Matrix-core use: fused conv+BN+SiLU, workload {wl.name}", "",
            "Counter run (from the repository root, on one MI355X):", "", "```",
            " ".join(["timeout -s KILL 60"] + c).replace(out, f"gpurun_out/rocprof/{args.workload}_mfma"), "```", "",
            "Per-dispatch means for the operator's kernel, SQ counters summed over the chip.  "
            f"mfma_busy_pct = SQ_VALU_MFMA_BUSY_CYCLES / {simds} SIMDs / (dispatch duration x 2.4 GHz) x 100, "
            "the duration from the dispatch's own timestamps in the same run (GRBM_GUI_ACTIVE is not used: "
            "under counter collection it also counts the time around each dispatch).  "
            "mfma_flop_counted = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 against the layer's 2*M*C_out*K "
            "(tile padding makes it larger).", "",
            "```json", json.dumps(rec, indent=1), "```", ""]
    os.makedirs(args.out, exist_ok=True)
    dst = os.path.join(args.out, f"mfma_{wl.name}.md")
    with open(dst, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {dst}: {json.dumps(rec)}", flush=True)


STALL_PASSES = (
    ["SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_UNALIGNED_STALL", "SQ_LDS_IDX_ACTIVE",
     "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS"],
    ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA"],
)


def do_stalls(args) -> None:
    from conv_bn_silu_amd import synth
    wl = synth.WORKLOADS[args.workload]
    vals, cmds, variant = {}, [], None
    for i, counters in enumerate(STALL_PASSES):
        out = os.path.join(RAW, f"{args.workload}_stalls{i}")
        c = ["rocprofv3", "--pmc"] + counters + ["--output-format", "csv", "-d", out, "-o", "run", "--"] + \
            bench_cmd(args.workload, 20)
        variant = last_json(run(c, 60))["config"]["variant"]
        cmds.append(" ".join(["timeout -s KILL 60"] + c).replace(out, f"gpurun_out/rocprof/{args.workload}_stalls{i}"))
        path = os.path.join(out, "run_counter_collection.csv")
        for ctr in counters:
            by = counter_by_kernel(path, ctr, lambda k: "cbs" in k)
            name = max(by, key=lambda n: sum(by[n]))
            vals[ctr] = mean(by[name])
            vals["_kernel"] = name[:100]
    def ratio(a, b):
        return round(vals[a] / vals[b], 4) if vals.get(b) else None
    rec = {"workload": wl.name, "variant": variant, "kernel": vals.pop("_kernel"),
           "counters_per_dispatch": {k: vals[k] for k in vals},
           "lds_bank_conflict_over_lds_active": ratio("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
           "lds_bank_conflict_cycles_per_lds_instruction": ratio("SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"),
           "wave_wait_share": ratio("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
           "wave_wait_inst_share": ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
           "wave_issue_share": ratio("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
           "wave_lds_wait_share": ratio("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
           "kernel_sources_digest": __import__("bench").kernel_sources_digest(variant)}
    text = [f"# LDS conflicts and wave stalls: fused conv+BN+SiLU, workload {wl.name}", "",
            "Two counter runs, each on its own (from the repository root, on one MI355X):", "", "```"] + cmds + \
           ["```", "",
            "Per-dispatch means for the operator's kernel, SQ counters summed over the chip.  "
            "lds_bank_conflict_over_lds_active = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (the share of the LDS "
            "unit's active cycles lost to bank conflicts); the wave shares divide by SQ_WAVE_CYCLES (the summed "
            "lifetime of the kernel's waves): SQ_WAIT_ANY counts cycles a wave waits for anything (a dependency, "
            "a counter, a barrier), SQ_WAIT_INST_ANY cycles it waits to issue its next instruction, "
            "SQ_ACTIVE_INST_ANY cycles in which it issues one, SQ_WAIT_INST_LDS cycles waiting to issue an LDS "
            "instruction.", "",
            "```json", json.dumps(rec, indent=1), "```", ""]
    os.makedirs(args.out, exist_ok=True)
    dst = os.path.join(args.out, f"stalls_{wl.name}.md")
    with open(dst, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {dst}: {json.dumps(rec)}", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("mode", choices=["trace", "traffic", "mfma", "stalls", "all"])
    ap.add_argument("--workload", default="c5")
    ap.add_argument("--out", default=PROFILES, help="where the summaries go (default profiles/)")
    args = ap.parse_args()
    os.makedirs(RAW, exist_ok=True)
    if args.mode == "trace":
        do_trace(args)
    elif args.mode == "mfma":
        do_mfma(args)
    elif args.mode == "traffic":
        do_traffic(args)
    elif args.mode == "stalls":
        do_stalls(args)
    else:
        for key in ("c1", "c2", "c3", "c4", "c5"):
            args.workload = key
            do_trace(args)
        for key in ("c2", "c3", "c4", "c5"):
            args.workload = key
            do_traffic(args)
        args.workload = "c5"
        do_mfma(args)
        for key in ("c2", "c3", "c4", "c5"):
            args.workload = key
            do_stalls(args)


if __name__ == "__main__":
    main()
