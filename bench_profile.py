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

  python3 bench_profile.py lds
      one counter run (SQ_INSTS_LDS, SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE)
      over the library's LDS probe (conv_bn_silu_bench_lds), one dispatch per
      address pattern: the bank model's test patterns and the fragment-read
      and staging patterns of the operator's kernels; writes
      profiles/lds_bank_model.md.

  python3 bench_profile.py isa
      times the library's instruction-issue probe (conv_bn_silu_bench_isa)
      with HIP events in a child process: cycles per wave instruction of
      fma, exp2, reciprocal, the BN + SiLU epilogue, and of MFMA with
      independent fmas among them, at 1, 2 and 4 waves per SIMD; writes
      profiles/isa_rates.md.

  python3 bench_profile.py resources
      (no GPU) the compiler's per-kernel resource report that
      conv_bn_silu_amd/build.py writes beside the library (registers,
      scratch, LDS, waves per SIMD), demangled, as
      profiles/kernel_resources.md.

  python3 bench_profile.py dispatch
      bench.py --variants --no-cpu-baseline in a child: every variant that
      supports each of the five workloads and of the dispatch sweep's
      shapes, timed (best of three interleaved rounds), against AUTO's
      pick; writes profiles/dispatch_sweep.md
      (exits non-zero, as bench.py does, when AUTO is more than 5% slower
      than the fastest variant anywhere).

  python3 bench_profile.py all
      trace for c1..c5, traffic for c2..c5, mfma for c5, stalls for c2..c5,
      lds, isa, resources: each rocprofv3 pass a run of its own.

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


def lds_cases() -> list[tuple[str, int, list[int]]]:
    """(name, op, 64 byte addresses): op 0 ds_read_b128, 1 ds_read_b64,
    2 ds_read_b64_tr_b16, 3 ds_write_b64, 4 ds_write_b128."""
    lanes = range(64)

    def tr32(pitch):  # 32x32x16 A fragment: 16-lane group g: pixels 16(g&1).., k half g>>1
        return [(8 * ((l >> 4) >> 1) + ((l & 15) >> 2)) * pitch + 2 * (16 * ((l >> 4) & 1) + 4 * (l & 3))
                for l in lanes]

    def tr16(pitch, swap=False):  # 16x16x32 A fragment: group g reads rows 8g + (j>>2)
        out = []
        for l in lanes:
            r = 8 * (l >> 4) + ((l & 15) >> 2)
            pb = 8 * (l & 3)
            if swap:
                pb ^= ((r >> 1) & 1) << 6
            out.append(r * pitch + pb)
        return out

    def stem(P=672, SLOT=6112):  # 27 (channel, tap row, tap column) arrays, plain pitch
        out = []
        for l in lanes:
            k = 8 * (l >> 4) + ((l & 15) >> 2)
            ci, r = divmod(k, 9)
            kh, kw = divmod(r, 3)
            out.append(kh * SLOT + (3 * ci + kw) * P + 8 * (l & 3))
        return out

    def win_write(plane):  # window32 staging write at one column, 20x20 tile, row pitch 36 records
        return [(l & 1) * plane + (((l >> 1) // 4) * 36 + 8 * ((l >> 1) % 4)) * 16 for l in lanes]

    return [
        ("b128 read, contiguous", 0, [16 * l for l in lanes]),
        ("b128 read, 16-lane groups contiguous (256 B), 1 KiB apart", 0, [16 * (l % 16) + 1024 * (l // 16) for l in lanes]),
        ("b128 read, 8-lane groups contiguous (128 B), 512 B apart", 0, [16 * (l % 8) + 512 * (l // 8) for l in lanes]),
        ("b128 read, stride 256 B", 0, [256 * l for l in lanes]),
        ("b128 read, one address", 0, [0 for l in lanes]),
        ("b64 read, contiguous", 1, [8 * l for l in lanes]),
        ("b64 read, 32-lane halves contiguous (256 B), 1 KiB apart", 1, [8 * (l % 32) + 1024 * (l // 32) for l in lanes]),
        ("b64 read, 16-lane groups contiguous (128 B), 1 KiB apart", 1, [8 * (l % 16) + 1024 * (l // 16) for l in lanes]),
        ("tr read, contiguous", 2, [8 * l for l in lanes]),
        ("tr read, 16-lane groups contiguous (128 B), 1 KiB apart", 2, [8 * (l % 16) + 1024 * (l // 16) for l in lanes]),
        ("tr read 32x32x16 fragment, row pitch 448 (pointwise)", 2, tr32(448)),
        ("tr read 32x32x16 fragment, row pitch 320 (strided_rows, OW 160)", 2, tr32(320)),
        ("tr read 32x32x16 fragment, row pitch 512", 2, tr32(512)),
        ("tr read 16x16x32 fragment, row pitch 128", 2, tr16(128)),
        ("tr read 16x16x32 fragment, row pitch 128, halves swapped on row bit 1", 2, tr16(128, True)),
        ("tr read 16x16x32 fragment, row pitch 192", 2, tr16(192)),
        ("tr read 16x16x32 fragment, stem arrays (672 B pitch, 6112 B rows)", 2, stem()),
        ("b64 write, contiguous", 3, [8 * l for l in lanes]),
        ("b128 write, contiguous", 4, [16 * l for l in lanes]),
        ("b128 write, window32 staging, octet planes 12672 B apart (792 records)", 4, win_write(12672)),
        ("b128 write, window32 staging, octet planes 12688 B apart (793 records)", 4, win_write(12688)),
    ]


def lds_child(path: str) -> None:
    """Child of the `lds` mode: one probe dispatch per case, in order."""
    import torch
    from conv_bn_silu_amd import binding as B
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    cases = lds_cases()
    for name, op, addrs in cases:
        assert len(addrs) == 64 and all(0 <= a < 65536 - 16 for a in addrs), name
        a = torch.tensor(addrs, dtype=torch.int32, device="cuda")
        if B.lib.conv_bn_silu_bench_lds(op, a.data_ptr(), out.data_ptr(), st) != 0:
            raise SystemExit(f"probe launch failed: {name}")
        torch.cuda.synchronize()
    with open(path, "w") as f:
        json.dump([c[0] for c in cases], f)
    print(json.dumps({"cases": len(cases)}), flush=True)


def do_lds(args) -> None:
    out = os.path.join(RAW, "lds_probe")
    names_path = os.path.join(out, "cases.json")
    os.makedirs(out, exist_ok=True)
    counters = ["SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"]
    c = ["rocprofv3", "--pmc"] + counters + ["--output-format", "csv", "-d", out, "-o", "run", "--",
                                             "python3", "bench_profile.py", "lds-child", "--cases", names_path]
    run(c, 90)
    names = json.load(open(names_path))
    per = {}
    for r in read_csv(os.path.join(out, "run_counter_collection.csv")):
        if "lds_probe" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)
    if len(ids) != len(names):
        raise SystemExit(f"{len(ids)} probe dispatches for {len(names)} cases")
    # 64 conflict-free 16-byte initial stores per lane precede the 256 probed
    # operations; per probed operation: (counter - init) / 256.
    init = per[ids[names.index("b128 write, contiguous")]]
    init_active = init["SQ_LDS_IDX_ACTIVE"] / 5.0  # 64 of the 320 writes there, each 8 cycles (see below)
    rows = []
    for i, name in zip(ids, names):
        d = per[i]
        conf = d["SQ_LDS_BANK_CONFLICT"] / 256.0
        active = (d["SQ_LDS_IDX_ACTIVE"] - init_active) / 256.0
        rows.append((name, round(conf, 2), round(active, 2)))
    text = ["# LDS bank model: measured per address pattern", "",
            "One counter run (from the repository root, on one MI355X):", "", "```",
            " ".join(["timeout -s KILL 90"] + c).replace(out, "gpurun_out/rocprof/lds_probe"), "```", "",
            "Each case is one dispatch of the library's LDS probe (`conv_bn_silu_bench_lds`): one wave repeats one "
            "LDS operation 256 times at the per-lane addresses the case lists (`lds_cases()` in "
            "bench_profile.py), after 64 conflict-free 16-byte stores per lane that fill the array.  Per probed "
            "operation: bank-conflict cycles (SQ_LDS_BANK_CONFLICT / 256) and LDS active cycles "
            "(SQ_LDS_IDX_ACTIVE less the initial stores, / 256).", "",
            "| pattern | conflict cycles per op | LDS cycles per op |", "|---|---|---|"]
    text += [f"| {n} | {cf} | {ac} |" for n, cf, ac in rows]
    text += ["", "Reading: 16-byte operations are served 16 lanes (256 bytes) per LDS cycle, 8-byte ones and the "
             "transposed read 32 lanes per cycle; a pass is conflict-free when its lanes cover 256 distinct "
             "bytes (one repeated address is broadcast).", ""]
    os.makedirs(args.out, exist_ok=True)
    dst = os.path.join(args.out, "lds_bank_model.md")
    with open(dst, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {dst}", flush=True)


ISA_KINDS = [(0, "v_fma_f32", 1), (1, "v_exp_f32", 1), (2, "v_add_f32 + v_rcp_f32", 2),
             (3, "BN + SiLU epilogue (2 fma, exp, add, rcp, mul)", 6)]
MFMA_KINDS = [(10, 0), (11, 8), (12, 16), (14, 32), (18, 64)]


def isa_child() -> None:
    """Child of the `isa` mode: times the issue probes with HIP events."""
    import torch
    from conv_bn_silu_amd import binding as B
    st = torch.cuda.current_stream()
    num_cu = 256
    sink = torch.empty(4 * num_cu * 256, device="cuda")

    def timed(kind, n_wg, iters):
        for _ in range(3):
            if B.lib.conv_bn_silu_bench_isa(kind, n_wg, iters, sink.data_ptr(), st.cuda_stream) != 0:
                raise SystemExit(f"probe launch failed: kind {kind}")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(5):
            B.lib.conv_bn_silu_bench_isa(kind, n_wg, iters, sink.data_ptr(), st.cuda_stream)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / 5

    clock = 2.4e9
    rec = {"clock_hz_assumed": clock, "vector": [], "mfma": []}
    for kind, what, n_instr in ISA_KINDS:
        for wps in (1, 2, 4):
            s = timed(kind, num_cu * wps, 20000)
            per = s * clock / (wps * 20000 * 8)  # cycles per 8-chain step of one wave, per SIMD
            rec["vector"].append({"what": what, "waves_per_simd": wps, "seconds": s,
                                  "cycles_per_element_group": round(per, 2),
                                  "cycles_per_instruction": round(per / n_instr, 2)})
    for kind, nv in MFMA_KINDS:
        for wps in (1, 2):
            s = timed(kind, num_cu * wps, 5000)
            rec["mfma"].append({"fmas_per_8_mfma": nv, "waves_per_simd": wps, "seconds": s,
                                "cycles_per_mfma": round(s * clock / (wps * 5000 * 8), 2)})
    print(json.dumps(rec), flush=True)


def do_isa(args) -> None:
    cmd = ["python3", "bench_profile.py", "isa-child"]
    rec = last_json(run(cmd, 300))
    text = ["# Instruction issue rates: measured", "", "Command (from the repository root, on one MI355X):", "",
            "```", "timeout -s KILL 300 " + " ".join(cmd), "```", "",
            "The library's issue probe (`conv_bn_silu_bench_isa`), 256, 512 or 1024 workgroups of 4 waves (1, 2, "
            "4 waves per SIMD), 8 independent chains per lane, register-only; HIP events around 5 launches.  "
            "Cycles at an assumed 2.4 GHz, per SIMD: for the vector kinds per 64-lane step of one chain "
            "(and per instruction of it), for the matrix kinds per v_mfma_f32_32x32x16_bf16 with the given "
            "number of independent v_fma_f32 per 8 of them.", "",
            "| vector work | waves/SIMD | cycles per 64 elements | per instruction |", "|---|---|---|---|"]
    text += [f"| {r['what']} | {r['waves_per_simd']} | {r['cycles_per_element_group']} | {r['cycles_per_instruction']} |"
             for r in rec["vector"]]
    text += ["", "| fmas per 8 MFMA | waves/SIMD | cycles per MFMA |", "|---|---|---|"]
    text += [f"| {r['fmas_per_8_mfma']} | {r['waves_per_simd']} | {r['cycles_per_mfma']} |" for r in rec["mfma"]]
    text += ["", "```json", json.dumps(rec, indent=1), "```", ""]
    os.makedirs(args.out, exist_ok=True)
    dst = os.path.join(args.out, "isa_rates.md")
    with open(dst, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {dst}", flush=True)


def do_resources(args) -> None:
    src = os.path.join(ROOT, "conv_bn_silu_amd", "libconv_bn_silu.resources.txt")
    if not os.path.exists(src):
        raise SystemExit("no resource report: run python3 conv_bn_silu_amd/build.py first")
    rows = [l.split() for l in open(src) if l.strip() and not l.startswith("#")]
    filt = "c++filt"
    names = subprocess.run([filt], input="\n".join(r[0] for r in rows), capture_output=True, text=True,
                           check=True).stdout.splitlines()
    text = ["# Kernel resources (compiler report)", "", "Command (from the repository root, no GPU needed):", "",
            "```", "python3 conv_bn_silu_amd/build.py && python3 bench_profile.py resources", "```", "",
            "Per kernel instantiation, from hipcc's `-Rpass-analysis=kernel-resource-usage` remarks for gfx950 "
            "(the build fails if any kernel needs scratch): VGPRs, AGPRs, scratch bytes per lane, LDS bytes "
            "per workgroup, waves per SIMD the registers and LDS allow.", "",
            "| kernel | VGPR | AGPR | scratch | LDS | waves/SIMD |", "|---|---|---|---|---|---|"]
    for r, n in zip(rows, names):
        short = n.replace("cbs::(anonymous namespace)::", "").split("(")[0]
        text.append(f"| `{short}` | {r[1]} | {r[2]} | {r[3]} | {r[4]} | {r[5]} |")
    os.makedirs(args.out, exist_ok=True)
    dst = os.path.join(args.out, "kernel_resources.md")
    with open(dst, "w") as f:
        f.write("\n".join(text) + "\n")
    print(f"[profile] wrote {dst}", flush=True)


def do_dispatch(args) -> None:
    cmd = ["python3", "bench.py", "--variants", "--no-cpu-baseline"]
    print("[profile] " + " ".join(cmd), flush=True)
    p = subprocess.run(["timeout", "-s", "KILL", "900"] + cmd, cwd=ROOT, stdout=subprocess.PIPE, text=True)
    if p.returncode not in (0, 3):
        raise SystemExit(f"bench.py failed with status {p.returncode}")
    d = last_json(p.stdout)["dispatch"]
    text = ["# Dispatch check: AUTO against every variant, fused conv+BN+SiLU", "",
            "Command (from the repository root, on one MI355X):", "", "```", " ".join(cmd), "```", "",
            "Every variant that supports each shape, timed (kernel microseconds per launch, HIP events over the "
            "timed region, after a short untimed settle); the five workloads first, then shapes on both sides of "
            "each dispatch rule (bench.py DISPATCH_SWEEP).  bench.py exits with status 3 when AUTO's pick is more "
            "than 5% slower than the fastest variant on any shape.", "",
            "| shape | N x C_in x H x W -> C_out, filter | variants (us, fastest first) | AUTO picks | AUTO / fastest |",
            "|---|---|---|---|---|"]
    for c in d["shapes"]:
        N, C_in, H, W, C_out, KH, KW, st, pad, dt = c["shape"]
        var = ", ".join(f"{k} {v:.1f}" for k, v in sorted(c["variants_us"].items(), key=lambda kv: kv[1]))
        text.append(f"| {c['name']} | {N}x{C_in}x{H}x{W} -> {C_out}, {KH}x{KW} s{st} p{pad}, "
                    f"{'bf16' if dt else 'fp32'} | {var} | {c['auto_picks']} | {c['auto_over_fastest']} |")
    text += ["", f"Worst AUTO / fastest: {d['worst_auto_over_fastest']} (within 5%: {d['auto_within_5pct']}).", ""]
    os.makedirs(args.out, exist_ok=True)
    dst = os.path.join(args.out, "dispatch_sweep.md")
    with open(dst, "w") as f:
        f.write("\n".join(text))
    print(f"[profile] wrote {dst}", flush=True)
    if not d["auto_within_5pct"]:
        raise SystemExit(3)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("mode", choices=["trace", "traffic", "mfma", "stalls", "lds", "isa", "resources", "dispatch", "all", "lds-child",
                                         "isa-child"])
    ap.add_argument("--cases", default="", help=argparse.SUPPRESS)
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
    elif args.mode == "lds":
        do_lds(args)
    elif args.mode == "isa":
        do_isa(args)
    elif args.mode == "resources":
        do_resources(args)
    elif args.mode == "dispatch":
        do_dispatch(args)
    elif args.mode == "lds-child":
        lds_child(args.cases)
    elif args.mode == "isa-child":
        isa_child()
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
        do_lds(args)
        do_isa(args)
        do_resources(args)


if __name__ == "__main__":
    main()
