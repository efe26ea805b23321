"""The measurement side without a GPU: counter parsing of the rocprofv3
harness, the roofline bound and fraction of each workload, and bench.py's
refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bench_profile  # noqa: E402
from conv_bn_silu_amd import synth  # noqa: E402

pytestmark = pytest.mark.cpu


def write_counters(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=cols)
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(cols, r)))


def test_counter_rows_of_a_dispatch_are_combined(tmp_path):
    p = str(tmp_path / "c.csv")
    write_counters(p, [
        (1, "cbs::k", "FETCH_SIZE", 10.0, 0, 100), (1, "cbs::k", "FETCH_SIZE", 5.0, 0, 100),
        (2, "cbs::k", "FETCH_SIZE", 7.0, 200, 300), (2, "cbs::k", "FETCH_SIZE", 9.0, 200, 300),
        (3, "copyBuffer", "FETCH_SIZE", 1000.0, 400, 500),
        (1, "cbs::k", "WRITE_SIZE", 3.0, 0, 100),
    ])
    summed = bench_profile.counter_by_kernel(p, "FETCH_SIZE", lambda k: "cbs" in k)
    assert summed == {"cbs::k": [15.0, 16.0]}
    largest = bench_profile.counter_by_kernel(p, "FETCH_SIZE", lambda k: "cbs" in k, max)
    assert largest == {"cbs::k": [10.0, 9.0]}
    assert bench_profile.mean(summed["cbs::k"]) == 15.5


def test_counter_parsing_refuses_a_missing_counter(tmp_path):
    p = str(tmp_path / "c.csv")
    write_counters(p, [(1, "cbs::k", "FETCH_SIZE", 1.0, 0, 1)])
    with pytest.raises(SystemExit):
        bench_profile.counter_by_kernel(p, "WRITE_SIZE", lambda k: True)


@pytest.mark.parametrize("key,bound", [("c1", "mfma"), ("c2", "hbm"), ("c3", "hbm"), ("c4", "hbm"),
                                       ("c5", "mfma")])
def test_roofline_bound_per_workload(key, bound):
    # bound = MFMA when FLOP / peak exceeds algorithmic bytes / 8 TB/s; c1 is
    # fp32 and priced against the fp32 matrix peak.
    assert bench.roofline_bound(synth.WORKLOADS[key]) == bound


def test_roofline_fraction_is_achieved_over_peak():
    wl = synth.WORKLOADS["c2"]
    seconds = wl.algorithmic_bytes / 4000e9  # exactly half of the 8 TB/s peak
    r = bench.roofline(wl, seconds)
    assert r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 4000.0) < 0.01 and abs(r["frac"] - 0.5) < 1e-4
    wl5 = synth.WORKLOADS["c5"]
    r5 = bench.roofline(wl5, wl5.flops / 1250e12)
    assert r5["unit"] == "TFLOP/s" and abs(r5["frac"] - 0.5) < 1e-4


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_traffic_records_are_tied_to_one_kernel_source():
    # the digest covers the variant's own kernel file and the shared device
    # headers only: editing another kernel leaves a record valid
    d = {v: bench.kernel_sources_digest(v) for v in bench.VARIANT_SOURCES}
    assert len(set(d.values())) == len(d)
    assert all(len(x) == 16 for x in d.values())


def test_layer_entry_fractions():
    wl = synth.WORKLOADS["c5"]
    kern = wl.flops / 1250e12  # half the bf16 peak
    q = {"wl": wl, "variant": "gemm_window32", "kernel_s": kern, "wall_per_step_s": kern * 1.01,
         "roofline": bench.roofline(wl, kern), "tflops_kernel": wl.flops / kern / 1e12,
         "hbm_gbs_alg": wl.algorithmic_bytes / kern / 1e9}
    e = bench.layer_entry(q, {"copy_gbs": 5000.0, "mfma_bf16_tflops": 2000.0})
    assert e["bound"] == "mfma" and abs(e["frac"] - 0.5) < 1e-4 and abs(e["mfma_frac"] - 0.5) < 1e-4
    assert abs(e["frac_of_mfma_ceiling"] - 0.625) < 1e-4
    assert e["kernel_us"] <= e["wall_us_per_step"]


def test_dispatch_sweep_shapes_are_valid():
    from conv_bn_silu_amd import binding as B
    for g in bench.DISPATCH_SWEEP:
        assert B.select_variant(*g[:10]) in range(1, 8), g


def test_lds_probe_cases_fit_the_probe():
    """Every LDS-probe address pattern stays inside the probe's 64 KiB array,
    is aligned for its operation and names one of the five operations."""
    import bench_profile as bp
    cases = bp.lds_cases()
    assert len({n for n, _, _ in cases}) == len(cases)
    for name, op, addrs in cases:
        assert op in (0, 1, 2, 3, 4), name
        assert len(addrs) == 64, name
        align = 16 if op in (0, 4) else 8
        assert all(0 <= a < 65536 - 16 and a % align == 0 for a in addrs), name
