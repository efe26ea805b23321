"""Compile the HIP library ``libconv_bn_silu.so`` for gfx950 (in-tree).

Every ``csrc/*.hip`` and ``csrc/*.cpp`` is compiled by hipcc to its own object
(in parallel) and linked into one shared library next to this file.  All HIP
code is compiled without packed-fp32 instructions.

The compiler's per-kernel resource report (registers, LDS, scratch) is written
to ``libconv_bn_silu.resources.txt`` beside the library, and the build fails if
a kernel needs scratch memory: register spills or an array the compiler could
not keep in registers turn the kernel's hot loop into memory traffic (one such
kernel ran six times slower than without), so they are treated as errors.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libconv_bn_silu.so")
RESOURCES = os.path.join(HERE, "libconv_bn_silu.resources.txt")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(HERE, "..", "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"LDS Size \[bytes/block\]|VGPRs Spill|SGPRs Spill):\s*(\S+)")


def parse_resources(text: str) -> list[dict]:
    """Per-kernel records from hipcc's kernel-resource-usage remarks."""
    out: list[dict] = []
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            out.append({"kernel": val})
        elif out:
            out[-1][key.split(" [")[0]] = int(val)
    return out


def _compile(src: str, extra: list[str]) -> tuple[str, list[dict]]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + extra + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # print only other diagnostics (not the resource remarks either).
    other = [l for l in res.stderr.splitlines()
             if "packed-fp32-ops" not in l and "-Rpass-analysis=kernel-resource-usage" not in l]
    if other:
        sys.stderr.write("\n".join(other) + "\n")
    return obj, parse_resources(res.stderr)


def build(extra: list[str] | None = None, jobs: int = 8) -> str:
    """Compile and link; returns the path of the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(lambda s: _compile(s, extra), sources()))
    objs = [o for o, _ in done]
    kernels = [k for _, ks in done for k in ks]
    with open(RESOURCES, "w") as f:
        f.write("# kernel  VGPRs  AGPRs  scratch_bytes_per_lane  LDS_bytes  waves_per_SIMD\n")
        for k in kernels:
            f.write(f"{k['kernel']}  {k.get('VGPRs')}  {k.get('AGPRs')}  {k.get('ScratchSize')}  "
                    f"{k.get('LDS Size')}  {k.get('Occupancy')}\n")
    spilling = [k["kernel"] for k in kernels if k.get("ScratchSize", 0) or k.get("VGPRs Spill", 0)]
    if spilling:
        raise RuntimeError("kernels using scratch memory: " + ", ".join(spilling))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
