"""Helpers for the GPU tests: upload seeded inputs, compare with the oracle
under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

from conv_bn_silu_amd import synth


def say(*a):
    """Name the case on stdout before the GPU runs it (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def upload(inp: synth.Inputs):
    import torch
    dev = torch.device("cuda", 0)
    if inp.wl.dtype == synth.DTYPE_BF16:
        x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        w = torch.from_numpy(inp.w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(inp.x).to(dev)
        w = torch.from_numpy(inp.w).to(dev)
    return x, w, torch.from_numpy(inp.scale).to(dev), torch.from_numpy(inp.bias).to(dev)


def to_f64(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> float64 numpy, exactly."""
    return t.float().cpu().numpy().astype(np.float64)


def tolerance(ref: np.ndarray, dtype: int) -> np.ndarray:
    """Stated tolerances: fp32 |err| <= 1e-4*(1+|ref|); bf16 |err| <= 1.6e-2*|ref| + 1e-3."""
    if dtype == synth.DTYPE_F32:
        return 1e-4 * (1.0 + np.abs(ref))
    return 1.6e-2 * np.abs(ref) + 1e-3


def check(got: np.ndarray, ref: np.ndarray, dtype: int, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    tol = tolerance(ref, dtype)
    ratio = np.where(np.isfinite(got), err / tol, np.inf)
    worst = int(np.argmax(ratio)) if ratio.size else 0
    bad = int(np.count_nonzero(ratio > 1.0))
    assert bad == 0, (f"{what}: {bad} of {ratio.size} outside tolerance; worst at flat index {worst}: "
                      f"got {got.ravel()[worst]!r} ref {ref.ravel()[worst]!r} ratio {ratio.ravel()[worst]:.3g}")
    return float(ratio.max()) if ratio.size else 0.0


def oracle_full(inp: synth.Inputs) -> np.ndarray:
    import oracle
    wl = inp.wl
    return oracle.get().forward(inp.x, inp.w, inp.scale, inp.bias, wl.stride, wl.pad)
