"""CPU oracle for the fused conv2d + folded BatchNorm + SiLU operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``conv_bn_silu_amd``) never imports, links or calls it, and this package
imports nothing from the product.

What it computes (page "Fusing an Epilogue", section "The problem"): the
unfused sequence conv -> batchnorm -> silu, each pass materialising its own
fp64 array (t1, t2, y).  The arithmetic lives in ``cbs_oracle.c`` (plain C,
fp64, OpenMP over output planes); this module only compiles it and marshals
numpy arrays into it.

Pins: every function here is pinned by CPU tests (``tests/test_oracle_*.py``)
to things other than itself -- a library convolution, closed forms of SiLU,
delta and all-ones inputs, identity weights, linearity, stride/pad
equivalences, a hand-checkable integer example under ``tests/golden/`` -- and
the suite builds deliberately broken variants of the C file (``mutant=k``)
and checks that the pins reject each one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cbs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcbs_oracle.so")

_lib = None


def build(out_path: str | None = None, mutant: int = 0) -> str:
    """Compile the C oracle with gcc (OpenMP, fp64, no FMA contraction).

    ``mutant`` > 0 builds a deliberately wrong variant for the pin tests.
    Returns the path of the shared object.
    """
    out = out_path or _LIB_PATH
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-Wall", "-o", out, _SRC, "-lm"]
    if mutant:
        cmd.insert(1, f"-DCBS_ORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes view of one build of ``cbs_oracle.c``."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        d, i, l = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
        lib.cbs_oracle_out_dim.argtypes = [i, i, i, i]
        lib.cbs_oracle_out_dim.restype = i
        lib.cbs_oracle_conv.argtypes = [d, d, d] + [i] * 10
        lib.cbs_oracle_conv.restype = i
        lib.cbs_oracle_bn.argtypes = [d, d, d, d, i, i, l]
        lib.cbs_oracle_bn.restype = None
        lib.cbs_oracle_silu.argtypes = [d, d, l]
        lib.cbs_oracle_silu.restype = None
        lib.cbs_oracle_points.argtypes = [d, d, d, d, d, l, d] + [i] * 9
        lib.cbs_oracle_points.restype = i
        self._lib = lib

    # -- shapes ---------------------------------------------------------------
    def out_dim(self, n_in: int, k: int, stride: int, pad: int) -> int:
        """OH = floor((H + 2p - KH)/s) + 1, or -1 if the window does not fit."""
        return int(self._lib.cbs_oracle_out_dim(n_in, k, stride, pad))

    # -- the three passes -----------------------------------------------------
    def conv(self, x, w, stride: int, pad: int, nthreads: int = 0) -> np.ndarray:
        """Pass 1, the convolution x -> t1: cross-correlation, zero pad."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        N, C_in, H, W = x.shape
        C_out, C_in_w, KH, KW = w.shape
        if C_in_w != C_in:
            raise ValueError("w and x disagree on C_in")
        OH, OW = self.out_dim(H, KH, stride, pad), self.out_dim(W, KW, stride, pad)
        if OH < 1 or OW < 1:
            raise ValueError("empty output")
        t1 = np.empty((N, C_out, OH, OW), dtype=np.float64)
        rc = self._lib.cbs_oracle_conv(x.ctypes.data, w.ctypes.data, t1.ctypes.data,
                                       N, C_in, H, W, C_out, KH, KW, stride, pad, nthreads)
        if rc != 0:
            raise ValueError("invalid shape")
        return t1

    def bn(self, t1, scale, bias) -> np.ndarray:
        """Pass 2, batch norm t1 -> t2: t1*scale[co] + bias[co]."""
        t1 = np.ascontiguousarray(t1, dtype=np.float64)
        scale = np.ascontiguousarray(scale, dtype=np.float64)
        bias = np.ascontiguousarray(bias, dtype=np.float64)
        N, C_out, OH, OW = t1.shape
        t2 = np.empty_like(t1)
        self._lib.cbs_oracle_bn(t1.ctypes.data, scale.ctypes.data, bias.ctypes.data,
                                t2.ctypes.data, N, C_out, OH * OW)
        return t2

    def silu(self, t2) -> np.ndarray:
        """Pass 3, SiLU t2 -> y: v * sigmoid(v)."""
        t2 = np.ascontiguousarray(t2, dtype=np.float64)
        y = np.empty_like(t2)
        self._lib.cbs_oracle_silu(t2.ctypes.data, y.ctypes.data, t2.size)
        return y

    def forward(self, x, w, scale, bias, stride: int, pad: int, nthreads: int = 0) -> np.ndarray:
        """The unfused three-pass sequence; returns y in fp64."""
        return self.silu(self.bn(self.conv(x, w, stride, pad, nthreads), scale, bias))

    def points(self, x, w, scale, bias, stride: int, pad: int, idx) -> np.ndarray:
        """The same three steps for selected flat NCHW output indices only."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        scale = np.ascontiguousarray(scale, dtype=np.float64)
        bias = np.ascontiguousarray(bias, dtype=np.float64)
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        N, C_in, H, W = x.shape
        C_out, _, KH, KW = w.shape
        y = np.empty(idx.shape, dtype=np.float64)
        rc = self._lib.cbs_oracle_points(x.ctypes.data, w.ctypes.data, scale.ctypes.data,
                                         bias.ctypes.data, idx.ctypes.data, idx.size,
                                         y.ctypes.data, N, C_in, H, W, C_out, KH, KW,
                                         stride, pad)
        if rc != 0:
            raise ValueError("invalid shape or index")
        return y


def get() -> Oracle:
    """The correct oracle, compiled on first use if no build is present."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = Oracle(_LIB_PATH)
    return _lib
