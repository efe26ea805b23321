"""Seeded synthetic inputs for the fused conv2d + BN + SiLU operator.

This module holds the workload definitions and the random draws only -- none
of the operator's arithmetic.  Both sides of every parity check (the HIP path
and the CPU oracle) take their inputs from here, and nothing else is shared
between them.  It imports neither side.

Recipe (the same for every workload):
  * generator: numpy ``Generator(PCG64(seed))``; draws in the order
    x, w, scale, bias, each in float32;
  * x: U[-1, 1], N(0, 1) or U[0, 1] ("image-like") per workload;
  * w: N(0, 1/fan_in) with fan_in = C_in*KH*KW, the second argument read as a
    variance (std = 1/sqrt(fan_in));
  * scale ~ U[0.5, 1.5]; bias ~ N(0, 0.1), again a variance (std = sqrt(0.1));
  * bf16 workloads round x and w to bfloat16 with round-to-nearest-even, and
    both sides consume exactly those rounded values; scale and bias stay fp32.
"""
from __future__ import annotations

import dataclasses
import hashlib
import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: int  # DTYPE_F32 or DTYPE_BF16 for x, w and y
    N: int
    C_in: int
    H: int
    W: int
    C_out: int
    KH: int
    KW: int
    stride: int
    pad: int
    x_dist: str  # "u11" = U[-1,1], "n01" = N(0,1), "u01" = U[0,1]
    seed: int

    @property
    def OH(self) -> int:
        return (self.H + 2 * self.pad - self.KH) // self.stride + 1

    @property
    def OW(self) -> int:
        return (self.W + 2 * self.pad - self.KW) // self.stride + 1

    @property
    def M(self) -> int:
        return self.N * self.OH * self.OW

    @property
    def K(self) -> int:
        return self.C_in * self.KH * self.KW

    @property
    def flops(self) -> int:
        """Conv multiply-adds counted as 2 flops: 2*M*C_out*K."""
        return 2 * self.M * self.C_out * self.K

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DTYPE_F32 else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Read x once, read w once, write y once, read fp32 scale and bias."""
        e = self.elem_bytes
        return (self.N * self.C_in * self.H * self.W * e + self.C_out * self.K * e
                + self.N * self.C_out * self.OH * self.OW * e + 8 * self.C_out)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five seeded YOLO-shaped layers (sizes as given in the workload
# descriptions; seeds 1000 + index).
WORKLOADS = {
    "c1": Workload("fp32_3x3_s1_p1_n1_16to32_32x32", DTYPE_F32, 1, 16, 32, 32, 32, 3, 3, 1, 1, "u11", 1001),
    "c2": Workload("bf16_1x1_s1_n8_256to256_80x80", DTYPE_BF16, 8, 256, 80, 80, 256, 1, 1, 1, 0, "n01", 1002),
    "c3": Workload("bf16_3x3_s2_p1_n16_64to128_320to160", DTYPE_BF16, 16, 64, 320, 320, 128, 3, 3, 2, 1, "n01", 1003),
    "c4": Workload("bf16_stem_3x3_s2_p1_n32_3to16_640to320", DTYPE_BF16, 32, 3, 640, 640, 16, 3, 3, 2, 1, "u01", 1004),
    "c5": Workload("bf16_3x3_s1_p1_n64_512to512_20x20", DTYPE_BF16, 64, 512, 20, 20, 512, 3, 3, 1, 1, "n01", 1005),
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they encode (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: np.ndarray       # float32 values (bf16-exact for bf16 workloads), NCHW
    w: np.ndarray       # float32 values (bf16-exact for bf16 workloads), OIHW
    scale: np.ndarray   # float32 [C_out]
    bias: np.ndarray    # float32 [C_out]
    x_bits: np.ndarray | None = None  # uint16 bf16 patterns, bf16 workloads only
    w_bits: np.ndarray | None = None

    def digest(self) -> str:
        """SHA-256 over the four arrays exactly as both sides consume them."""
        h = hashlib.sha256()
        for a in (self.x_bits if self.x_bits is not None else self.x,
                  self.w_bits if self.w_bits is not None else self.w,
                  self.scale, self.bias):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def _draw_x(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "n01":
        return rng.standard_normal(shape, dtype=np.float32)
    u = rng.random(shape, dtype=np.float32)
    if dist == "u01":
        return u
    if dist == "u11":
        return u * np.float32(2.0) - np.float32(1.0)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(wl: Workload, seed: int | None = None) -> Inputs:
    """Draw x, w, scale, bias for a workload (seed defaults to the workload's)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    x = _draw_x(rng, wl.x_dist, (wl.N, wl.C_in, wl.H, wl.W))
    fan_in = wl.C_in * wl.KH * wl.KW
    w = rng.standard_normal((wl.C_out, wl.C_in, wl.KH, wl.KW), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(fan_in))
    scale = rng.random(wl.C_out, dtype=np.float32) + np.float32(0.5)
    bias = rng.standard_normal(wl.C_out, dtype=np.float32) * np.float32(np.sqrt(0.1))
    if wl.dtype == DTYPE_BF16:
        xb, wb = bf16_bits(x), bf16_bits(w)
        return Inputs(wl, bf16_to_f32(xb), bf16_to_f32(wb), scale, bias, xb, wb)
    return Inputs(wl, x, w, scale, bias)
