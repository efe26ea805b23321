"""MI355X-native fused conv2d + folded BatchNorm + SiLU.

The operator runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/conv_bn_silu.h``, built into ``libconv_bn_silu.so`` next to this
file).  ``binding`` is a thin ctypes layer over that ABI; PyTorch supplies
device memory and streams only.  The binding is imported lazily so that the
input generator (``synth``) can be used without the shared library.
"""
from __future__ import annotations

import importlib

__all__ = ["conv_bn_silu", "conv_bn_silu_unfused", "fold_bn", "binding", "synth"]


def __getattr__(name):
    if name in ("binding", "synth"):
        return importlib.import_module(f"{__name__}.{name}")
    if name in ("conv_bn_silu", "conv_bn_silu_unfused", "fold_bn", "Library"):
        return getattr(importlib.import_module(f"{__name__}.binding"), name)
    raise AttributeError(name)
