"""Thin ctypes binding over ``libconv_bn_silu.so`` (C ABI in
``include/conv_bn_silu.h``).

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory (tensor data
pointers) and the current HIP stream.  If the shared library is missing the
import fails: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

# torch must be imported before the library is loaded: torch ships its own
# HIP runtime, and the library has to bind to that same runtime, or the
# process would hold two HIP runtimes and torch's streams and allocations
# would be foreign to the library's.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libconv_bn_silu.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_DEVICE, ERR_HIP, ERR_BAD_HANDLE = range(6)
DTYPE_F32, DTYPE_BF16 = 0, 1
VARIANTS = {"auto": 0, "gemm_gather": 1, "gemm_window": 2, "pointwise": 3, "small_k": 4, "scalar": 5,
            "gemm_window32": 6, "strided_rows": 7}

# Every symbol include/conv_bn_silu.h declares; the CPU tests check the
# library exports each.
EXPORTS = [
    "conv_bn_silu_create", "conv_bn_silu_destroy", "conv_bn_silu_run", "conv_bn_silu_run_variant",
    "conv_bn_silu_run_unfused", "conv_bn_silu_run_unfused_noalloc", "conv_bn_silu_output_hw", "conv_bn_silu_validate",
    "conv_bn_silu_select_variant", "conv_bn_silu_variant_supports", "conv_bn_silu_status_string",
    "conv_bn_silu_variant_name", "conv_bn_silu_last_hip_error", "conv_bn_silu_fold_bn",
]
# Measurement support (include/conv_bn_silu_bench.h).
BENCH_EXPORTS = [
    "conv_bn_silu_bench_device_info", "conv_bn_silu_bench_mfma", "conv_bn_silu_bench_mfma_flops",
    "conv_bn_silu_bench_copy", "conv_bn_silu_bench_lds", "conv_bn_silu_bench_isa",
]


class CbsError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        msg = f"{what}: {status_string(status)} (status {status})"
        if hip_error:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          f"python conv_bn_silu_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i, cp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int, ctypes.c_char_p
    ip = ctypes.POINTER(ctypes.c_int)
    geo = [i] * 10  # N, C_in, H, W, C_out, KH, KW, stride, pad, dtype
    lib.conv_bn_silu_create.argtypes = [ctypes.POINTER(vp)]
    lib.conv_bn_silu_destroy.argtypes = [vp]
    lib.conv_bn_silu_run.argtypes = [vp, vp, vp, vp, vp, vp] + geo + [vp]
    lib.conv_bn_silu_run_variant.argtypes = [vp, i, vp, vp, vp, vp, vp] + geo + [vp]
    lib.conv_bn_silu_run_unfused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp] + geo + [vp]
    lib.conv_bn_silu_run_unfused_noalloc.argtypes = [vp, vp, vp, vp, vp, vp] + geo + [vp]
    lib.conv_bn_silu_output_hw.argtypes = [i] * 6 + [ip, ip]
    lib.conv_bn_silu_validate.argtypes = [vp, vp, vp, vp, vp] + geo
    lib.conv_bn_silu_select_variant.argtypes = geo + [i]
    lib.conv_bn_silu_variant_supports.argtypes = [i] + geo
    lib.conv_bn_silu_status_string.argtypes = [i]
    lib.conv_bn_silu_status_string.restype = cp
    lib.conv_bn_silu_variant_name.argtypes = [i]
    lib.conv_bn_silu_variant_name.restype = cp
    lib.conv_bn_silu_last_hip_error.argtypes = [vp]
    lib.conv_bn_silu_fold_bn.argtypes = [fp, fp, fp, fp, ctypes.c_float, fp, i, fp, fp]
    for name in EXPORTS:
        if name not in ("conv_bn_silu_status_string", "conv_bn_silu_variant_name"):
            getattr(lib, name).restype = i
    lib.conv_bn_silu_bench_device_info.argtypes = [ip, ip, ip]
    lib.conv_bn_silu_bench_device_info.restype = i
    lib.conv_bn_silu_bench_mfma.argtypes = [i, i, vp, vp]
    lib.conv_bn_silu_bench_mfma.restype = i
    lib.conv_bn_silu_bench_mfma_flops.argtypes = [i, i]
    lib.conv_bn_silu_bench_mfma_flops.restype = ctypes.c_int64
    lib.conv_bn_silu_bench_copy.argtypes = [vp, vp, ctypes.c_uint64, vp]
    lib.conv_bn_silu_bench_copy.restype = i
    lib.conv_bn_silu_bench_lds.argtypes = [i, vp, vp, vp]
    lib.conv_bn_silu_bench_lds.restype = i
    lib.conv_bn_silu_bench_isa.argtypes = [i, i, i, vp, vp]
    lib.conv_bn_silu_bench_isa.restype = i
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.conv_bn_silu_status_string(int(status)).decode()


def variant_name(variant: int) -> str:
    return lib.conv_bn_silu_variant_name(int(variant)).decode()


def output_hw(H, W, KH, KW, stride, pad):
    oh, ow = ctypes.c_int(), ctypes.c_int()
    rc = lib.conv_bn_silu_output_hw(H, W, KH, KW, stride, pad, ctypes.byref(oh), ctypes.byref(ow))
    if rc != OK:
        raise CbsError(rc, "conv_bn_silu_output_hw")
    return oh.value, ow.value


def select_variant(N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, num_cu=256) -> int:
    return lib.conv_bn_silu_select_variant(N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, num_cu)


def variant_supports(variant, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype) -> bool:
    return bool(lib.conv_bn_silu_variant_supports(variant, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype))


def validate(x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype) -> int:
    """The host-side argument checks on raw integer addresses; returns a status."""
    return lib.conv_bn_silu_validate(x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype)


def fold_bn(gamma, beta, mean, var, eps, conv_bias=None):
    """Fold batch-norm statistics into (scale, bias), as float32 numpy arrays."""
    import numpy as np
    arrs = [np.ascontiguousarray(a, dtype=np.float32) for a in (gamma, beta, mean, var)]
    C = arrs[0].size
    cb = None if conv_bias is None else np.ascontiguousarray(conv_bias, dtype=np.float32)
    scale = np.empty(C, np.float32)
    bias = np.empty(C, np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    as_fp = lambda a: a.ctypes.data_as(fp)
    rc = lib.conv_bn_silu_fold_bn(*(as_fp(a) for a in arrs), ctypes.c_float(eps),
                                  None if cb is None else as_fp(cb), C, as_fp(scale), as_fp(bias))
    if rc != OK:
        raise CbsError(rc, "conv_bn_silu_fold_bn")
    return scale, bias


class Library:
    """One handle on the current device (conv_bn_silu_create/destroy).  The
    handle is read-only after creation: one may serve every stream and
    thread of the process."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = lib.conv_bn_silu_create(ctypes.byref(h))
        if rc != OK:
            raise CbsError(rc, "conv_bn_silu_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib.conv_bn_silu_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc, what):
        if rc != OK:
            raise CbsError(rc, what, lib.conv_bn_silu_last_hip_error(self.handle))

    def run_ptr(self, variant, x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype, stream):
        """Raw-pointer call of conv_bn_silu_run_variant (variant 0 = AUTO)."""
        self._check(lib.conv_bn_silu_run_variant(self.handle, variant, x, w, scale, bias, y, N, C_in, H, W,
                                                 C_out, KH, KW, stride, pad, dtype, stream),
                    "conv_bn_silu_run_variant")

    def run_unfused_noalloc_ptr(self, x, w, scale, bias, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype,
                                stream):
        self._check(lib.conv_bn_silu_run_unfused_noalloc(self.handle, x, w, scale, bias, y, N, C_in, H, W, C_out,
                                                         KH, KW, stride, pad, dtype, stream),
                    "conv_bn_silu_run_unfused_noalloc")

    def run_unfused_ptr(self, x, w, scale, bias, t1, t2, y, N, C_in, H, W, C_out, KH, KW, stride, pad, dtype,
                        stream):
        self._check(lib.conv_bn_silu_run_unfused(self.handle, x, w, scale, bias, t1, t2, y, N, C_in, H, W,
                                                 C_out, KH, KW, stride, pad, dtype, stream),
                    "conv_bn_silu_run_unfused")


_default = None


def default_library() -> Library:
    global _default
    if _default is None:
        _default = Library()
    return _default


def _geometry(x, w, scale, bias, stride, pad):
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16) or w.dtype != x.dtype:
        raise TypeError("x and w must both be float32 or both bfloat16")
    if scale.dtype != torch.float32 or bias.dtype != torch.float32:
        raise TypeError("scale and bias must be float32")
    for t in (x, w, scale, bias):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
        if t.device != x.device:
            raise ValueError("all tensors must be on x's device")
    N, C_in, H, W = x.shape
    C_out, C_in_w, KH, KW = w.shape
    if C_in_w != C_in or scale.numel() != C_out or bias.numel() != C_out:
        raise ValueError("inconsistent shapes")
    OH, OW = output_hw(H, W, KH, KW, stride, pad)
    dtype = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    return (N, C_in, H, W, C_out, KH, KW, stride, pad, dtype), (N, C_out, OH, OW)


def _check_output(t, x, yshape, what):
    """An output buffer the kernels may write: x's device, dtype, the output
    shape, contiguous."""
    if not t.is_cuda or t.device != x.device:
        raise ValueError(f"{what} must be a device tensor on x's device")
    if tuple(t.shape) != yshape or t.dtype != x.dtype or not t.is_contiguous():
        raise ValueError(f"{what} has the wrong shape, dtype or layout")


def conv_bn_silu(x, w, scale, bias, stride: int = 1, pad: int = 0, out=None, variant: str = "auto",
                 library: Library | None = None):
    """y = SiLU(conv2d(x, w) * scale[co] + bias[co]) on the current stream.

    x: NCHW, w: OIHW, both float32 or both bfloat16; scale, bias: float32
    [C_out]; all contiguous on the device.  Returns y (NCHW, dtype of x).
    """
    import torch
    geo, yshape = _geometry(x, w, scale, bias, stride, pad)
    y = torch.empty(yshape, dtype=x.dtype, device=x.device) if out is None else out
    _check_output(y, x, yshape, "out")
    lib_ = library or default_library()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    lib_.run_ptr(VARIANTS[variant], x.data_ptr(), w.data_ptr(), scale.data_ptr(), bias.data_ptr(),
                 y.data_ptr(), *geo, stream)
    return y


def conv_bn_silu_unfused(x, w, scale, bias, stride: int = 1, pad: int = 0, library: Library | None = None,
                         out=None):
    """The three-kernel sequence conv -> BN -> SiLU with t1, t2 in memory;
    returns (y, t1, t2).  `out`, if given, is a tuple (y, t1, t2) of buffers
    to write."""
    import torch
    geo, yshape = _geometry(x, w, scale, bias, stride, pad)
    if out is None:
        y, t1, t2 = (torch.empty(yshape, dtype=x.dtype, device=x.device) for _ in range(3))
    else:
        y, t1, t2 = out
        for t, name in ((y, "y"), (t1, "t1"), (t2, "t2")):
            _check_output(t, x, yshape, name)
    lib_ = library or default_library()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    lib_.run_unfused_ptr(x.data_ptr(), w.data_ptr(), scale.data_ptr(), bias.data_ptr(), t1.data_ptr(),
                         t2.data_ptr(), y.data_ptr(), *geo, stream)
    return y, t1, t2


def conv_bn_silu_unfused_noalloc(x, w, scale, bias, stride: int = 1, pad: int = 0, out=None,
                                 library: Library | None = None):
    """The unfused sequence with its intermediates in the library's static
    device scratch (conv_bn_silu_run_unfused_noalloc); returns y.  With
    `out` given, nothing is allocated."""
    import torch
    geo, yshape = _geometry(x, w, scale, bias, stride, pad)
    y = torch.empty(yshape, dtype=x.dtype, device=x.device) if out is None else out
    _check_output(y, x, yshape, "out")
    lib_ = library or default_library()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    lib_.run_unfused_noalloc_ptr(x.data_ptr(), w.data_ptr(), scale.data_ptr(), bias.data_ptr(), y.data_ptr(),
                                 *geo, stream)
    return y
