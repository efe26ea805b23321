"""The C ABI without a GPU: the library loads, exports everything the header
declares, and its host-side logic (validation, output size, dispatch, status
strings, batch-norm folding, handle checks) behaves as documented.  No call
here reaches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

from conv_bn_silu_amd import binding as B
from conv_bn_silu_amd import synth

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions(header=None):
    """Functions declared in include/*.h (or in one header)."""
    names = set()
    for h in ([header] if header else sorted(os.listdir(os.path.join(ROOT, "include")))):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(conv_bn_silu_\w+)\s*\(", text))
    return sorted(names)


def test_header_and_binding_agree():
    assert declared_functions("conv_bn_silu.h") == sorted(B.EXPORTS)
    assert declared_functions("conv_bn_silu_bench.h") == sorted(B.BENCH_EXPORTS)
    assert declared_functions() == sorted(B.EXPORTS + B.BENCH_EXPORTS)


def test_bench_helpers_without_device():
    assert B.lib.conv_bn_silu_bench_mfma_flops(256, 10) == 256 * 4 * 10 * 8 * 2 * 32 * 32 * 16
    assert B.lib.conv_bn_silu_bench_mfma_flops(0, 10) == -1
    assert B.lib.conv_bn_silu_bench_copy(None, None, 16, None) == 1
    # the probes reject bad arguments before touching a device
    assert B.lib.conv_bn_silu_bench_lds(0, None, None, None) == 1
    assert B.lib.conv_bn_silu_bench_lds(5, 16, 16, None) == 1
    assert B.lib.conv_bn_silu_bench_lds(-1, 16, 16, None) == 1
    assert B.lib.conv_bn_silu_bench_isa(0, 256, 10, None, None) == 1
    assert B.lib.conv_bn_silu_bench_isa(7, 256, 10, 16, None) == 1
    assert B.lib.conv_bn_silu_bench_isa(0, 0, 10, 16, None) == 1
    assert B.lib.conv_bn_silu_bench_isa(0, 256, 0, 16, None) == 1


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports(name):
    assert hasattr(B.lib, name)


def test_create_without_device_reports_no_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    h = ctypes.c_void_p(1234)
    assert B.lib.conv_bn_silu_create(ctypes.byref(h)) == B.ERR_NO_DEVICE
    assert h.value is None
    assert B.lib.conv_bn_silu_create(None) == B.ERR_INVALID_ARG


def test_bad_handles():
    args = [0] * 5 + [1, 1, 4, 4, 1, 1, 1, 1, 0, B.DTYPE_F32, None]
    assert B.lib.conv_bn_silu_run(None, *args) == B.ERR_BAD_HANDLE
    assert B.lib.conv_bn_silu_run(ctypes.c_void_p(0xdeadbeef), *args) == B.ERR_BAD_HANDLE
    assert B.lib.conv_bn_silu_run_variant(None, 1, *args) == B.ERR_BAD_HANDLE
    assert B.lib.conv_bn_silu_destroy(None) == B.OK
    assert B.lib.conv_bn_silu_destroy(ctypes.c_void_p(0xdeadbeef)) == B.ERR_BAD_HANDLE
    assert B.lib.conv_bn_silu_last_hip_error(None) == 0


def test_status_and_variant_names():
    assert B.status_string(0) == "ok"
    assert B.status_string(99) == "unknown"
    assert [B.variant_name(v) for v in range(8)] == list(B.VARIANTS)
    assert B.variant_name(-1) == "unknown"


@pytest.mark.parametrize("key", sorted(synth.WORKLOADS))
def test_output_hw_matches_workloads(key):
    wl = synth.WORKLOADS[key]
    assert B.output_hw(wl.H, wl.W, wl.KH, wl.KW, wl.stride, wl.pad) == (wl.OH, wl.OW)


def test_output_hw_rejects():
    for bad in [(2, 2, 3, 3, 1, 0), (4, 4, 3, 3, 0, 1), (4, 4, 3, 3, 1, -1), (0, 4, 1, 1, 1, 0)]:
        with pytest.raises(B.CbsError):
            B.output_hw(*bad)
    assert B.output_hw(7, 9, 3, 3, 2, 1) == (4, 5)  # floor on a ragged case


# Fake device addresses: validation only compares and alignment-checks them.
BASE = 0x7F0000000000


def geo(N=2, C_in=3, H=8, W=8, C_out=4, KH=3, KW=3, stride=1, pad=1, dtype=B.DTYPE_BF16):
    return [N, C_in, H, W, C_out, KH, KW, stride, pad, dtype]


def ptrs(g, gap=1 << 30):
    return [BASE, BASE + gap, BASE + 2 * gap, BASE + 3 * gap, BASE + 4 * gap]


def test_validate_accepts_good_call():
    g = geo()
    assert B.validate(*ptrs(g), *g) == B.OK
    assert B.validate(*ptrs(g), *geo(dtype=B.DTYPE_F32)) == B.OK


@pytest.mark.parametrize("field,value", [
    (1, 0), (2, 0), (3, -1), (4, 0), (5, 0), (6, 0), (7, 0), (8, -1), (9, 2), (9, -1)])
def test_validate_rejects_bad_sizes(field, value):
    g = geo()
    g[field] = value
    assert B.validate(*ptrs(g), *g) == B.ERR_INVALID_ARG


def test_validate_rejects_window_that_does_not_fit():
    g = geo(H=2, W=8, KH=3, pad=0)
    assert B.validate(*ptrs(g), *g) == B.ERR_INVALID_ARG


def test_validate_null_pointers_and_empty_batch():
    g = geo()
    for i in range(5):
        p = ptrs(g)
        p[i] = 0
        assert B.validate(*p, *g) == B.ERR_INVALID_ARG
    g0 = geo(N=0)
    assert B.validate(0, 0, 0, 0, 0, *g0) == B.OK


def test_validate_alignment():
    # a pointer off its element size is a well-formed call the kernels do
    # not serve: unsupported, not invalid
    g = geo()
    p = ptrs(g)
    p[0] += 1  # bf16 x at an odd address
    assert B.validate(*p, *g) == B.ERR_UNSUPPORTED
    gf = geo(dtype=B.DTYPE_F32)
    p = ptrs(gf)
    p[4] += 2  # fp32 y at a 2-byte offset
    assert B.validate(*p, *gf) == B.ERR_UNSUPPORTED
    p = ptrs(g)
    p[2] += 2  # scale must be 4-byte aligned
    assert B.validate(*p, *g) == B.ERR_UNSUPPORTED
    p = ptrs(g)
    p[1] += 2  # bf16 w at a 2-byte (element) boundary is fine
    assert B.validate(*p, *g) == B.OK


def test_validate_overlap():
    g = geo()  # y = 2*4*8*8 bf16 = 1024 bytes
    p = ptrs(g)
    p[4] = p[0] + 64  # y inside x
    assert B.validate(*p, *g) == B.ERR_INVALID_ARG
    p = ptrs(g)
    p[4] = p[3] - 1024 + 4  # y's tail overlaps bias
    assert B.validate(*p, *g) == B.ERR_INVALID_ARG
    p = ptrs(g)
    p[4] = p[3] + 16  # adjacent but disjoint: bias is 4 floats = 16 bytes
    assert B.validate(*p, *g) == B.OK


def test_validate_rejects_beyond_int32():
    g = geo(N=1, C_in=3, H=30000, W=30000, C_out=4, KH=1, KW=1, pad=0)  # x = 2.7e9 elements
    assert B.validate(*ptrs(g, gap=1 << 40), *g) == B.ERR_UNSUPPORTED
    g = geo(N=1, C_in=2, H=32767, W=32767, C_out=2, KH=1, KW=1, pad=0)  # just under 2^31
    assert B.validate(*ptrs(g, gap=1 << 40), *g) == B.OK


def test_select_variant_on_workloads():
    for wl in synth.WORKLOADS.values():
        v = B.select_variant(wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad, wl.dtype)
        assert v in range(1, 8)
        assert B.variant_supports(v, wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad,
                                  wl.dtype)
    assert B.select_variant(1, 1, 2, 2, 1, 3, 3, 1, 0, 1) == -1


def test_fold_bn_textbook():
    rng = np.random.default_rng(0)
    C = 37
    gamma, beta = rng.standard_normal(C), rng.standard_normal(C)
    mean, var = rng.standard_normal(C), rng.uniform(0.1, 2.0, C)
    cb = rng.standard_normal(C)
    eps = 1e-5
    sc, bi = B.fold_bn(gamma, beta, mean, var, eps, cb)
    g32 = [np.float32(a).astype(np.float64) for a in (gamma, beta, mean, var, cb)]
    want_sc = g32[0] / np.sqrt(g32[3] + np.float64(np.float32(eps)))
    want_bi = g32[1] + (g32[4] - g32[2]) * want_sc
    np.testing.assert_allclose(sc, want_sc, rtol=1e-7)
    np.testing.assert_allclose(bi, want_bi, rtol=1e-6, atol=1e-6)
    # folded affine == batch norm applied to the conv output (+ conv bias)
    t = rng.standard_normal((5, C))
    bn = g32[0] * (t + g32[4] - g32[2]) / np.sqrt(g32[3] + np.float32(eps)) + g32[1]
    np.testing.assert_allclose(t * sc + bi, bn, rtol=1e-5, atol=1e-5)
    sc0, bi0 = B.fold_bn(gamma, beta, mean, var, eps)
    np.testing.assert_allclose(bi0, g32[1] - g32[2] * want_sc, rtol=1e-6, atol=1e-6)


def test_fold_bn_rejects():
    one = np.ones(3)
    with pytest.raises(B.CbsError):
        B.fold_bn(one, one, one, -one, 0.0)  # var + eps <= 0
    with pytest.raises(B.CbsError):
        B.fold_bn(one, one, one, one, -1.0)  # negative eps


def test_misaligned_and_overlapping_reports_the_overlap():
    # both faults at once: the overlap (a malformed call) wins
    g = geo()
    p = ptrs(g)
    p[4] = p[0] + 65  # y inside x and at an odd address
    assert B.validate(*p, *g) == B.ERR_INVALID_ARG


def test_grid_stride_index_never_wraps():
    """The element-wise kernels' grid-stride loop (k_scalar.hip): the next
    index is formed in 64 bits and clamped to the total, so for every total
    up to INT32_MAX and the largest grid the launcher uses (65536 blocks of
    256) the sequence of indices a lane visits stays in [0, total) and ends.
    The loop is modelled here with the same arithmetic, at the totals where
    a 32-bit sum would wrap."""
    stride = 65536 * 256
    int32_max = 2**31 - 1
    for total in (int32_max, int32_max - 1, int32_max - stride + 7, 3 * stride + 5):
        for first in (0, 1, stride - 1):
            idx, visits = first, 0
            while idx < total:
                assert 0 <= idx < total <= int32_max
                nxt = idx + stride  # 64-bit sum
                idx = nxt if nxt < total else total
                visits += 1
            assert visits == -(-(total - first) // stride)


def test_binding_rejects_host_output_buffers():
    """conv_bn_silu(out=...) must be a device tensor on x's device; a host
    tensor is refused before any pointer reaches the library."""
    import torch
    x = torch.empty(1, 2, 4, 4, dtype=torch.float32)
    out = torch.empty(1, 3, 4, 4, dtype=torch.float32)
    with pytest.raises(ValueError):
        B._check_output(out, x, (1, 3, 4, 4), "out")
    if not torch.cuda.is_available():
        return
    xd = x.cuda()
    with pytest.raises(ValueError):
        B._check_output(out, xd, (1, 3, 4, 4), "out")
