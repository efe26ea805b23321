"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises ``AssertionError`` if it is
wrong.  ``test_oracle_pins.py`` runs them on the real oracle; the mutant test
builds deliberately broken oracles and checks that at least one pin rejects
each of them.  Sources of truth used here:

  * hand-worked integer examples and closed forms under ``tests/golden/``;
  * ``torch.nn.functional.conv2d`` in float64 on the CPU (a library routine);
  * an explicit patch-matrix (im2col) formulation evaluated with numpy;
  * mathematical identities of the operator (delta input, linearity, stride
    and padding equivalences, identity weights reducing to SiLU(x)).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _torch_conv(x, w, s, p):
    import torch
    return torch.nn.functional.conv2d(torch.from_numpy(np.asarray(x, np.float64)),
                                      torch.from_numpy(np.asarray(w, np.float64)),
                                      stride=s, padding=p).numpy()


def _im2col_conv(x, w, s, p):
    """Same operator as a patch matrix times the flattened weights."""
    N, C, H, W = x.shape
    O, _, KH, KW = w.shape
    xp = np.zeros((N, C, H + 2 * p, W + 2 * p))
    xp[:, :, p:p + H, p:p + W] = x
    OH = (H + 2 * p - KH) // s + 1
    OW = (W + 2 * p - KW) // s + 1
    cols = np.empty((N, OH, OW, C, KH, KW))
    for i in range(OH):
        for j in range(OW):
            cols[:, i, j] = xp[:, :, i * s:i * s + KH, j * s:j * s + KW]
    out = cols.reshape(N * OH * OW, -1) @ w.reshape(O, -1).T
    return out.reshape(N, OH, OW, O).transpose(0, 3, 1, 2)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# shape
def pin_output_sizes(o):
    for sh in _load("workload_shapes.json")["shapes"]:
        assert o.out_dim(sh["H"], sh["K"], sh["stride"], sh["pad"]) == sh["OH"], sh
    # floor convention on a ragged case: (7 + 2 - 3)/2 = 3 -> 4 outputs
    assert o.out_dim(7, 3, 2, 1) == 4
    assert o.out_dim(2, 3, 1, 0) == -1


# ---------------------------------------------------------------------------
# convolution pass
def pin_hand_examples(o):
    g = _load("hand_examples.json")
    x = np.array(g["x"], np.float64)[None, None]
    for case in g["cases"]:
        w = np.array(case["w"], np.float64)[None, None]
        t1 = o.conv(x, w, case["stride"], case["pad"])
        np.testing.assert_array_equal(t1[0, 0], np.array(case["t1"], np.float64), err_msg=case["name"])


def pin_conv_vs_torch(o):
    rng = _rng(1)
    for (N, C, H, W, O, KH, KW) in [(2, 3, 7, 6, 4, 3, 3), (1, 2, 5, 9, 3, 1, 3),
                                    (2, 4, 6, 6, 5, 3, 2), (1, 5, 8, 7, 2, 2, 2)]:
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((O, C, KH, KW))
        for s in (1, 2, 3):
            for p in (0, 1, 2):
                if (H + 2 * p - KH) < 0 or (W + 2 * p - KW) < 0:
                    continue
                got = o.conv(x, w, s, p)
                ref = _torch_conv(x, w, s, p)
                assert got.shape == ref.shape, (got.shape, ref.shape)
                np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_conv_vs_im2col(o):
    rng = _rng(2)
    x = rng.standard_normal((2, 3, 9, 8))
    w = rng.standard_normal((4, 3, 3, 3))
    for s, p in [(1, 1), (2, 1), (2, 0), (3, 2)]:
        np.testing.assert_allclose(o.conv(x, w, s, p), _im2col_conv(x, w, s, p), rtol=1e-12, atol=1e-12)


def pin_delta_input(o):
    """x = one-hot at (n0, c0, h0, w0): t1[n0, co, oh, ow] reads back the
    weight tap w[co, c0, h0 - oh*s + p, w0 - ow*s + p] where it exists."""
    rng = _rng(3)
    C, H, W, O, KH, KW = 3, 6, 7, 2, 3, 3
    w = rng.standard_normal((O, C, KH, KW))
    for s, p, (n0, c0, h0, w0) in [(1, 1, (1, 2, 0, 5)), (2, 1, (0, 1, 3, 2)), (2, 0, (1, 0, 4, 4))]:
        x = np.zeros((2, C, H, W))
        x[n0, c0, h0, w0] = 1.0
        t1 = o.conv(x, w, s, p)
        OH, OW = t1.shape[2:]
        expect = np.zeros_like(t1)
        for oh in range(OH):
            for ow in range(OW):
                kh, kw = h0 - oh * s + p, w0 - ow * s + p
                if 0 <= kh < KH and 0 <= kw < KW:
                    expect[n0, :, oh, ow] = w[:, c0, kh, kw]
        np.testing.assert_array_equal(t1, expect)


def pin_all_ones_input(o):
    """All-ones x, pad 1, stride 1, 3x3: interior outputs are the sum of all
    weights of the output channel; a corner drops one row and one column."""
    rng = _rng(4)
    w = rng.standard_normal((3, 2, 3, 3))
    t1 = o.conv(np.ones((1, 2, 5, 5)), w, 1, 1)
    full = w.sum(axis=(1, 2, 3))
    corner = w[:, :, 1:, 1:].sum(axis=(1, 2, 3))
    np.testing.assert_allclose(t1[0, :, 2, 2], full, rtol=1e-13)
    np.testing.assert_allclose(t1[0, :, 0, 0], corner, rtol=1e-13)
    np.testing.assert_allclose(t1[0, :, 4, 4], w[:, :, :2, :2].sum(axis=(1, 2, 3)), rtol=1e-13)


def pin_linearity(o):
    rng = _rng(5)
    x1, x2 = rng.standard_normal((2, 1, 3, 6, 6))
    w = rng.standard_normal((2, 3, 3, 3))
    a, b = 0.75, -2.5
    lhs = o.conv(a * x1 + b * x2, w, 2, 1)
    rhs = a * o.conv(x1, w, 2, 1) + b * o.conv(x2, w, 2, 1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def pin_stride_is_subsampling(o):
    """A stride-s convolution is the stride-1 result sampled every s outputs."""
    rng = _rng(6)
    x = rng.standard_normal((1, 2, 9, 10))
    w = rng.standard_normal((3, 2, 3, 3))
    for s in (2, 3):
        full = o.conv(x, w, 1, 1)
        sub = o.conv(x, w, s, 1)
        np.testing.assert_allclose(sub, full[:, :, ::s, ::s][:, :, :sub.shape[2], :sub.shape[3]], rtol=1e-13, atol=1e-13)


def pin_pad_is_zero_border(o):
    """Padding p equals explicit zero borders of width p and no padding."""
    rng = _rng(7)
    x = rng.standard_normal((1, 2, 5, 6))
    w = rng.standard_normal((2, 2, 3, 2))
    for p in (1, 2):
        xp = np.zeros((1, 2, 5 + 2 * p, 6 + 2 * p))
        xp[:, :, p:p + 5, p:p + 6] = x
        np.testing.assert_array_equal(o.conv(x, w, 1, p), o.conv(xp, w, 1, 0))


def pin_channels_sum(o):
    """Convolving a multi-channel input equals the sum over single channels."""
    rng = _rng(8)
    x = rng.standard_normal((1, 4, 5, 5))
    w = rng.standard_normal((2, 4, 3, 3))
    total = sum(o.conv(x[:, c:c + 1], w[:, c:c + 1], 1, 1) for c in range(4))
    np.testing.assert_allclose(o.conv(x, w, 1, 1), total, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# batch-norm pass
def pin_bn(o):
    rng = _rng(9)
    t1 = rng.standard_normal((2, 3, 4, 5))
    np.testing.assert_array_equal(o.bn(t1, np.ones(3), np.zeros(3)), t1)
    bias = np.array([0.5, -1.0, 2.0])
    np.testing.assert_array_equal(o.bn(t1, np.zeros(3), bias), np.broadcast_to(bias[None, :, None, None], t1.shape))
    scale = np.array([2.0, -3.0, 0.25])
    np.testing.assert_array_equal(o.bn(np.ones((1, 3, 1, 1)), scale, bias)[0, :, 0, 0], scale + bias)


# ---------------------------------------------------------------------------
# SiLU pass
def pin_silu_closed_forms(o):
    g = _load("silu_closed_forms.json")
    xs = np.array([p["x"] for p in g["points"]] + [g["minimum"]["x"]])
    want = np.array([p["silu"] for p in g["points"]] + [g["minimum"]["silu"]])
    got = o.silu(xs)
    np.testing.assert_allclose(got, want, rtol=2e-15, atol=1e-300)
    # odd part: SiLU(x) - SiLU(-x) = x
    v = np.linspace(-30, 30, 241)
    np.testing.assert_allclose(o.silu(v) - o.silu(-v), v, rtol=1e-14, atol=1e-14)
    # the minimum is a minimum
    x0 = g["minimum"]["x"]
    near = o.silu(np.array([x0 - 1e-3, x0, x0 + 1e-3]))
    assert near[1] < near[0] and near[1] < near[2]
    # extremes: no overflow, correct limits
    big = o.silu(np.array([-1000.0, 1000.0]))
    assert big[0] == 0.0 and math.copysign(1.0, big[0]) == -1.0
    assert big[1] == 1000.0


# ---------------------------------------------------------------------------
# the composition
def pin_hand_bn_silu(o):
    g = _load("hand_examples.json")
    x = np.array(g["x"], np.float64)[None, None]
    w = np.ones((1, 1, 3, 3))
    bs = g["bn_silu"]
    y = o.forward(x, w, np.array([bs["scale"]]), np.array([bs["bias"]]), 1, 1)
    assert y[0, 0, 1, 1] == 0.0
    np.testing.assert_allclose(y[0, 0, 0, 0], -20.0 / (1.0 + math.exp(20.0)), rtol=1e-15)
    np.testing.assert_allclose(y[0, 0, 2, 1], 18.0 / (1.0 + math.exp(-18.0)), rtol=1e-15)


def pin_identity_weights_give_silu(o):
    """1x1 identity weights, scale 1, bias 0: y = SiLU(x) element-wise."""
    rng = _rng(10)
    x = rng.standard_normal((2, 4, 3, 5)) * 3
    w = np.eye(4).reshape(4, 4, 1, 1)
    y = o.forward(x, w, np.ones(4), np.zeros(4), 1, 0)
    np.testing.assert_allclose(y, x / (1.0 + np.exp(-x)), rtol=1e-15, atol=1e-300)


def pin_forward_vs_torch_composition(o):
    """The whole operator against torch conv2d + affine + torch SiLU (float64)."""
    import torch
    rng = _rng(11)
    x = rng.standard_normal((2, 3, 8, 7))
    w = rng.standard_normal((5, 3, 3, 3)) / 3
    scale = rng.uniform(0.5, 1.5, 5)
    bias = rng.standard_normal(5) * 0.3
    for s, p in [(1, 1), (2, 1)]:
        t = torch.from_numpy(_torch_conv(x, w, s, p))
        ref = torch.nn.functional.silu(t * torch.from_numpy(scale)[None, :, None, None]
                                       + torch.from_numpy(bias)[None, :, None, None]).numpy()
        np.testing.assert_allclose(o.forward(x, w, scale, bias, s, p), ref, rtol=1e-12, atol=1e-13)


def pin_points_match_forward(o):
    rng = _rng(12)
    x = rng.standard_normal((2, 3, 7, 9))
    w = rng.standard_normal((4, 3, 3, 3))
    scale, bias = rng.uniform(0.5, 1.5, 4), rng.standard_normal(4)
    y = o.forward(x, w, scale, bias, 2, 1)
    idx = np.arange(y.size)
    np.testing.assert_array_equal(o.points(x, w, scale, bias, 2, 1, idx), y.ravel())


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
