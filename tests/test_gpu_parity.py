"""GPU parity: the HIP kernels, called through the C ABI, against the fp64
CPU oracle on the same seeded inputs, element by element, under the stated
tolerances (fp32: |err| <= 1e-4*(1+|ref|); bf16: |err| <= 1.6e-2*|ref| + 1e-3).

Coverage: every variant on every shape of a sweep of small and ragged
geometries (odd sizes, kernel sizes 1-7, strides 1-3, padding 0-3, channel
counts off the tile sizes, M and K tails); the five workloads with a reduced
batch checked in full; the five workloads at full size, in the launch
configuration the benchmark times, every output checked; the epilogue's
special values (SiLU(0) = 0, the closed forms, saturation to -0 and to v) on
every variant; one handle driving two streams at once; the call captured in a
HIP graph and replayed; and the degenerate cases (empty batch, 1x1x1, padding
wider than the window's reach)."""
import numpy as np
import pytest

from conv_bn_silu_amd import synth
import gpu_util as U

pytestmark = pytest.mark.gpu

F32, BF16 = synth.DTYPE_F32, synth.DTYPE_BF16


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from conv_bn_silu_amd import binding
    return binding


def run(B, inp, variant="auto", stride=None):
    import torch
    x, w, sc, bi = U.upload(inp)
    y = B.conv_bn_silu(x, w, sc, bi, stride=inp.wl.stride, pad=inp.wl.pad, variant=variant)
    torch.cuda.synchronize()
    return y


SWEEP = [
    # N, C_in, H, W, C_out, KH, KW, stride, pad
    (1, 3, 7, 9, 5, 3, 3, 1, 1),
    (2, 16, 13, 11, 33, 3, 3, 2, 1),
    (1, 8, 5, 5, 17, 5, 5, 1, 2),
    (3, 5, 9, 10, 7, 7, 7, 3, 3),
    (2, 32, 17, 17, 48, 1, 1, 1, 0),
    (1, 40, 10, 12, 70, 1, 1, 2, 0),
    (2, 3, 33, 31, 16, 3, 3, 2, 1),
    (1, 64, 9, 9, 130, 3, 3, 1, 1),
    (2, 72, 6, 7, 64, 3, 3, 1, 0),
    (1, 1, 1, 1, 1, 1, 1, 1, 0),
    (1, 2, 3, 3, 3, 3, 3, 1, 3),
    (1, 4, 4, 6, 2, 2, 3, 2, 0),
    (2, 512, 4, 4, 40, 3, 3, 1, 1),
    (1, 256, 20, 20, 256, 1, 1, 1, 0),
    (2, 24, 21, 19, 144, 3, 3, 1, 1),
    (1, 3, 64, 64, 16, 3, 3, 2, 1),
    (2, 96, 12, 12, 64, 3, 3, 2, 1),
    # 1x1 shapes for the pointwise variant: K tail, channel tails, several
    # channel tiles, tiny and many images
    (3, 40, 4, 6, 70, 1, 1, 1, 0),
    (2, 72, 8, 10, 300, 1, 1, 1, 0),
    (5, 256, 8, 8, 16, 1, 1, 1, 0),
    (1, 8, 1, 8, 1, 1, 1, 1, 0),
    (7, 128, 12, 12, 200, 1, 1, 1, 0),
    # 64-pixel tiles: three channel tiles with a partial last tile, and
    # 8-pixel images (one tile spans 8 images) with a 200-channel tail
    (3, 256, 5, 8, 520, 1, 1, 1, 0),
    (9, 200, 2, 4, 64, 1, 1, 1, 0),
    # enough pixels for full 224-pixel ranges: ranges across image
    # boundaries and a short last range
    (11, 16, 64, 64, 24, 1, 1, 1, 0),
    # stems for the small-K variant: odd output-row counts, 1-3 channels,
    # C_out below 16, each row width class, more images than compute units
    (2, 3, 18, 64, 16, 3, 3, 2, 1),
    (1, 1, 33, 96, 5, 3, 3, 2, 1),
    (3, 2, 40, 640, 16, 3, 3, 2, 1),
    (2, 3, 7, 160, 12, 3, 3, 2, 1),
    (300, 3, 6, 32, 16, 3, 3, 2, 1),
    # channel-heavy 3x3 layers for the 32x32 window variant: whole-image
    # tiles, several tiles per image with ragged edges, partial channel
    # blocks, two output-channel tiles, stride 2, a 5x5 filter
    (2, 64, 20, 20, 128, 3, 3, 1, 1),
    (1, 96, 12, 16, 200, 3, 3, 1, 1),
    (2, 40, 16, 12, 64, 3, 3, 1, 1),
    (1, 128, 24, 24, 64, 3, 3, 2, 1),
    (3, 64, 36, 8, 48, 5, 5, 1, 2),
    (2, 32, 30, 28, 96, 3, 3, 1, 1),
    # stride-2 downsampling layers for the strided-rows variant: one to four
    # 16-channel chunks, a partial and a second output-channel tile, odd
    # heights, each row-width class
    (2, 16, 18, 24, 40, 3, 3, 2, 1),
    (1, 64, 33, 64, 128, 3, 3, 2, 1),
    (3, 32, 20, 320, 136, 3, 3, 2, 1),
    (2, 48, 12, 96, 64, 3, 3, 2, 1),
    # more output rows than ranks: several rows per workgroup with three
    # chunks (a prefetch depth of three units), and with one chunk (the
    # producers' loop ends in a partial round of units)
    (6, 48, 200, 32, 64, 3, 3, 2, 1),
    (5, 16, 240, 16, 24, 3, 3, 2, 1),
    # widest row class with OW not a multiple of 8 (8-byte output pieces;
    # with one or two chunks a prefetch depth of two units)
    (1, 32, 10, 296, 64, 3, 3, 2, 1),
    (2, 16, 6, 296, 40, 3, 3, 2, 1),
    # 32x32 window variant: more tiles than compute units (two tiles per
    # workgroup: the tile loop and the next tile's BN factors), an odd chunk
    # count (a padding chunk), a partial last channel tile, stride 2 with
    # 8-column loads
    (300, 16, 12, 12, 128, 3, 3, 1, 1),
    (3, 48, 20, 20, 72, 3, 3, 1, 1),
    (2, 64, 32, 32, 160, 3, 3, 2, 1),
]


def sweep_cases():
    from conv_bn_silu_amd import binding as B
    out = []
    for i, (N, C_in, H, W, C_out, KH, KW, s, p) in enumerate(SWEEP):
        for dt in (F32, BF16):
            for vname, v in B.VARIANTS.items():
                if v == 0 or not B.variant_supports(v, N, C_in, H, W, C_out, KH, KW, s, p, dt):
                    continue
                out.append(pytest.param(i, dt, vname, id=f"s{i}-{'bf16' if dt else 'f32'}-{vname}"))
            out.append(pytest.param(i, dt, "auto", id=f"s{i}-{'bf16' if dt else 'f32'}-auto"))
    return out


@pytest.mark.parametrize("case,dt,variant", sweep_cases())
def test_sweep(lib, case, dt, variant):
    N, C_in, H, W, C_out, KH, KW, s, p = SWEEP[case]
    wl = synth.Workload(f"sweep{case}", dt, N, C_in, H, W, C_out, KH, KW, s, p, "n01", 2000 + case)
    inp = synth.make_inputs(wl)
    U.say(f"[sweep] case {case} {SWEEP[case]} dtype {dt} variant {variant}")
    y = run(lib, inp, variant)
    U.check(U.to_f64(y), U.oracle_full(inp), dt, f"sweep{case}/{variant}")


REDUCED = {"c1": {}, "c2": {"N": 1}, "c3": {"N": 1, "H": 96, "W": 80}, "c4": {"N": 2, "H": 130},
           "c5": {"N": 3}}


def workload_variants(key, reduced=True):
    from conv_bn_silu_amd import binding as B
    wl = synth.WORKLOADS[key].with_(**REDUCED[key]) if reduced else synth.WORKLOADS[key]
    vs = ["auto"] + [n for n, v in B.VARIANTS.items()
                     if v and B.variant_supports(v, wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW,
                                                 wl.stride, wl.pad, wl.dtype)]
    return [pytest.param(key, v, id=f"{key}-{v}") for v in vs]


@pytest.mark.parametrize("key,variant", [p for k in sorted(REDUCED) for p in workload_variants(k)])
def test_workload_reduced_full_check(lib, key, variant):
    """Each workload's layer at a reduced batch/size (several tiles, ragged
    tails), every output checked against the full oracle."""
    wl = synth.WORKLOADS[key].with_(**REDUCED[key])
    inp = synth.make_inputs(wl)
    U.say(f"[reduced] {key} {wl} variant {variant}")
    y = run(lib, inp, variant)
    U.check(U.to_f64(y), U.oracle_full(inp), wl.dtype, f"{key}/{variant}")


@pytest.mark.parametrize("key", sorted(synth.WORKLOADS))
def test_workload_full_size(lib, key):
    """Each workload at its full size through AUTO dispatch -- the launch the
    benchmark times -- with every output checked against the full oracle."""
    wl = synth.WORKLOADS[key]
    inp = synth.make_inputs(wl)
    U.say(f"[full] {key} {wl.name}")
    y = U.to_f64(run(lib, inp))
    U.say(f"[full] {key} oracle")
    U.check(y, U.oracle_full(inp), wl.dtype, f"{key}/full")


# Epilogue special values: with x = 0 the accumulator is exactly 0, so
# v = bias[co] and y = SiLU(bias[co]) for every pixel.  The bias pattern puts
# v at 0 (SiLU(0) = 0), +-1 and 2 (closed forms), +-20, -100, -1000 (e^-v
# overflows: the result saturates to -0) and 1000 (e^-v underflows: y = v).
EDGE_BIAS = [0.0, 1.0, -1.0, 2.0, 20.0, -20.0, -100.0, -1000.0, 1000.0]
EDGE_SHAPES = [
    # N, C_in, H, W, C_out, KH, KW, stride, pad
    (2, 16, 9, 9, 18, 3, 3, 1, 1),      # gather, scalar
    (2, 32, 8, 8, 20, 3, 3, 1, 1),      # window, window32
    (2, 64, 8, 8, 40, 1, 1, 1, 0),      # pointwise
    (2, 3, 16, 64, 16, 3, 3, 2, 1),     # small_k (stem)
    (2, 32, 16, 64, 40, 3, 3, 2, 1),    # strided rows
]


def edge_cases():
    from conv_bn_silu_amd import binding as B
    out = []
    for i, shp in enumerate(EDGE_SHAPES):
        for dt in (F32, BF16):
            for vname, v in B.VARIANTS.items():
                if v == 0 or not B.variant_supports(v, *shp, dt):
                    continue
                out.append(pytest.param(i, dt, vname, id=f"e{i}-{'bf16' if dt else 'f32'}-{vname}"))
    return out


@pytest.mark.parametrize("case,dt,variant", edge_cases())
def test_epilogue_special_values(lib, case, dt, variant):
    import torch
    N, C_in, H, W, C_out, KH, KW, s_, p_ = EDGE_SHAPES[case]
    wl = synth.Workload(f"edge{case}", dt, N, C_in, H, W, C_out, KH, KW, s_, p_, "n01", 3000 + case)
    inp = synth.make_inputs(wl)
    inp.x[...] = 0.0
    if inp.x_bits is not None:
        inp.x_bits[...] = 0
    inp.bias[:] = np.resize(np.array(EDGE_BIAS, np.float32), C_out)
    U.say(f"[edge] case {case} dtype {dt} variant {variant}")
    y = U.to_f64(run(lib, inp, variant))
    ref = U.oracle_full(inp)
    U.check(y, ref, dt, f"edge{case}/{variant}")
    bias = inp.bias.astype(np.float64)[None, :, None, None] * np.ones_like(y)
    # exact where the value is exact in the output type
    assert np.all(y[bias == 0.0] == 0.0), "SiLU(0) must be 0"
    assert np.all(y[bias == -1000.0] == 0.0), "SiLU(-1000) must saturate to (-)0"
    assert np.all(y[bias == 1000.0] == 1000.0), "SiLU(1000) must be 1000"
    assert np.all(np.abs(y[bias == -100.0]) <= 1e-30), "SiLU(-100) is below 1e-41"
    del torch


def test_empty_batch_is_a_no_op(lib):
    import torch
    h = lib.default_library()
    U.say("[edge] N=0")
    h.run_ptr(0, 0, 0, 0, 0, 0, 0, 3, 8, 8, 4, 3, 3, 1, 1, lib.DTYPE_BF16,
              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()


def test_deterministic_and_no_stray_writes(lib):
    """Two runs give the same bits, and the guard bands around y stay intact."""
    import torch
    for key in ("c1", "c5"):
        wl = synth.WORKLOADS[key].with_(**REDUCED[key])
        inp = synth.make_inputs(wl)
        x, w, sc, bi = U.upload(inp)
        n_out = wl.N * wl.C_out * wl.OH * wl.OW
        guard = 4096
        dt = torch.bfloat16 if wl.dtype == BF16 else torch.float32
        buf = torch.full((n_out + 2 * guard,), 12345.0, dtype=dt, device="cuda")
        U.say(f"[guard] {key}")
        outs = []
        for _ in range(2):
            y = buf[guard:guard + n_out].view(wl.N, wl.C_out, wl.OH, wl.OW)
            lib.conv_bn_silu(x, w, sc, bi, stride=wl.stride, pad=wl.pad, out=y)
            torch.cuda.synchronize()
            outs.append(y.clone())
        assert torch.equal(outs[0].view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           outs[1].view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        assert bool((buf[:guard] == 12345.0).all()) and bool((buf[guard + n_out:] == 12345.0).all())


def test_side_stream(lib):
    import torch
    wl = synth.WORKLOADS["c5"].with_(N=2)
    inp = synth.make_inputs(wl)
    x, w, sc, bi = U.upload(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    U.say("[stream] side stream")
    with torch.cuda.stream(s):
        y = lib.conv_bn_silu(x, w, sc, bi, stride=1, pad=1)
    s.synchronize()
    U.check(U.to_f64(y), U.oracle_full(inp), BF16, "side stream")


@pytest.mark.parametrize("key", ["c1", "c2", "c5"])
def test_graph_capture_replays(lib, key):
    """The fused call captured in a HIP graph (torch.cuda.CUDAGraph) and
    replayed four times, with eager work and synchronisations between the
    replays: every replay writes exactly the eager call's bits, and the
    eager call matches the oracle.  The call only enqueues kernels (no
    allocation, no memset), so it can be captured."""
    import torch
    wl = synth.WORKLOADS[key]
    if key != "c1":
        wl = wl.with_(N=1)
    inp = synth.make_inputs(wl)
    x, w, sc, bi = U.upload(inp)
    U.say(f"[graph] {key} eager")
    ref = lib.conv_bn_silu(x, w, sc, bi, stride=wl.stride, pad=wl.pad)
    torch.cuda.synchronize()
    U.check(U.to_f64(ref), U.oracle_full(inp), wl.dtype, f"{key} eager")
    bits = torch.int16 if ref.dtype == torch.bfloat16 else torch.int32
    y = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up call off the default stream before capture
        lib.conv_bn_silu(x, w, sc, bi, stride=wl.stride, pad=wl.pad, out=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    U.say(f"[graph] {key} capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.conv_bn_silu(x, w, sc, bi, stride=wl.stride, pad=wl.pad, out=y)
    torch.cuda.synchronize()
    for r in range(4):
        y.view(bits).fill_(0x5A5A)  # a replay that wrote nothing would leave this pattern
        torch.cuda.synchronize()
        U.say(f"[graph] {key} replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(bits), ref.view(bits)), f"{key}: replay {r} differs from the eager call"
        z = lib.conv_bn_silu(x, w, sc, bi, stride=wl.stride, pad=wl.pad)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(z.view(bits), ref.view(bits))
    del g


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_unfused_sequence(lib, key):
    """The three-kernel baseline: each pass checked against the oracle's pass
    applied to the GPU's own input of that pass (so the bf16 rounding of the
    stored intermediates does not enter the comparison)."""
    import oracle
    o = oracle.get()
    wl = synth.WORKLOADS[key].with_(**REDUCED[key])
    inp = synth.make_inputs(wl)
    x, w, sc, bi = U.upload(inp)
    U.say(f"[unfused] {key}")
    y, t1, t2 = lib.conv_bn_silu_unfused(x, w, sc, bi, stride=wl.stride, pad=wl.pad)
    import torch
    torch.cuda.synchronize()
    U.check(U.to_f64(t1), o.conv(inp.x, inp.w, wl.stride, wl.pad), wl.dtype, "conv pass")
    t1h, t2h = U.to_f64(t1), U.to_f64(t2)
    U.check(t2h, o.bn(t1h, inp.scale, inp.bias), wl.dtype, "bn pass")
    U.check(U.to_f64(y), o.silu(t2h), wl.dtype, "silu pass")


def test_one_handle_two_streams(lib):
    """One handle, two streams, different weights and inputs on each, calls
    interleaved so that kernels of both streams run at the same time: each
    stream's result matches its own oracle (the handle holds no per-call
    state, so concurrent calls cannot disturb each other)."""
    import torch
    h = lib.default_library()
    inputs, uploads = [], []
    for seed in (5101, 5102):
        inp = synth.make_inputs(synth.WORKLOADS["c5"].with_(N=3), seed=seed)
        inputs.append(inp)
        uploads.append(U.upload(inp))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    U.say("[streams] two streams, one handle")
    for _ in range(4):
        for (x, w, sc, bi), st in zip(uploads, streams):
            with torch.cuda.stream(st):
                outs.append(lib.conv_bn_silu(x, w, sc, bi, stride=1, pad=1, library=h))
    torch.cuda.synchronize()
    refs = [U.oracle_full(inp) for inp in inputs]
    for i, y in enumerate(outs):
        U.check(U.to_f64(y), refs[i % 2], BF16, f"stream {i % 2} call {i // 2}")


def test_element_misaligned_pointers_are_unsupported(lib):
    import torch
    wl = synth.Workload("odd", BF16, 1, 8, 8, 8, 8, 3, 3, 1, 1, "n01", 4243)
    inp = synth.make_inputs(wl)
    x, w, sc, bi = U.upload(inp)
    buf = torch.empty(x.numel() * 2 + 8, dtype=torch.uint8, device="cuda")
    h = lib.default_library()
    U.say("[misaligned] odd byte address")
    with pytest.raises(lib.CbsError) as ei:
        h.run_ptr(0, buf.data_ptr() + 1, w.data_ptr(), sc.data_ptr(), bi.data_ptr(),
                  torch.empty(wl.N * wl.C_out * wl.OH * wl.OW, dtype=torch.bfloat16, device="cuda").data_ptr(),
                  wl.N, wl.C_in, wl.H, wl.W, wl.C_out, wl.KH, wl.KW, wl.stride, wl.pad, wl.dtype,
                  torch.cuda.current_stream().cuda_stream)
    assert ei.value.status == lib.ERR_UNSUPPORTED


def test_misaligned_pointers_fall_back(lib):
    """A y that is element-aligned but not 16-byte aligned: AUTO still serves
    the call (with a variant that needs no vector alignment) and the result is
    right; forcing the vectorised pointwise variant is refused."""
    import torch
    wl = synth.Workload("misaligned", BF16, 2, 64, 8, 8, 48, 1, 1, 1, 0, "n01", 4242)
    inp = synth.make_inputs(wl)
    x, w, sc, bi = U.upload(inp)
    n_out = wl.N * wl.C_out * wl.OH * wl.OW
    buf = torch.empty(n_out + 8, dtype=torch.bfloat16, device="cuda")
    y = buf[1:1 + n_out].view(wl.N, wl.C_out, wl.OH, wl.OW)
    U.say("[misaligned] auto")
    lib.conv_bn_silu(x, w, sc, bi, stride=1, pad=0, out=y)
    torch.cuda.synchronize()
    U.check(U.to_f64(y), U.oracle_full(inp), BF16, "misaligned auto")
    with pytest.raises(lib.CbsError) as ei:
        lib.conv_bn_silu(x, w, sc, bi, stride=1, pad=0, out=y, variant="pointwise")
    assert ei.value.status == lib.ERR_UNSUPPORTED
