"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: |y - ref| <= tol * (1 + |ref|) elementwise with tol = 1e-5 for float32 and
2e-3 for float16 inputs (float32 accumulation).  Small-integer-valued inputs must give
exactly the oracle's value rounded once to the element type.  Full-size benchmark
shapes are checked on every output in the dispatcher's own launch configuration (the
family it must pick is asserted too); reduced shapes with the same attributes, ragged
sizes and several tiles are checked on every output."""
import contextlib
import zlib

import numpy as np
import pytest
import torch

import pins
import workloads as W
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3}
NPT = {"f32": np.float32, "f16": np.float16}
FAMILIES = ["auto", "direct", "grouped", "igemm"]


@pytest.fixture(scope="module")
def T():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import transposed_convolution_amd as T
    T.load_library()
    return T


def gpu_run(T, x, w, b, attrs, cl=False, kernel="auto"):
    """Run on the GPU; returns the logical-layout result as float64, or None when the
    forced kernel family does not serve this problem."""
    dev = torch.device("cuda:0")
    tx = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    if cl:
        tx = T.to_channels_last(tx)
    tw = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    tb = None if b is None else torch.from_numpy(b).to(dev)
    try:
        y = T.convtranspose_nd(tx, tw, tb, channels_last=cl, kernel=kernel, **attrs)
    except T.ConvTransposeError as e:
        if e.status == 3 and kernel not in ("auto", "direct"):
            return None
        raise
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def check(got, ref, dtype, integer, what=""):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if integer:
        want = ref.astype(NPT[dtype]).astype(np.float64)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {np.unravel_index(bad[0], got.shape)}: " \
                              f"{got.flat[bad[0]]} vs {want.flat[bad[0]]}"
    else:
        if got.size == 0:
            return
        err = np.abs(got - ref) / (1.0 + np.abs(ref))
        i = int(np.argmax(err))
        assert err.flat[i] <= TOL[dtype], \
            f"{what}: max rel err {err.flat[i]:.3e} at {np.unravel_index(i, got.shape)}: {got.flat[i]} vs {ref.flat[i]}"


def _log(msg):
    print(msg, flush=True)


@contextlib.contextmanager
def forced_tile(T, tile):
    """Run the float16 MFMA kernel with one block shape (None: the automatic choice)."""
    T.set_igemm_tile(tile)
    try:
        yield
    finally:
        T.set_igemm_tile(None)


# --------------------------------------------------------------------------------------
# benchmark configurations
# --------------------------------------------------------------------------------------
WHOLE = [W.C1, W.C2, W.C3, W.C3_NHWC, W.G2_NCHW, W.G2_NHWC]
FULL = [W.C4, W.C4_NHWC, W.C5_S1, W.C5_S1_P1, W.C5_S2, W.G3_DW]
# the family the dispatcher must pick for each configuration (a silent fall-back to the
# gather kernel would still be correct, so parity alone would not notice it)
EXPECTED_FAMILY = {W.C1.name: "direct", W.C2.name: "igemm", W.C3.name: "grouped", W.C3_NHWC.name: "grouped",
                   W.C4.name: "igemm",
                   W.C4_NHWC.name: "igemm", W.C5_S1.name: "igemm", W.C5_S1_P1.name: "igemm", W.C5_S2.name: "igemm",
                   W.G3_DW.name: "grouped", W.G2_NCHW.name: "grouped", W.G2_NHWC.name: "grouped"}


def _auto_family(T, wl, x, w, b):
    dev = torch.device("cuda:0")
    tx = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    if wl.channels_last:
        tx = T.to_channels_last(tx)
    tw = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    tb = None if b is None else torch.from_numpy(b).to(dev)
    return T.convtranspose_select_kernel(tx, tw, tb, channels_last=wl.channels_last, **wl.attrs)


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("kernel", FAMILIES)
@pytest.mark.parametrize("wl", WHOLE, ids=lambda w: w.name)
def test_config_whole_output(T, wl, kernel, integer):
    _log(f"[case] whole {wl.name} kernel={kernel} integer={integer}")
    x, w, b = W.make_inputs(wl, integer=integer)
    if kernel == "auto":
        assert _auto_family(T, wl, x, w, b) == EXPECTED_FAMILY[wl.name]
    got = gpu_run(T, x, w, b, wl.attrs, wl.channels_last, kernel)
    if got is None:
        pytest.skip(f"{kernel} does not serve {wl.name}")
    ref = O.convtranspose(x, w, b, **wl.attrs)
    check(got, ref, wl.dtype, integer, wl.name)


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_config_full_size_whole_output(T, wl, integer):
    """Full benchmark size, in the dispatcher's own launch configuration (the one the
    benchmark times), compared on every output element with the oracle."""
    _log(f"[case] full size {wl.name} integer={integer}")
    x, w, b = W.make_inputs(wl, integer=integer)
    assert _auto_family(T, wl, x, w, b) == EXPECTED_FAMILY[wl.name]
    got = gpu_run(T, x, w, b, wl.attrs, wl.channels_last, "auto")
    assert np.all(np.isfinite(got))
    ref = O.convtranspose(x, w, b, **wl.attrs)
    check(got, ref, wl.dtype, integer, wl.name)


def reduced(wl, x_shape, w_shape, **kw):
    return wl.with_(name=wl.name + "_reduced", x_shape=x_shape, w_shape=w_shape, **kw)


REDUCED = [
    reduced(W.C3, (3, 40, 29, 37), (40, 1, 4, 4), attrs=dict(W.C3.attrs, group=40)),
    reduced(W.C3, (2, 24, 13, 70), (24, 2, 4, 4), attrs=dict(W.C3.attrs, group=12)),
    reduced(W.C4, (2, 64, 20, 36), (64, 48, 4, 4)),
    reduced(W.C4, (3, 40, 11, 70), (40, 72, 4, 4)),
    reduced(W.C4_NHWC, (2, 64, 20, 36), (64, 48, 4, 4)),
    reduced(W.C4_NHWC, (1, 136, 9, 17), (136, 24, 4, 4)),
    reduced(W.C5_S1, (1, 32, 5, 9, 11), (32, 24, 3, 3, 3)),
    reduced(W.C5_S1_P1, (2, 48, 4, 7, 10), (48, 40, 3, 3, 3)),
    reduced(W.C5_S2, (1, 32, 5, 9, 11), (32, 24, 3, 3, 3)),
    reduced(W.C5_S2.with_(channels_last=True), (2, 40, 3, 6, 9), (40, 16, 3, 3, 3)),
    reduced(W.C2, (3, 24, 77), (24, 40, 5)),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("kernel", FAMILIES)
@pytest.mark.parametrize("wl", REDUCED, ids=lambda w: f"{w.name}_{w.x_shape}_{'cl' if w.channels_last else 'nc'}")
def test_reduced_whole_output(T, wl, kernel, integer):
    _log(f"[case] reduced {wl.name} {wl.x_shape} kernel={kernel} integer={integer}")
    x, w, b = W.make_inputs(wl, integer=integer)
    got = gpu_run(T, x, w, b, wl.attrs, wl.channels_last, kernel)
    if got is None:
        pytest.skip(f"{kernel} does not serve this shape")
    ref = O.convtranspose(x, w, b, **wl.attrs)
    check(got, ref, wl.dtype, integer, f"{wl.name}{wl.x_shape}")


# --------------------------------------------------------------------------------------
# random small problems and edge cases
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("kernel", FAMILIES)
def test_random_small_problems(T, kernel, dtype, cl):
    rng = np.random.default_rng(1000 + FAMILIES.index(kernel) * 10 + (dtype == "f16") * 2 + cl)
    ran = 0
    for t in range(50):
        x, w, b, attrs = pins.random_case(rng, auto=(t % 4 == 3), max_L=9)
        x, w = x.astype(NPT[dtype]), w.astype(NPT[dtype])
        b = None if b is None else b.astype(NPT[dtype])
        _log(f"[case] random #{t} {kernel} {dtype} cl={cl} x{x.shape} w{w.shape} {attrs}")
        got = gpu_run(T, x, w, b, attrs, cl, kernel)
        if got is None:
            continue
        ran += 1
        check(got, O.convtranspose(x, w, b, **attrs), dtype, False, f"random #{t} {attrs}")
    if kernel in ("auto", "direct"):
        assert ran == 50


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
def test_random_igemm_shaped_problems(T, cl):
    """Shapes the implicit-GEMM path accepts (channels per group a multiple of 8; an even
    innermost input size for NC.. layout, a multiple of 8 or not), random
    strides/dilations/pads/groups, ragged channel and pixel tails; forced igemm with the
    automatic block shape and with one forced shape per case, and the dispatcher's choice."""
    rng = np.random.default_rng(77 + cl)
    ran = 0
    for t in range(40):
        nsp = int(rng.integers(1, 4))
        G = int(rng.choice([1, 1, 1, 2]))
        Cg = int(rng.choice([8, 16, 24, 40, 64]))
        Mg = int(rng.integers(1, 80))
        L = [int(rng.integers(1, 7)) for _ in range(nsp - 1)] + [int(rng.choice([8, 16, 24, 32, 6, 10, 18, 34]))]
        K = [int(rng.integers(1, 5)) for _ in range(nsp)]
        s = [int(rng.integers(1, 4)) for _ in range(nsp)]
        d = [int(rng.integers(1, 3)) for _ in range(nsp)]
        op = [int(rng.integers(0, max(a, b))) for a, b in zip(s, d)]
        attrs = dict(strides=s, dilations=d, output_padding=op, group=G,
                     pads=[int(rng.integers(0, 3)) for _ in range(2 * nsp)])
        try:
            O.output_shape((2, G * Cg, *L), (G * Cg, Mg, *K), **attrs)
        except O.OracleError:
            continue
        integer = bool(t % 2)
        gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
        x = gen((2, G * Cg, *L)).astype(np.float16)
        w = (gen((G * Cg, Mg, *K)) * (1 if integer else 0.2)).astype(np.float16)
        b = gen(G * Mg).astype(np.float16)
        tile = T.IGEMM_TILES[t % len(T.IGEMM_TILES)]
        _log(f"[case] igemm-random #{t} cl={cl} x{x.shape} w{w.shape} {attrs} (and tile {tile})")
        ref = O.convtranspose(x, w, b, **attrs)
        for kernel, forced in (("igemm", None), ("auto", None), ("igemm", tile)):
            with forced_tile(T, forced):
                got = gpu_run(T, x, w, b, attrs, cl, kernel)
            if got is None:
                continue
            ran += kernel == "igemm" and forced is None
            check(got, ref, "f16", integer, f"igemm-random #{t} {kernel} tile {forced} {attrs}")
    assert ran >= 25


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
def test_random_float32_mfma_problems(T, cl):
    """float32 implicit GEMM on MFMA: random rank, strides, dilations, pads, groups and
    ragged channel counts, several 64 x 64 tiles and 16-deep depth steps; forced and via
    the dispatcher.  Tolerance 1e-5 (1+|ref|); integer-valued inputs bit-exact."""
    rng = np.random.default_rng(303 + cl)
    ran = 0
    for t in range(30):
        nsp = int(rng.integers(1, 4))
        G = int(rng.choice([1, 1, 2, 3]))
        Cg = int(rng.integers(1, 70))
        Mg = int(rng.integers(1, 90))
        L = [int(rng.integers(1, 9)) for _ in range(nsp - 1)] + [int(rng.integers(1, 40))]
        K = [int(rng.integers(1, 4)) for _ in range(nsp)]
        s = [int(rng.integers(1, 4)) for _ in range(nsp)]
        d = [int(rng.integers(1, 3)) for _ in range(nsp)]
        attrs = dict(strides=s, dilations=d, group=G,
                     output_padding=[int(rng.integers(0, max(a, b))) for a, b in zip(s, d)],
                     pads=[int(rng.integers(0, 3)) for _ in range(2 * nsp)])
        xs, ws = (2, G * Cg, *L), (G * Cg, Mg, *K)
        try:
            O.output_shape(xs, ws, **attrs)
        except O.OracleError:
            continue
        integer = bool(t % 2)
        gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
        x = gen(xs).astype(np.float32)
        w = (gen(ws) * (1 if integer else 0.2)).astype(np.float32)
        b = gen(G * Mg).astype(np.float32)
        _log(f"[case] f32-mfma-random #{t} cl={cl} x{x.shape} w{w.shape} {attrs}")
        ref = O.convtranspose(x, w, b, **attrs)
        for kernel in ("igemm", "auto"):
            got = gpu_run(T, x, w, b, attrs, cl, kernel)
            assert got is not None, f"float32 MFMA path refused #{t}"
            ran += kernel == "igemm"
            check(got, ref, "f32", integer, f"f32-mfma-random #{t} {kernel} {attrs}")
    assert ran >= 20


EDGE = [
    # (name, x_shape, w_shape, attrs, bias)
    ("empty_batch", (0, 8, 5, 5), (8, 4, 3, 3), dict(strides=[2, 2]), True),
    ("zero_output_width", (1, 4, 5, 1), (4, 4, 3, 2), dict(pads=[0, 0, 1, 1]), True),
    ("no_input_channels", (2, 0, 4, 4), (0, 3, 3, 3), dict(strides=[2, 2]), True),
    ("empty_spatial_input", (1, 3, 0, 4), (3, 2, 4, 3), dict(strides=[2, 1]), True),
    # empty inputs with C/group >= 16: routed to the gather kernel, never to the MFMA kernels
    ("empty_spatial_wide", (1, 16, 4, 0), (16, 16, 4, 4), dict(strides=[2, 2]), True),
    ("empty_spatial_wide_3d", (1, 16, 3, 0, 4), (16, 16, 3, 3, 3), dict(strides=[2, 2, 2]), True),
    ("empty_spatial_wide_grouped", (1, 64, 0, 3), (64, 32, 3, 3), dict(strides=[2, 2], group=2), False),
    ("kernel_smaller_than_stride", (1, 8, 5, 6), (8, 8, 2, 1), dict(strides=[3, 2]), True),
    ("large_pads_crop", (1, 8, 9, 9), (8, 8, 5, 5), dict(strides=[2, 2], pads=[4, 3, 2, 5]), True),
    ("same_upper_negative", (1, 4, 6, 5), (4, 4, 1, 1), dict(strides=[2, 3], auto_pad="SAME_UPPER"), True),
    ("same_lower_odd", (1, 16, 7, 7), (16, 8, 3, 3), dict(strides=[2, 2], auto_pad="SAME_LOWER"), True),
    ("output_shape", (1, 16, 7, 7), (16, 8, 4, 4), dict(strides=[2, 2], output_shape=[15, 13]), True),
    ("pointwise", (2, 64, 6, 7), (64, 32, 1, 1), {}, True),
    ("pointwise_s2", (2, 64, 6, 7), (64, 32, 1, 1), dict(strides=[2, 2]), False),
    ("dilated", (1, 32, 8, 8), (32, 16, 3, 3), dict(dilations=[2, 3], strides=[2, 1], output_padding=[1, 2]), True),
    ("depthwise_3d", (1, 8, 4, 5, 6), (8, 1, 3, 3, 3), dict(strides=[2, 2, 2], group=8), True),
    ("grouped_mixed", (2, 12, 6, 6), (12, 5, 3, 3), dict(strides=[2, 2], group=3, pads=[1, 0, 0, 1]), True),
    ("long_1d", (1, 16, 3000), (16, 8, 7), dict(strides=[4], pads=[3, 3], output_padding=[3]), True),
    ("stride_larger_than_kernel_3d", (1, 16, 3, 4, 5), (16, 16, 2, 2, 2), dict(strides=[3, 3, 3]), True),
]


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("kernel", FAMILIES)
@pytest.mark.parametrize("case", EDGE, ids=lambda c: c[0])
def test_edge_cases(T, case, kernel, dtype, cl):
    name, xs, ws, attrs, has_b = case
    _log(f"[case] edge {name} {kernel} {dtype} cl={cl}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    x = rng.integers(-2, 3, size=xs).astype(NPT[dtype])
    w = rng.integers(-2, 3, size=ws).astype(NPT[dtype])
    m = ws[1] * attrs.get("group", 1)
    b = rng.integers(-4, 5, size=m).astype(NPT[dtype]) if has_b else None
    got = gpu_run(T, x, w, b, attrs, cl, kernel)
    if got is None:
        pytest.skip(f"{kernel} does not serve {name}")
    check(got, O.convtranspose(x, w, b, **attrs), dtype, True, name)


DEPTHWISE = [
    # (x_shape, kernel size, attrs): one channel in and out per group, equal strides
    ((2, 5, 13, 21), 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 3, 9, 300), 4, dict(strides=[2, 2])),
    ((2, 4, 10, 17), 3, dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1])),
    ((1, 6, 31, 9), 3, dict(pads=[1, 1, 1, 1])),
    ((1, 2, 12, 40), 3, dict(dilations=[2, 2], pads=[2, 2, 2, 2])),
    ((1, 2, 7, 11), 5, {}),
    ((1, 2, 150, 1500), 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 3, 8, 12), 4, dict(strides=[2, 2], pads=[0, 1, 2, 1])),
    ((2, 2, 6, 1), 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 4, 9, 14), 4, dict(strides=[2, 2], auto_pad="SAME_UPPER")),
    ((3, 7, 5, 6), 3, dict(strides=[2, 2], pads=[2, 0, 0, 2], output_padding=[1, 0])),
    ((2, 3, 9, 16), 8, dict(strides=[4, 4], pads=[2, 2, 2, 2])),
    ((1, 4, 10, 24), 2, dict(strides=[2, 2])),
    ((1, 3, 11, 16), 6, dict(strides=[2, 2], pads=[2, 2, 2, 2])),
    ((1, 3, 7, 16), 3, dict(strides=[2, 2], dilations=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1])),
    ((2, 2, 12, 13), 5, dict(pads=[2, 2, 2, 2])),
    ((1, 2, 5, 24), 4, dict(strides=[4, 4], pads=[0, 1, 3, 0])),
    ((1, 3, 20, 24), 4, dict(strides=[2, 2], pads=[3, 0, 0, 3], output_padding=[1, 1])),
    # stride 1 with rows of whole 8-column pieces (the streaming-store path)
    ((1, 3, 10, 16), 3, dict(pads=[1, 1, 1, 1])),
    ((2, 2, 6, 24), 5, dict(pads=[2, 2, 2, 2])),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", DEPTHWISE, ids=lambda c: f"{c[0]}_k{c[1]}_{sorted(c[2].items())}")
def test_depthwise_shapes(T, case, integer):
    """Depthwise problems (group == C, one output channel per group) in float16: the
    banded per-phase effective-kernel path where the window shape is one it serves, the
    generic grouped kernel elsewhere; ragged rows and columns, several bands per plane."""
    xs, k, attrs = case
    C = xs[1]
    attrs = dict(attrs, group=C)
    _log(f"[case] depthwise x{xs} k{k} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen((C, 1, k, k)) * (1 if integer else 0.3)).astype(np.float16)
    b = gen(C).astype(np.float16)
    ref = O.convtranspose(x, w, b, **attrs)
    ref_nb = O.convtranspose(x, w, None, **attrs)
    for kernel in ("grouped", "auto"):
        got = gpu_run(T, x, w, b, attrs, False, kernel)
        check(got, ref, "f16", integer, f"depthwise {kernel} x{xs} {attrs}")
    got = gpu_run(T, x, w, None, attrs, False, "grouped")
    check(got, ref_nb, "f16", integer, f"depthwise no-bias x{xs} {attrs}")


GROUPED_3D = [
    # (x_shape, w_shape, attrs): rank-3 grouped and depthwise calls (C/group, M/group <= 8),
    # channels-first, on the grouped bandwidth kernel: strides, dilations, pads, output
    # padding, residue classes without taps, several row bands per plane
    ((2, 4, 5, 6, 7), (4, 1, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, group=4)),
    ((1, 6, 4, 9, 11), (6, 2, 2, 4, 3), dict(strides=[1, 2, 2], pads=[0, 1, 1, 1, 0, 1], group=3)),
    ((1, 8, 3, 5, 5), (8, 3, 3, 2, 2), dict(strides=[3, 1, 2], dilations=[2, 1, 1], group=2, output_padding=[1, 0, 1])),
    ((2, 3, 6, 4, 8), (3, 1, 4, 3, 3), dict(strides=[2, 1, 1], pads=[1, 1, 1, 2, 1, 1], group=3)),
    ((1, 16, 4, 40, 36), (16, 1, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1], group=16)),
    ((1, 4, 2, 3, 4), (4, 2, 1, 1, 1), dict(strides=[4, 2, 3], group=2)),
    # depthwise with rows of a multiple of 8 inputs: the depthwise kernel's planes of
    # first-axis taps (1, 2 or 3 per output plane, planes outside the input, dilation and
    # stride 3 on the first axis, row bands)
    ((2, 8, 5, 12, 16), (8, 1, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1], group=8)),
    ((1, 4, 6, 9, 24), (4, 1, 4, 4, 4), dict(strides=[2, 2, 2], pads=[1] * 6, group=4)),
    ((1, 3, 4, 7, 16), (3, 1, 3, 3, 3), dict(pads=[1] * 6, group=3)),
    ((1, 2, 3, 5, 8), (2, 1, 2, 2, 2), dict(strides=[2, 2, 2], group=2)),
    ((1, 4, 5, 6, 16), (4, 1, 3, 3, 3), dict(strides=[2, 2, 2], dilations=[2, 1, 1], pads=[2, 1, 1, 0, 1, 1], group=4)),
    ((1, 2, 3, 4, 8), (2, 1, 3, 2, 2), dict(strides=[3, 2, 2], pads=[2, 0, 0, 3, 0, 0], group=2)),
    ((1, 6, 3, 70, 32), (6, 1, 3, 4, 4), dict(strides=[2, 2, 2], pads=[1] * 6, group=6)),
]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", GROUPED_3D, ids=lambda c: f"{c[0]}_{c[1]}")
def test_grouped_rank3(T, case, integer, dtype):
    """Rank-3 grouped calls on the grouped family (the dispatcher must pick it) against
    the oracle on whole outputs; bit-exact on integer inputs."""
    xs, ws, attrs = case
    _log(f"[case] grouped rank 3 x{xs} w{ws} {attrs} integer={integer} {dtype}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer + (dtype == "f32") * 2)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(NPT[dtype])
    w = (gen(ws) * (1 if integer else 0.3)).astype(NPT[dtype])
    b = gen(ws[1] * attrs["group"]).astype(NPT[dtype])
    dev = torch.device("cuda:0")
    assert T.convtranspose_select_kernel(torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev),
                                         torch.from_numpy(b).to(dev), **attrs) == "grouped"
    ref = O.convtranspose(x, w, b, **attrs)
    for kernel in ("grouped", "auto"):
        got = gpu_run(T, x, w, b, attrs, False, kernel)
        check(got, ref, dtype, integer, f"grouped rank 3 {kernel} x{xs} w{ws} {attrs}")


DEPTHWISE_CL = [
    # (x_shape, kernel shape, attrs): channels-last depthwise (group == C), float16, C a
    # multiple of 8: the channels-last bandwidth kernel (ragged tiles, octet tiles of 32,
    # residue classes with fewer taps, rank 1)
    ((2, 64, 9, 13), (4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 32, 7, 10), (3, 3), dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1])),
    ((2, 16, 5, 6), (3, 3), dict(pads=[1, 1, 1, 1])),
    ((1, 264, 6, 9), (4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 40, 5, 7), (2, 2), dict(strides=[2, 2])),
    ((1, 8, 6, 5), (2, 2), dict(pads=[0, 1, 1, 0])),
    ((2, 24, 17), (4,), dict(strides=[2], pads=[1, 1])),
    ((1, 16, 9), (3,), dict(strides=[2], pads=[1, 0], output_padding=[1])),
    ((1, 8, 11), (3,), dict(pads=[1, 1])),
    ((1, 16, 4, 8), (4, 4), dict(strides=[2, 2], auto_pad="SAME_LOWER")),
    # rank 3: the planes of each output plane's first-axis taps (1, 2 or 3), planes
    # outside the input, dilation and stride 3 on the first axis, 64-channel tiles
    ((2, 16, 5, 6, 7), (3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1])),
    ((1, 8, 4, 5, 6), (3, 3, 3), dict(pads=[1] * 6)),
    ((1, 24, 3, 4, 5), (2, 2, 2), dict(strides=[2, 2, 2])),
    ((1, 64, 4, 9, 13), (4, 4, 4), dict(strides=[2, 2, 2], pads=[1] * 6)),
    ((1, 16, 5, 4, 4), (3, 1, 1), dict(strides=[2, 1, 1], dilations=[2, 1, 1], pads=[2, 0, 0, 0, 0, 0])),
    ((1, 8, 3, 4, 5), (3, 2, 2), dict(strides=[3, 2, 2], pads=[2, 0, 0, 3, 0, 0])),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", DEPTHWISE_CL, ids=lambda c: f"{c[0]}_k{c[1]}_{sorted(c[2].items())}")
def test_depthwise_channels_last(T, case, integer):
    """Channels-last depthwise calls on the grouped family's channels-last kernel (the
    dispatcher must pick it) against the oracle on whole outputs, with and without bias."""
    xs, ks, attrs = case
    C = xs[1]
    attrs = dict(attrs, group=C)
    _log(f"[case] depthwise channels-last x{xs} k{ks} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen((C, 1) + tuple(ks)) * (1 if integer else 0.3)).astype(np.float16)
    b = gen(C).astype(np.float16)
    dev = torch.device("cuda:0")
    tx = T.to_channels_last(torch.from_numpy(x).to(dev))
    assert T.convtranspose_select_kernel(tx, torch.from_numpy(w).to(dev), torch.from_numpy(b).to(dev),
                                         channels_last=True, **attrs) == "grouped"
    ref = O.convtranspose(x, w, b, **attrs)
    for kernel in ("grouped", "auto"):
        got = gpu_run(T, x, w, b, attrs, True, kernel)
        check(got, ref, "f16", integer, f"depthwise channels-last {kernel} x{xs} {attrs}")
    got = gpu_run(T, x, w, None, attrs, True, "grouped")
    check(got, O.convtranspose(x, w, None, **attrs), "f16", integer, f"depthwise channels-last no-bias x{xs}")


GROUPED_NC = [
    # (x_shape, C/group, kernel size, attrs): channels-first grouped calls with
    # C/group = M/group in {2, 4, 8}: rows of a multiple of 8 inputs take the depthwise
    # kernel's group mode (a unit stages the group's input planes and writes its output
    # planes), the others and the uncompiled combinations the generic grouped kernel
    ((2, 16, 9, 16), 2, 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 32, 7, 24), 4, 3, dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1])),
    ((2, 64, 5, 8), 8, 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 24, 6, 16), 4, 3, dict(pads=[1, 1, 1, 1])),
    ((1, 16, 5, 16), 2, 6, dict(strides=[2, 2], pads=[2, 2, 2, 2])),
    ((1, 64, 6, 8), 8, 3, dict(pads=[1, 1, 1, 1])),
    ((1, 48, 10, 40), 2, 2, dict(strides=[2, 2])),
    ((1, 16, 150, 64), 2, 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((2, 8, 7, 13), 2, 4, dict(strides=[2, 2], pads=[1, 1, 1, 1])),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", GROUPED_NC, ids=lambda c: f"{c[0]}_g{c[1]}_k{c[2]}")
def test_grouped_channels_first(T, case, integer):
    """Channels-first grouped calls with small groups on the grouped family (the
    dispatcher must pick it) against the oracle on whole outputs, with and without bias;
    bit-exact on integer inputs."""
    xs, cg, k, attrs = case
    C = xs[1]
    attrs = dict(attrs, group=C // cg)
    _log(f"[case] grouped channels-first x{xs} cg{cg} k{k} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen((C, cg, k, k)) * (1 if integer else 0.3)).astype(np.float16)
    b = gen(C).astype(np.float16)
    dev = torch.device("cuda:0")
    assert T.convtranspose_select_kernel(torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev),
                                         torch.from_numpy(b).to(dev), **attrs) == "grouped"
    ref = O.convtranspose(x, w, b, **attrs)
    for kernel in ("grouped", "auto"):
        got = gpu_run(T, x, w, b, attrs, False, kernel)
        check(got, ref, "f16", integer, f"grouped channels-first {kernel} x{xs} cg{cg} {attrs}")
    got = gpu_run(T, x, w, None, attrs, False, "grouped")
    check(got, O.convtranspose(x, w, None, **attrs), "f16", integer, f"grouped channels-first no-bias x{xs}")


GROUPED_CL = [
    # (x_shape, C/group, kernel shape, attrs): channels-last grouped calls with
    # C/group = M/group in {2, 4, 8} on the channels-last bandwidth kernel (every output
    # channel of an octet sums its group's inputs; ragged tiles, tap-less residues)
    ((2, 16, 9, 13), 2, (4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 32, 7, 10), 4, (3, 3), dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1])),
    ((2, 64, 5, 6), 8, (3, 3), dict(pads=[1, 1, 1, 1])),
    ((1, 72, 6, 9), 2, (2, 2), dict(strides=[2, 2])),
    ((1, 128, 5, 7), 8, (4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 24, 6, 5), 4, (1, 1), dict()),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", GROUPED_CL, ids=lambda c: f"{c[0]}_g{c[1]}_k{c[2]}")
def test_grouped_channels_last(T, case, integer):
    """Channels-last grouped calls (C/group = M/group in {2, 4, 8}) on the grouped family's
    channels-last kernel (the dispatcher must pick it) against the oracle on whole
    outputs, with and without bias; bit-exact on integer inputs."""
    xs, cg, ks, attrs = case
    C = xs[1]
    attrs = dict(attrs, group=C // cg)
    _log(f"[case] grouped channels-last x{xs} cg{cg} k{ks} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen((C, cg) + tuple(ks)) * (1 if integer else 0.3)).astype(np.float16)
    b = gen(C).astype(np.float16)
    dev = torch.device("cuda:0")
    tx = T.to_channels_last(torch.from_numpy(x).to(dev))
    assert T.convtranspose_select_kernel(tx, torch.from_numpy(w).to(dev), torch.from_numpy(b).to(dev),
                                         channels_last=True, **attrs) == "grouped"
    ref = O.convtranspose(x, w, b, **attrs)
    for kernel in ("grouped", "auto"):
        got = gpu_run(T, x, w, b, attrs, True, kernel)
        check(got, ref, "f16", integer, f"grouped channels-last {kernel} x{xs} cg{cg} {attrs}")
    got = gpu_run(T, x, w, None, attrs, True, "grouped")
    check(got, O.convtranspose(x, w, None, **attrs), "f16", integer, f"grouped channels-last no-bias x{xs}")


PAIRS = [
    # (x_shape, w_shape, attrs): M/group > 64 and stride 2 on the innermost axis, the
    # channels-first shapes whose two column phases one block computes together when the
    # output width is even and both phases have the same tap count
    ((2, 64, 9, 16), (64, 96, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 16, 264), (16, 72, 4), dict(strides=[2], pads=[1, 1])),  # tiles inside one row, ragged
    ((2, 16, 3, 24), (16, 72, 2, 4), dict(strides=[1, 2], pads=[0, 1, 0, 1])),
    ((2, 24, 6, 24), (24, 130, 3, 6), dict(strides=[2, 2], pads=[1, 2, 0, 2])),  # 3 taps a phase, 2 channel tiles
    ((1, 40, 40), (40, 100, 4), dict(strides=[2], pads=[1, 1])),
    ((1, 16, 3, 5, 16), (16, 72, 3, 3, 4), dict(strides=[1, 2, 2], pads=[1] * 6)),
    ((1, 8, 7, 8), (8, 65, 2, 2), dict(strides=[2, 2], output_padding=[1, 0])),  # one tap a phase
    ((2, 16, 5, 24), (16, 96, 4, 4), dict(strides=[2, 2], pads=[1] * 4, dilations=[1, 3])),  # width 54
    ((1, 16, 6, 40), (16, 80, 3, 5), dict(strides=[2, 2], pads=[1, 2, 1, 2], output_padding=[1, 1])),  # 3 + 2 taps
    ((1, 16, 4, 16), (16, 200, 4, 4), dict(strides=[2, 2], pads=[1] * 4, output_padding=[0, 1])),  # odd width
    ((2, 32, 4, 32), (32, 96, 4, 4), dict(strides=[2, 2], pads=[1] * 4, group=2)),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", PAIRS, ids=lambda c: f"{c[0]}_{c[1]}")
def test_column_phase_pairs(T, case, integer):
    """Dense float16 problems around the column-phase pairing of the MFMA kernel: paired
    shapes (vector and element stores, tiles inside one row, several channel tiles) and
    neighbours that stay unpaired (odd width, unequal tap counts)."""
    xs, ws, attrs = case
    _log(f"[case] pair x{xs} w{ws} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
    b = gen(ws[1] * attrs.get("group", 1)).astype(np.float16)
    ref = O.convtranspose(x, w, b, **attrs)
    # the two block shapes with two wave rows pair column phases; the automatic choice
    # takes a smaller tile for problems this small
    for kernel, tile in (("igemm", "256x256"), ("igemm", "128x256"), ("igemm", None), ("auto", None)):
        with forced_tile(T, tile):
            got = gpu_run(T, x, w, b, attrs, False, kernel)
        assert got is not None, "the implicit-GEMM kernel serves these shapes"
        check(got, ref, "f16", integer, f"pair {kernel} tile {tile} x{xs} w{ws} {attrs}")


TILE_CASES = [
    # (x_shape, w_shape, attrs): several pixel tiles with ragged ends for every block shape,
    # several channel tiles, 1-D / 2-D / 3-D, strides 1-3
    ((2, 64, 20, 36), (64, 48, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((3, 40, 11, 24), (40, 72, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((2, 72, 13, 40), (72, 300, 3, 3), dict(strides=[1, 1], pads=[1, 1, 1, 1])),
    ((1, 32, 5, 9, 16), (32, 24, 3, 3, 3), dict(strides=[1, 1, 1])),
    ((1, 32, 5, 7, 16), (32, 40, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1] * 3)),
    ((2, 48, 600), (48, 130, 5), dict(strides=[3], pads=[2, 1], dilations=[2])),
    ((2, 32, 6, 16), (32, 64, 1, 1), dict(strides=[1, 1])),
    ((1, 16, 4, 5, 18), (16, 40, 3, 3, 3), dict(strides=[1, 1, 1], pads=[2] * 6)),  # rows of 18: 4-byte loads
    ((2, 24, 7, 34), (24, 96, 4, 4), dict(strides=[2, 2], pads=[1] * 4)),             # rows of 34, unpaired
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("tile", ["256x256", "128x256", "64x512", "64x256", "64x128"])
def test_forced_tiles(T, tile, cl, integer):
    """Every block shape of the float16 MFMA kernel on whole outputs."""
    ran = 0
    for xs, ws, attrs in TILE_CASES:
        _log(f"[case] tile {tile} cl={cl} x{xs} w{ws} {attrs} integer={integer}")
        rng = np.random.default_rng(zlib.crc32(repr((xs, ws, attrs)).encode()) + integer)
        gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
        x = gen(xs).astype(np.float16)
        w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
        b = gen(ws[1] * attrs.get("group", 1)).astype(np.float16)
        with forced_tile(T, tile):
            got = gpu_run(T, x, w, b, attrs, cl, "igemm")
        if got is None:
            continue
        ran += 1
        check(got, O.convtranspose(x, w, b, **attrs), "f16", integer, f"tile {tile} x{xs} w{ws} {attrs}")
    assert ran >= len(TILE_CASES) - 2, f"tile {tile} served only {ran} of {len(TILE_CASES)} shapes"


WDMA_CASES = [
    # (x_shape, w_shape, attrs): shapes on which the 256 x 256 block takes its weight tiles
    # through the three-buffer LDS copy ring (four taps per (channel chunk, axis-0 tap)
    # group in every phase with taps; channels-first rows of whole 16-byte vectors)
    ((2, 64, 9, 16), (64, 40, 4, 2), dict(strides=[2, 1], pads=[1, 0, 1, 1])),        # channels-first, unpaired
    ((1, 64, 4, 6, 16), (64, 48, 3, 4, 4), dict(strides=[1, 2, 2], pads=[1] * 6)),    # 3-D: axis-0 taps cropped
    ((1, 200, 6, 8), (200, 72, 4, 4), dict(strides=[2, 2], pads=[1] * 4)),            # partial chunk, padded rows
    ((2, 256, 5, 8), (256, 32, 4, 4), dict(strides=[2, 2], pads=[1] * 4)),            # 16 steps round the ring
    ((1, 16, 3, 8), (16, 16, 4, 4), dict(strides=[2, 2], pads=[1] * 4)),              # one group of four steps
    ((3, 40, 11, 24), (40, 300, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),      # several channel tiles
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("case", WDMA_CASES, ids=lambda c: f"{c[0]}_{c[1]}")
def test_weight_copy_ring(T, case, cl, integer):
    """The 256 x 256 float16 block with weight tiles copied into a ring of three LDS
    buffers two steps ahead, on whole outputs: unpaired and paired channels-first rows,
    channels-last, 3-D with axis-0 taps outside the input, a partial channel chunk,
    padded output-channel rows, several laps of the ring and a single group."""
    xs, ws, attrs = case
    _log(f"[case] weight ring cl={cl} x{xs} w{ws} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + 2 * integer + cl)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
    b = gen(ws[1] * attrs.get("group", 1)).astype(np.float16)
    ref = O.convtranspose(x, w, b, **attrs)
    for _ in range(2):  # a second call finds the ring's buffers holding the first call's tiles
        with forced_tile(T, "256x256"):
            got = gpu_run(T, x, w, b, attrs, cl, "igemm")
        assert got is not None, "the 256 x 256 block serves these shapes"
        check(got, ref, "f16", integer, f"weight ring cl={cl} x{xs} w{ws} {attrs}")


ALLPHASE = [
    # (x_shape, w_shape, attrs): strided calls with >= 4 residue classes and C/group a
    # multiple of 32, on the all-phase kernel (every class of a box in one workgroup)
    ((1, 32, 5, 8, 16), (32, 24, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1])),
    ((2, 64, 4, 9, 8), (64, 64, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6)),
    ((1, 32, 7, 40), (32, 48, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 32, 5, 16), (32, 16, 3, 3), dict(strides=[2, 2], pads=[1, 0, 0, 1])),
    ((1, 64, 3, 6, 8), (64, 16, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6, group=2)),
    ((1, 32, 4, 6, 8), (32, 80, 2, 2, 2), dict(strides=[2, 2, 2])),
    ((1, 32, 6, 8), (32, 40, 3, 3), dict(strides=[2, 2], dilations=[2, 2], pads=[1, 1, 1, 1])),
    ((2, 32, 3, 24), (32, 8, 5, 3), dict(strides=[2, 2], pads=[2, 1, 2, 1], output_padding=[1, 1])),
    # a window too wide for the two-row box (192 channels): the four-row box
    ((1, 192, 3, 5, 8), (192, 16, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6)),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("case", ALLPHASE, ids=lambda c: f"{c[0]}_{c[1]}")
def test_allphase_kernel(T, case, cl, integer):
    """The all-phase MFMA kernel (forced) on whole outputs; bit-exact on integer inputs."""
    xs, ws, attrs = case
    _log(f"[case] allphase cl={cl} x{xs} w{ws} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
    b = gen(ws[1] * attrs.get("group", 1)).astype(np.float16)
    with forced_tile(T, "allphase"):
        got = gpu_run(T, x, w, b, attrs, cl, "igemm")
    assert got is not None, "the all-phase kernel must serve this shape"
    check(got, O.convtranspose(x, w, b, **attrs), "f16", integer, f"allphase x{xs} w{ws} {attrs}")


TAPSPLIT = [
    # (x_shape, w_shape, attrs): stride 1, C/group a multiple of 32, on the tap-split kernel
    # (64 or 96 consecutive output positions x 64 channels per workgroup, taps split over waves)
    ((1, 32, 3, 6, 16), (32, 24, 3, 3, 3), dict()),                                   # rows of 18 flattened
    ((2, 64, 4, 5, 8), (64, 64, 3, 3, 3), dict(pads=[1] * 6)),
    ((1, 32, 2, 3, 72), (32, 40, 2, 3, 3), dict(dilations=[1, 2, 1], pads=[0, 1, 1, 0, 0, 2])),  # runs in a row
    ((1, 64, 5, 16), (64, 96, 3, 3), dict(pads=[1, 1, 1, 1])),                        # two channel tiles
    ((1, 64, 3, 4, 8), (64, 16, 3, 3, 3), dict(group=2)),
    ((2, 32, 40), (32, 32, 5), dict(dilations=[3], pads=[2, 1])),
    ((1, 32, 2, 2, 8), (32, 16, 1, 1, 1), dict()),                                   # one tap: idle waves
    ((1, 128, 3, 6, 32), (128, 64, 3, 3, 3), dict()),                                # C5's channels and rows
    # 1800 boxes of 64 positions or 1200 of 96 (planes of 192 outputs): the planner takes
    # the 96-position boxes, which need fewer rounds of block slots
    ((1, 32, 600, 12, 16), (32, 64, 1, 3, 3), dict(pads=[0, 1, 1, 0, 1, 1])),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("case", TAPSPLIT, ids=lambda c: f"{c[0]}_{c[1]}")
def test_tapsplit_kernel(T, case, cl, integer):
    """The tap-split MFMA kernel (forced) on whole outputs; bit-exact on integer inputs."""
    xs, ws, attrs = case
    _log(f"[case] tapsplit cl={cl} x{xs} w{ws} {attrs} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + integer + 11)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
    b = gen(ws[1] * attrs.get("group", 1)).astype(np.float16)
    with forced_tile(T, "tapsplit"):
        got = gpu_run(T, x, w, b, attrs, cl, "igemm")
    assert got is not None, "the tap-split kernel must serve this shape"
    check(got, O.convtranspose(x, w, b, **attrs), "f16", integer, f"tapsplit x{xs} w{ws} {attrs}")


SINGLE_TAP = [
    # (x_shape, w_shape, attrs): M/group > 64 and at most one tap per axis in every phase
    # (kernels no longer than the stride, 1x1): the implicit-GEMM kernel's instance that
    # double-buffers each step's input tile
    ((2, 64, 9, 16), (64, 96, 1, 1), dict(strides=[1, 1])),
    ((2, 64, 9, 16), (64, 80, 1, 1), dict(strides=[1, 1])),
    ((2, 32, 7, 16), (32, 72, 2, 2), dict(strides=[2, 2])),
    ((1, 40, 6, 24), (40, 130, 3, 3), dict(strides=[3, 3], pads=[0, 1, 0, 1])),
    ((1, 16, 3, 5, 8), (16, 72, 2, 2, 2), dict(strides=[2, 2, 2])),
    ((2, 24, 5, 16), (24, 100, 2, 1), dict(strides=[2, 1], output_padding=[1, 0])),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("case", SINGLE_TAP, ids=lambda c: f"{c[0]}_{c[1]}")
def test_single_tap_groups(T, case, cl, integer):
    xs, ws, attrs = case
    _log(f"[case] single-tap x{xs} w{ws} {attrs} cl={cl} integer={integer}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + 2 * cl + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
    b = gen(ws[1]).astype(np.float16)
    ref = O.convtranspose(x, w, b, **attrs)
    for kernel in ("igemm", "auto"):
        got = gpu_run(T, x, w, b, attrs, cl, kernel)
        assert got is not None, "the implicit-GEMM kernel serves these shapes"
        check(got, ref, "f16", integer, f"single-tap {kernel} x{xs} w{ws} {attrs} cl={cl}")


ACT_CASES = [
    # (name, x_shape, w_shape, attrs, dtype, channels_last, forced kernel)
    ("igemm16_pair", (2, 64, 9, 16), (64, 96, 4, 4), dict(strides=[2, 2], pads=[1] * 4), "f16", False, "igemm"),
    ("igemm16_nc", (2, 32, 6, 16), (32, 80, 3, 3), dict(strides=[2, 2], pads=[1] * 4), "f16", False, "igemm"),
    ("igemm16_cl", (2, 64, 9, 13), (64, 80, 4, 4), dict(strides=[2, 2], pads=[1] * 4), "f16", True, "igemm"),
    ("igemm16_narrow", (1, 32, 4, 5, 8), (32, 24, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6,
                                                                  output_padding=[1] * 3), "f16", False, "igemm"),
    ("igemm32", (3, 24, 77), (24, 40, 5), dict(strides=[3], dilations=[2], pads=[2, 2], output_padding=[1]),
     "f32", False, "igemm"),
    ("igemm32_cl", (2, 16, 6, 7), (16, 24, 3, 3), dict(strides=[2, 2], pads=[1] * 4), "f32", True, "igemm"),
    ("depthwise", (2, 16, 9, 16), (16, 1, 4, 4), dict(strides=[2, 2], pads=[1] * 4, group=16), "f16", False,
     "grouped"),
    ("grouped", (2, 24, 13, 70), (24, 2, 4, 4), dict(strides=[2, 2], pads=[1] * 4, group=12), "f16", False,
     "grouped"),
    ("direct16", (1, 6, 5, 7), (6, 5, 3, 2), dict(strides=[2, 3], pads=[1, 0, 0, 1]), "f16", True, "direct"),
    ("direct32", (2, 4, 9), (4, 3, 4), dict(strides=[2], dilations=[2], pads=[1, 2]), "f32", False, "direct"),
]
ACTS = [("relu", ()), ("leaky_relu", (0.25,)), ("clip", (-2.0, 3.0))]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("case", ACT_CASES, ids=lambda c: c[0])
def test_fused_activation(T, case, integer):
    """The output activation fused into every kernel family's output stage (float32,
    after the bias, before the one rounding) against the oracle's activation of its
    fp64 result; integer-valued inputs bit-exact."""
    name, xs, ws, attrs, dtype, cl, kernel = case
    rng = np.random.default_rng(zlib.crc32(name.encode()) + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(NPT[dtype])
    w = (gen(ws) * (1 if integer else 0.3)).astype(NPT[dtype])
    b = gen(ws[1] * attrs.get("group", 1)).astype(NPT[dtype])
    ref = O.convtranspose(x, w, b, **attrs)
    dev = torch.device("cuda:0")
    tx = torch.from_numpy(x).to(dev)
    if cl:
        tx = T.to_channels_last(tx)
    tw, tb = torch.from_numpy(w).to(dev), torch.from_numpy(b).to(dev)
    for act, params in ACTS:
        _log(f"[case] activation {name} {act} integer={integer}")
        y = T.convtranspose_nd(tx, tw, tb, channels_last=cl, kernel=kernel, activation=act, act_params=params,
                               **attrs)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        check(got, O.activation(ref, act, params), dtype, integer, f"{name} {act}")
    # the default stays the plain operation
    y = T.convtranspose_nd(tx, tw, tb, channels_last=cl, kernel=kernel, **attrs)
    torch.cuda.synchronize()
    check(y.cpu().numpy().astype(np.float64), ref, dtype, integer, f"{name} identity")


# --------------------------------------------------------------------------------------
# the forward convolution with the same W (the adjoint)
# --------------------------------------------------------------------------------------
def conv_gpu_run(T, x, w, b, attrs, cl=False, kernel="auto"):
    dev = torch.device("cuda:0")
    tx = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    if cl:
        tx = T.to_channels_last(tx)
    tw = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    tb = None if b is None else torch.from_numpy(b).to(dev)
    y = T.convolution_nd(tx, tw, tb, channels_last=cl, kernel=kernel, **attrs)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("kernel", ["direct", "auto"])
def test_convolution_random_small(T, kernel, dtype, cl):
    rng = np.random.default_rng(500 + (dtype == "f16") * 2 + cl + 10 * (kernel == "auto"))
    for t in range(40):
        x, w, b, attrs = pins.random_conv_case(rng, auto=(t % 4 == 3))
        integer = t % 2 == 1
        if integer:
            x, w = np.round(x), np.round(w)
            b = None if b is None else np.round(b)
        x, w = x.astype(NPT[dtype]), w.astype(NPT[dtype])
        b = None if b is None else b.astype(NPT[dtype])
        _log(f"[case] conv random #{t} {kernel} {dtype} cl={cl} x{x.shape} w{w.shape} {attrs}")
        got = conv_gpu_run(T, x, w, b, attrs, cl, kernel)
        check(got, O.conv(x, w, b, **attrs), dtype, integer, f"conv random #{t} {attrs}")


CONV_S1 = [
    # (x_shape, w_shape, attrs): stride 1 with C/group and M/group >= 16, the MFMA path
    ((2, 64, 10, 64), (96, 64, 3, 3), dict(pads=[1, 1, 1, 1])),
    ((2, 32, 9, 16), (80, 32, 4, 4), dict(pads=[2, 1, 1, 2])),
    ((1, 48, 12, 24), (64, 48, 3, 3), dict(dilations=[2, 1], auto_pad="SAME_LOWER")),
    ((1, 32, 6, 16), (72, 32, 2, 2), dict(pads=[3, 0, 0, 3])),          # pads beyond the kernel: crops
    ((1, 64, 5, 8, 8), (48, 64, 3, 3, 3), dict(pads=[1] * 6)),
    ((2, 64, 32), (64, 32, 5), dict(pads=[2, 2], group=2)),
]


@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("case", CONV_S1, ids=lambda c: f"{c[0]}_{c[1]}")
def test_convolution_stride1_mfma(T, case, cl, integer):
    xs, ws, attrs = case
    if cl and xs[1] % 8:
        pytest.skip("channels-last MFMA path needs C % 8 == 0")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + 2 * cl + integer)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(np.float16)
    w = (gen(ws) * (1 if integer else 0.1)).astype(np.float16)
    b = gen(ws[0]).astype(np.float16)
    _log(f"[case] conv s1 x{xs} w{ws} {attrs} cl={cl} integer={integer}")
    ref = O.conv(x, w, b, **attrs)
    for kernel in ("igemm", "auto", "direct"):
        got = conv_gpu_run(T, x, w, b, attrs, cl, kernel)
        check(got, ref, "f16", integer, f"conv s1 {kernel} x{xs} w{ws} {attrs}")


CONV_STRIDED = [
    # (x_shape, w_shape, attrs): strided, dilation 1, on the MFMA path through the input
    # phases taken as channels (C/group x stride product >= 16, M/group >= 16); kernels
    # shorter, equal to and longer than the stride, odd phase-copy widths, SAME, groups
    ((2, 16, 16, 30), (48, 16, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),      # the C4 adjoint's form
    ((1, 8, 13, 20), (32, 8, 3, 3), dict(strides=[2, 2], pads=[1, 0, 1, 2])),
    ((1, 16, 9, 24), (40, 16, 5, 3), dict(strides=[3, 2], auto_pad="SAME_UPPER")),
    ((2, 32, 40), (24, 32, 2), dict(strides=[2])),                                    # K = s: one tap per phase
    ((1, 8, 6, 10, 12), (32, 8, 3, 3, 3), dict(strides=[2, 2, 2], pads=[1] * 6)),
    ((2, 32, 12, 12), (32, 16, 4, 4), dict(strides=[2, 2], pads=[1] * 4, group=2)),
]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("integer", [False, True], ids=["float", "int"])
@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("case", CONV_STRIDED, ids=lambda c: f"{c[0]}_{c[1]}")
def test_convolution_strided_mfma(T, case, cl, integer, dtype):
    xs, ws, attrs = case
    if cl and xs[1] % 8:
        pytest.skip("channels-last MFMA path needs C % 8 == 0")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) + 2 * cl + integer + 7)
    gen = (lambda sz: rng.integers(-2, 3, size=sz)) if integer else (lambda sz: rng.normal(size=sz))
    x = gen(xs).astype(NPT[dtype])
    w = (gen(ws) * (1 if integer else 0.1)).astype(NPT[dtype])
    b = gen(ws[0]).astype(NPT[dtype])
    _log(f"[case] conv strided x{xs} w{ws} {attrs} cl={cl} integer={integer} {dtype}")
    ref = O.conv(x, w, b, **attrs)
    for kernel in ("igemm", "auto"):
        got = conv_gpu_run(T, x, w, b, attrs, cl, kernel)
        check(got, ref, dtype, integer, f"conv strided {kernel} x{xs} w{ws} {attrs}")


def test_convolution_adjoint_of_c4_sampled(T):
    """The adjoint of the C4 configuration at full size (stride 2, pads 1, MFMA path
    through the input phases): whole output planes of several (image, channel) pairs
    against the oracle run on that image and channel."""
    wl = W.C4
    _, w, _ = W.make_inputs(wl)
    ys, pads = O.output_shape(wl.x_shape, wl.w_shape, **wl.attrs)
    rng = np.random.default_rng(404)
    a = rng.normal(size=ys).astype(np.float16)
    b = rng.normal(size=wl.w_shape[0]).astype(np.float16)
    attrs = dict(strides=[2, 2], pads=list(pads))
    _log(f"[case] conv adjoint of C4: x{ys} w{wl.w_shape} {attrs}")
    got = conv_gpu_run(T, a, w, b, attrs, False, "igemm")
    assert got.shape == tuple(wl.x_shape)
    for n, m in ((0, 0), (7, 511), (3, 200), (5, 17)):
        ref = O.conv(a[n:n + 1], w[m:m + 1], b[m:m + 1], **attrs)
        check(got[n:n + 1, m:m + 1], ref, "f16", False, f"C4 adjoint plane ({n}, {m})")


def test_convolution_is_the_adjoint(T):
    """<ConvT_W(x), y> = <x, Conv_W(y)> with both operators on the GPU (float32 inputs,
    float64 sums on the host), for the transposed convolution's attributes."""
    rng = np.random.default_rng(77)
    done = 0
    while done < 30:
        x, w, _, attrs = pins.random_case(rng)
        nsp = x.ndim - 2
        _, pads = O.output_shape(x.shape, w.shape, **attrs)
        op = attrs["output_padding"]
        ends = [pads[nsp + a] - op[a] for a in range(nsp)]
        if min(ends) < 0 or min(pads[:nsp]) < 0:
            continue
        x, w = x.astype(np.float32), w.astype(np.float32)
        yt = gpu_run(T, x, w, None, attrs)
        a = rng.normal(size=yt.shape).astype(np.float32)
        back = conv_gpu_run(T, a, w, None, dict(strides=attrs["strides"], dilations=attrs["dilations"],
                                                group=attrs["group"], pads=list(pads[:nsp]) + ends))
        lhs, rhs = float(np.sum(a.astype(np.float64) * yt)), float(np.sum(x.astype(np.float64) * back))
        assert abs(lhs - rhs) <= 1e-4 * (1.0 + np.sum(np.abs(a * yt))), (lhs, rhs, attrs)
        done += 1


def test_convolution_adjoint_of_3d_config_sampled(T):
    """The adjoint of the 3-D stride-1 configuration at full size (Y[2,64,18,34,34] back to
    X[2,128,16,32,32] with W[128,64,3,3,3]) on the MFMA path, checked at sampled outputs."""
    wl = W.C5_S1
    ys, pads = O.output_shape(wl.x_shape, wl.w_shape, **wl.attrs)
    rng = np.random.default_rng(9)
    a = rng.normal(size=ys).astype(np.float16)
    w = (rng.normal(size=wl.w_shape) / np.sqrt(64 * 27)).astype(np.float16)
    b = rng.normal(size=wl.w_shape[0]).astype(np.float16)
    attrs = dict(pads=list(pads))
    got = conv_gpu_run(T, a, w, b, attrs, False, "auto")
    assert got.shape == tuple(wl.x_shape)
    pts = W.make_points(got.shape, 200, seed=3)
    # the oracle at the sampled points: outputs of a box of rows around each point
    for p in pts[:24]:
        n, m = int(p[0]), int(p[1])
        sub = O.conv(a[n:n + 1], w[m:m + 1], b[m:m + 1], **attrs)
        assert abs(got[tuple(p)] - sub[(0, 0) + tuple(p[2:])]) <= 2e-3 * (1 + abs(sub[(0, 0) + tuple(p[2:])]))


def test_repeat_runs_bitwise_identical(T):
    wl = REDUCED[2]
    x, w, b = W.make_inputs(wl)
    a = gpu_run(T, x, w, b, wl.attrs)
    c = gpu_run(T, x, w, b, wl.attrs)
    assert np.array_equal(a, c)


def test_nondefault_stream_and_out_buffer(T):
    wl = REDUCED[2]
    x, w, b = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    tx, tw, tb = (torch.from_numpy(v).to(dev) for v in (x, w, b))
    yshape = T.convtranspose_output_shape(x.shape, w.shape, **wl.attrs)[0]
    out = torch.full(yshape, 7.0, dtype=tx.dtype, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = T.convtranspose_nd(tx, tw, tb, out=out, **wl.attrs)
    s.synchronize()
    assert y.data_ptr() == out.data_ptr()
    check(out.cpu().numpy().astype(np.float64), O.convtranspose(x, w, b, **wl.attrs), "f16", False)


def test_errors_leave_output_untouched(T):
    dev = torch.device("cuda:0")
    x = torch.ones((1, 4, 5, 5), dtype=torch.float16, device=dev)
    w = torch.ones((4, 3, 3, 3), dtype=torch.float16, device=dev)
    out = torch.full((1, 3, 7, 7), 3.0, dtype=torch.float16, device=dev)
    with pytest.raises(T.ConvTransposeError):
        T.convtranspose_nd(x, w, None, out=out, strides=[2, 2])   # shape mismatch
    with pytest.raises(T.ConvTransposeError):
        T.convtranspose_nd(x, w, None, out=out, output_padding=[1, 1])
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


# --------------------------------------------------------------------------------------
# quantized transposed convolution (QLinear scheme): bit-exact against the oracle
# --------------------------------------------------------------------------------------
_TQ = {"uint8": torch.uint8, "int8": torch.int8}


def qgpu_run(T, q, attrs, cl=False, kernel="auto"):
    """The quantized op on the GPU for oracle-style arguments (numpy, NC.. layout);
    returns int64 codes in the logical layout, or None when a forced kernel family does
    not serve the call."""
    dev = torch.device("cuda:0")
    tx = torch.from_numpy(np.ascontiguousarray(q["x"]).astype(np.dtype(str(q["x"].dtype)))).to(dev)
    if cl:
        tx = T.to_channels_last(tx)
    tw = torch.from_numpy(np.ascontiguousarray(q["w"])).to(dev)
    ws = torch.from_numpy(np.asarray(q["w_scale"], dtype=np.float32).reshape(-1)).to(dev)
    wz = torch.from_numpy(np.asarray(q["w_zero_point"]).reshape(-1).astype(q["w"].dtype)).to(dev)
    tb = None if q["bias"] is None else torch.from_numpy(np.asarray(q["bias"], dtype=np.int32)).to(dev)
    try:
        y = T.qlinear_convtranspose_nd(tx, float(q["x_scale"]), int(q["x_zero_point"]), tw, ws, wz,
                                       float(q["y_scale"]), int(q["y_zero_point"]), _TQ[q["y_type"]], tb,
                                       channels_last=cl, kernel=kernel, **attrs)
    except T.ConvTransposeError as e:
        if e.status == 3 and kernel not in ("auto", "direct"):
            return None
        raise
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.int64)


def _as_types(q, tx, tw):
    npt = {"uint8": np.uint8, "int8": np.int8}
    return dict(q, x=q["x"].astype(npt[tx]), w=q["w"].astype(npt[tw]),
                w_zero_point=np.asarray(q["w_zero_point"]).astype(npt[tw]))


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
def test_qlinear_random_small(T, cl):
    """Random 1-D/2-D/3-D problems over every uint8/int8 combination of x, w and y,
    per-tensor and per-channel weight parameters, with and without bias: every output
    code equal to the oracle's."""
    rng = np.random.default_rng(500 + cl)
    for t in range(60):
        q, attrs, (tx, tw) = pins.random_qcase(rng, auto=(t % 4 == 3))
        q = _as_types(q, tx, tw)
        _log(f"[case] qlinear #{t} cl={cl} x{q['x'].shape}:{tx} w{q['w'].shape}:{tw} y:{q['y_type']} {attrs}")
        got = qgpu_run(T, q, attrs, cl)
        ref = O.qconvtranspose(**q, **attrs)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, f"qlinear #{t}: {bad.size} codes differ, first {got.flat[bad[0]]} vs {ref.flat[bad[0]]}"


QREDUCED = [
    W.F4_C4.with_(x_shape=(2, 64, 9, 11), w_shape=(64, 40, 4, 4)),
    W.F4_C4.with_(x_shape=(1, 24, 7, 5), w_shape=(24, 16, 3, 3), x_type="int8", x_zero_point=-3, w_type="uint8",
                  y_type="int8", y_zero_point=5, per_channel=False,
                  attrs=dict(strides=[2, 3], pads=[1, 0, 2, 1], output_padding=[1, 2], dilations=[2, 1])),
    W.F4_C4.with_(x_shape=(2, 16, 3, 4, 5), w_shape=(16, 8, 3, 3, 3), bias_max=0,
                  attrs=dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1] * 3)),
    W.F4_C4.with_(x_shape=(2, 32, 6, 6), w_shape=(32, 4, 2, 2), attrs=dict(strides=[2, 2], group=4)),
]


@pytest.mark.parametrize("cl", [False, True], ids=["nc", "cl"])
@pytest.mark.parametrize("qw", QREDUCED, ids=lambda w: f"{w.x_shape}_{w.x_type}_{w.w_type}_{w.y_type}")
def test_qlinear_reduced_whole_output(T, qw, cl):
    q = W.make_qinputs(qw)
    _log(f"[case] qlinear reduced {qw.x_shape} {qw.attrs} cl={cl}")
    got = qgpu_run(T, q, qw.attrs, cl)
    assert np.array_equal(got, O.qconvtranspose(**q, **qw.attrs))


def test_qlinear_full_size_sampled(T):
    """The quantized C4-shaped workload at full size: whole output planes of the first
    and last image and of the first and last 8 output channels against the oracle run on
    those images and channels only."""
    qw = W.F4_C4
    q = W.make_qinputs(qw)
    _log(f"[case] qlinear full size {qw.x_shape} channels_last={qw.channels_last}")
    got = qgpu_run(T, q, qw.attrs, qw.channels_last)
    M = got.shape[1]
    for n in (0, qw.x_shape[0] - 1):
        for m0 in (0, M - 8):
            sub = dict(q, x=q["x"][n:n + 1], w=q["w"][:, m0:m0 + 8], w_scale=q["w_scale"][m0:m0 + 8],
                       w_zero_point=q["w_zero_point"][m0:m0 + 8], bias=q["bias"][m0:m0 + 8])
            ref = O.qconvtranspose(**sub, **qw.attrs)
            assert np.array_equal(got[n:n + 1, m0:m0 + 8], ref), f"image {n}, channels {m0}..{m0 + 7}"
    lo, hi = W.QRANGE[qw.y_type]
    assert 0.0 < np.mean((got == lo) | (got == hi)) < 0.05   # the recipe's spread: few saturated codes


def test_qlinear_empty_and_tapless(T):
    """An empty batch launches nothing; outputs no tap reaches (kernel shorter than the
    stride) hold the requantized bias."""
    q = W.make_qinputs(W.F4_C4.with_(x_shape=(0, 8, 4, 4), w_shape=(8, 8, 1, 1), attrs=dict(strides=[3, 3])))
    assert qgpu_run(T, q, dict(strides=[3, 3])).shape == (0, 8, 10, 10)
    qw = W.F4_C4.with_(x_shape=(1, 8, 4, 4), w_shape=(8, 8, 1, 1), attrs=dict(strides=[3, 3]))
    q = W.make_qinputs(qw)
    got = qgpu_run(T, q, qw.attrs)
    ref = O.qconvtranspose(**q, **qw.attrs)
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, :, 1, 1], O.requantize(q["bias"], q["x_scale"], q["w_scale"], np.arange(8),
                                                         q["y_scale"], q["y_zero_point"], q["y_type"]))


Q8_CASES = [
    # (x_shape, w_shape, attrs): C/group a multiple of 16 (the int8 MFMA kernel's
    # channels-last 16-byte vectors); ragged output channels and pixel tiles, a second
    # partial channel step (C/group = 160), groups, 1-D / 2-D / 3-D
    ((2, 64, 9, 12), (64, 40, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 32, 5, 9, 11), (32, 24, 3, 3, 3), dict(strides=[1, 1, 1])),
    ((1, 48, 6, 7), (48, 72, 3, 3), dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1])),
    ((2, 32, 50), (32, 20, 5), dict(strides=[3], dilations=[2], pads=[2, 1])),
    ((2, 64, 6, 6), (64, 8, 2, 2), dict(strides=[2, 2], group=2)),
    ((1, 160, 5, 6), (160, 24, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 256, 8, 8), (256, 64, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1])),
    ((1, 16, 5, 6), (16, 32, 1, 2), dict(strides=[3, 2], output_padding=[2, 1])),   # phases no tap reaches
]


@pytest.mark.parametrize("cl", [True, False], ids=["cl", "nc"])
@pytest.mark.parametrize("tile", [None, "256x256", "128x256", "64x128"])
def test_qlinear_int8_mfma(T, tile, cl):
    """The int8 MFMA implicit GEMM on whole outputs, every uint8/int8 combination:
    symmetric weights (no input-sum correction) and arbitrary zero points (per-channel
    weight zero points exercise the per-pixel input sums); channels-first tensors go
    through the layout transposes."""
    rng = np.random.default_rng(900 + (0 if tile is None else T.IGEMM_TILES.index(tile) + 1) + 10 * (not cl))
    ran = 0
    for ci, (xs, ws, attrs) in enumerate(Q8_CASES):
        for general in (False, True):
            tx, tw, ty = (str(rng.choice(["uint8", "int8"])) for _ in range(3))
            M = ws[1] * attrs.get("group", 1)
            nq = M if (general or ci % 2) else 1
            lo, hi = pins.QT[tx]
            x = rng.integers(lo, hi + 1, size=xs)
            x_zp = int(rng.integers(lo, hi + 1))
            lo, hi = pins.QT[tw]
            w = rng.integers(lo, hi + 1, size=ws)
            w_zp = rng.integers(lo, hi + 1, size=nq) if general else np.full(nq, 0 if tw == "int8" else 128)
            depth = xs[1] // attrs.get("group", 1) * 4
            q = _as_types(dict(x=x, w=w, x_scale=np.float32(0.02), x_zero_point=x_zp,
                               w_scale=rng.uniform(0.5, 1.5, size=nq).astype(np.float32) * np.float32(0.01),
                               w_zero_point=w_zp, y_scale=np.float32(0.0004 * np.sqrt(depth) * 74 * 74 / 50),
                               y_zero_point=int(rng.integers(*pins.QT[ty])), y_type=ty,
                               bias=rng.integers(-50000, 50001, size=M) if ci % 3 else None), tx, tw)
            _log(f"[case] int8 mfma tile {tile} cl={cl} #{ci} general={general} x{xs}:{tx} w{ws}:{tw} y:{ty} {attrs}")
            with forced_tile(T, tile):
                got = qgpu_run(T, q, attrs, cl=cl, kernel="igemm")
            if got is None:
                continue
            ran += 1
            ref = O.qconvtranspose(**q, **attrs)
            bad = np.flatnonzero(got != ref)
            assert bad.size == 0, f"int8 mfma #{ci}: {bad.size} of {got.size} codes differ, first at " \
                                  f"{np.unravel_index(bad[0], got.shape)}: {got.flat[bad[0]]} vs {ref.flat[bad[0]]}"
    assert ran >= len(Q8_CASES), f"the int8 kernel served only {ran} cases"


def test_prepared_calls_repeat_the_direct_call(T):
    """PreparedCall (arguments marshalled once) gives, call after call, exactly what the
    direct call gives, for the forward convolution and the quantized operation."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(31)
    a = torch.from_numpy(rng.normal(size=(2, 16, 10, 16)).astype(np.float16)).to(dev)
    w = torch.from_numpy((rng.normal(size=(48, 16, 4, 4)) * 0.1).astype(np.float16)).to(dev)
    b = torch.from_numpy(rng.normal(size=48).astype(np.float16)).to(dev)
    attrs = dict(strides=[2, 2], pads=[1, 1, 1, 1])
    want = T.convolution_nd(a, w, b, **attrs).clone()
    call = T.PreparedCall(T.convolution_nd, a, w, b, **attrs)
    for _ in range(3):
        assert torch.equal(call(), want)
    qw = W.F4_C4.with_(x_shape=(1, 32, 6, 8), w_shape=(32, 24, 4, 4))
    q = W.make_qinputs(qw)
    args = dict(x=torch.from_numpy(q["x"]).to(dev), x_scale=float(q["x_scale"]), x_zero_point=int(q["x_zero_point"]),
                w=torch.from_numpy(q["w"]).to(dev), w_scale=torch.from_numpy(q["w_scale"]).to(dev),
                w_zero_point=torch.from_numpy(q["w_zero_point"]).to(dev), y_scale=float(q["y_scale"]),
                y_zero_point=int(q["y_zero_point"]), y_dtype=torch.uint8, bias=torch.from_numpy(q["bias"]).to(dev))
    want = T.qlinear_convtranspose_nd(**args, **qw.attrs).clone()
    call = T.PreparedCall(T.qlinear_convtranspose_nd, **args, **qw.attrs)
    for _ in range(3):
        assert torch.equal(call(), want)
    torch.cuda.synchronize()
