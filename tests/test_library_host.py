"""Host-side checks of libconvtranspose.so that need no GPU: exported symbols, the
attribute resolver and useful-MAC count against the oracle's independent ones, and
argument validation (every case here fails validation or has an empty output, so no
kernel is ever launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import pins
import workloads as W
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def T():
    import transposed_convolution_amd as T
    if not os.path.exists(T.library_path()):
        from transposed_convolution_amd import build
        build.build()
    T.load_library()
    return T


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(T):
    names = _declared_functions()
    assert "convtranspose_nd" in names and len(names) >= 6
    lib = ctypes.CDLL(T.library_path())
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def _random_attrs(rng, nsp):
    at = {}
    if rng.random() < 0.8:
        at["strides"] = [int(v) for v in rng.integers(1, 4, size=nsp)]
    if rng.random() < 0.6:
        at["dilations"] = [int(v) for v in rng.integers(1, 4, size=nsp)]
    s = at.get("strides", [1] * nsp)
    d = at.get("dilations", [1] * nsp)
    if rng.random() < 0.5:
        at["output_padding"] = [int(rng.integers(0, max(a, b) + (1 if rng.random() < 0.1 else 0)))
                                for a, b in zip(s, d)]
    mode = rng.choice(["NOTSET", "NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"])
    at["auto_pad"] = str(mode)
    if mode == "NOTSET" or rng.random() < 0.05:
        if rng.random() < 0.8:
            at["pads"] = [int(v) for v in rng.integers(-1 if rng.random() < 0.05 else 0, 4, size=2 * nsp)]
    if rng.random() < 0.15:
        at["output_shape"] = [int(v) for v in rng.integers(0, 12, size=nsp)]
    if rng.random() < 0.1:
        at["kernel_shape"] = [int(v) for v in rng.integers(1, 4, size=nsp)]
    at["group"] = int(rng.choice([1, 1, 2, 3, 0]) if rng.random() < 0.95 else -1)
    return at


def test_resolver_matches_oracle(T):
    rng = np.random.default_rng(101)
    agree_ok = agree_err = 0
    for _ in range(3000):
        nsp = int(rng.integers(1, 4))
        C = int(rng.integers(0, 7))
        xs = (int(rng.integers(0, 3)), C) + tuple(int(v) for v in rng.integers(0, 7, size=nsp))
        ws = (C if rng.random() < 0.97 else C + 1, int(rng.integers(1, 4))) + tuple(
            int(v) for v in rng.integers(1, 5, size=nsp))
        at = _random_attrs(rng, nsp)
        try:
            want = O.output_shape(xs, ws, **at)
        except O.OracleError:
            want = None
        try:
            got = T.convtranspose_output_shape(xs, ws, **at)
        except T.ConvTransposeError as e:
            assert e.status == 1
            got = None
        if want is None:
            assert got is None, (xs, ws, at, got)
            agree_err += 1
        else:
            assert got is not None, (xs, ws, at, T.convtranspose_last_error())
            assert tuple(got[0]) == tuple(want[0]) and list(got[1]) == list(want[1]), (xs, ws, at)
            assert T.convtranspose_useful_macs(xs, ws, **at) == O.useful_macs(xs, ws, **at)
            agree_ok += 1
    assert agree_ok > 800 and agree_err > 300


def test_config_shapes_and_macs(T):
    for wl in W.CONFIGS.values():
        assert T.convtranspose_output_shape(wl.x_shape, wl.w_shape, **wl.attrs)[0] == \
            O.output_shape(wl.x_shape, wl.w_shape, **wl.attrs)[0]
        assert T.convtranspose_useful_macs(wl.x_shape, wl.w_shape, **wl.attrs) == \
            O.useful_macs(wl.x_shape, wl.w_shape, **wl.attrs)


def _raw_call(T, kernel=0, dtype=1, nsp=2, cl=0, x=256, xs=(1, 4, 5, 5), w=512, ws=(4, 3, 3, 3),
              bias=None, y=1024, ys=None, attrs=None):
    lib = T.load_library()
    attrs = attrs or {}
    if ys is None:
        ys = T.convtranspose_output_shape(xs, ws, **attrs)[0]
    at = T._attr_args(nsp, **attrs)
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return lib.convtranspose_nd_with_kernel(kernel, dtype, nsp, cl, vp(x), T._i64(xs), vp(w), T._i64(ws),
                                            vp(bias), vp(y), T._i64(ys), *at, None, 0, None)


def test_validation_errors_launch_nothing(T):
    assert _raw_call(T, ys=(1, 3, 7, 8)) == 2                       # y_shape mismatch
    assert _raw_call(T, dtype=7) == 3                                # dtype not served
    assert _raw_call(T, x=257) == 1                                  # misaligned fp16 pointer
    assert _raw_call(T, x=None) == 1                                 # NULL x with data
    assert _raw_call(T, y=None) == 1                                 # NULL y
    assert _raw_call(T, cl=2) == 1
    assert _raw_call(T, kernel=9) == 1
    assert _raw_call(T, nsp=2, attrs=dict(strides=[0, 1]), ys=(1, 3, 7, 7)) == 1
    assert "stride" in T.convtranspose_last_error()
    assert _raw_call(T, kernel=2) == 3                               # group 1: not a grouped problem
    assert _raw_call(T, kernel=3, dtype=0, attrs=dict(strides=[17, 1])) == 3  # stride beyond the MFMA plan
    # empty outputs: OK with nothing launched (no device is touched)
    assert _raw_call(T, xs=(0, 4, 5, 5), x=None, y=None) == 0
    assert T.convtranspose_last_error() == ""


def _fused_call(T, act, p0=0.0, p1=0.0, **kw):
    """convtranspose_nd_fused with the arguments of _raw_call and an activation."""
    lib = T.load_library()
    xs, ws = (1, 4, 5, 5), (4, 3, 3, 3)
    ys = kw.get("ys") or T.convtranspose_output_shape(xs, ws)[0]
    at = T._attr_args(2)
    vp = ctypes.c_void_p
    return lib.convtranspose_nd_fused(0, 1, 2, 0, vp(256), T._i64(xs), vp(512), T._i64(ws), None, vp(1024),
                                      T._i64(ys), *at, act, p0, p1, None, 0, None)


def test_activation_arguments_validated_before_launch(T):
    inf, nan = float("inf"), float("nan")
    assert _fused_call(T, 9) == 1 and "activation" in T.convtranspose_last_error()
    assert _fused_call(T, -1) == 1
    assert _fused_call(T, 2, inf) == 1 and "slope" in T.convtranspose_last_error()   # leaky ReLU slope
    assert _fused_call(T, 2, nan) == 1
    assert _fused_call(T, 3, 1.0, 0.0) == 1 and "clip" in T.convtranspose_last_error()  # lower > upper
    assert _fused_call(T, 3, nan, 1.0) == 1
    assert _fused_call(T, 3, 0.0, inf) == 1
    # a valid activation still meets the ordinary validation (y_shape mismatch, nothing launched)
    assert _fused_call(T, 1, ys=(1, 3, 7, 8)) == 2
    assert _fused_call(T, 3, -1.0, 1.0, ys=(1, 3, 7, 8)) == 2
    assert set(T.ACTIVATIONS) == set(O.ACTIVATIONS)


def test_convolution_resolver_matches_oracle(T):
    rng = np.random.default_rng(41)
    for t in range(400):
        x, w, b, attrs = pins.random_conv_case(rng, auto=(t % 3 == 2))
        assert T.convolution_output_shape(x.shape, w.shape, **attrs) == \
            tuple(map(tuple, O.conv_output_shape(x.shape, w.shape, **attrs)))
    # the adjoint shapes: the convolution maps the benchmark outputs back to the inputs
    for wl in W.CONFIGS.values():
        ys, pads = T.convtranspose_output_shape(wl.x_shape, wl.w_shape, **wl.attrs)
        nsp = len(wl.x_shape) - 2
        op = wl.attrs.get("output_padding") or [0] * nsp
        cp = list(pads[:nsp]) + [pads[nsp + a] - op[a] for a in range(nsp)]
        if min(cp) < 0:
            continue
        got, _ = T.convolution_output_shape(ys, wl.w_shape, strides=wl.attrs.get("strides"),
                                            dilations=wl.attrs.get("dilations"), pads=cp,
                                            group=wl.attrs.get("group", 1))
        assert got == tuple(wl.x_shape), (wl.name, got)


def test_convolution_validation_launches_nothing(T):
    lib = T.load_library()
    vp = ctypes.c_void_p

    def call(xs=(1, 4, 6, 6), ws=(6, 2, 3, 3), ys=None, kernel=0, dtype=1, cl=0, **attrs):
        attrs.setdefault("group", 2)
        if ys is None:
            ys = T.convolution_output_shape(xs, ws, **attrs)[0]
        return lib.convolution_nd(kernel, dtype, 2, cl, vp(256), T._i64(xs), vp(512), T._i64(ws), None, vp(1024),
                                  T._i64(ys), *T._conv_attr_args(2, **attrs), None)

    assert call(ys=(1, 6, 4, 5)) == 2
    assert call(dtype=5) == 3
    assert call(kernel=2) == 1                                     # the grouped family is not a conv path
    assert call(kernel=3) == 3                                     # MFMA path: C/group 2 is below its minimum
    assert call(cl=3) == 1
    assert call(ws=(6, 3, 3, 3), ys=(1, 6, 4, 4)) == 1 and "C / group" in T.convtranspose_last_error()
    assert call(ys=(1, 6, 4, 4), pads=[1, 1, 1, 1], auto_pad="VALID") == 1
    assert call(ys=(1, 6, 4, 4), strides=[0, 1]) == 1
    assert call(xs=(0, 4, 6, 6)) == 0                              # empty output: nothing launched
    assert T.convtranspose_last_error() == ""


def test_dispatcher_choices(T):
    lib = T.load_library()

    def pick(wl, dtype=1, cl=0):
        at = T._attr_args(wl.nsp, **wl.attrs)
        k = lib.convtranspose_select_kernel(dtype, wl.nsp, cl, ctypes.c_void_p(256), T._i64(wl.x_shape),
                                            ctypes.c_void_p(256), T._i64(wl.w_shape),
                                            ctypes.c_void_p(256) if wl.has_bias else None,
                                            ctypes.c_void_p(256), *at)
        return T.convtranspose_kernel_name(k)

    assert pick(W.C1, dtype=0) == "direct"
    assert pick(W.C2, dtype=0) == "igemm"     # float32 implicit GEMM on MFMA
    assert pick(W.C3) == "grouped"            # the depthwise specialisation of the grouped family
    assert pick(W.C3_NHWC, cl=1) == "grouped"  # its channels-last kernel
    assert pick(W.C4) == "igemm"
    assert pick(W.C4_NHWC, cl=1) == "igemm"
    for wl in (W.C5_S1, W.C5_S1_P1, W.C5_S2):
        assert pick(wl) == "igemm", wl.name


def _select(T, dtype, xs, ws, cl=0, **attrs):
    lib = T.load_library()
    at = T._attr_args(len(xs) - 2, **attrs)
    k = lib.convtranspose_select_kernel(dtype, len(xs) - 2, cl, ctypes.c_void_p(256), T._i64(xs),
                                        ctypes.c_void_p(256), T._i64(ws), ctypes.c_void_p(256),
                                        ctypes.c_void_p(256), *at)
    return T.convtranspose_kernel_name(k)


@pytest.mark.parametrize("dtype", [0, 1], ids=["f32", "f16"])
@pytest.mark.parametrize("cl", [0, 1], ids=["nc", "cl"])
@pytest.mark.parametrize("case", [
    ((1, 16, 4, 0), (16, 16, 4, 4), dict(strides=[2, 2])),
    ((1, 16, 0, 8), (16, 16, 4, 4), dict(strides=[2, 2], pads=[0, 1, 0, 1])),
    ((2, 32, 0), (32, 16, 3), dict(strides=[2])),
    ((1, 16, 3, 0, 4), (16, 16, 3, 3, 3), dict(strides=[2, 2, 2])),
    ((1, 64, 0, 3), (64, 32, 3, 3), dict(strides=[2, 2], group=2)),
], ids=["2d_last_axis", "2d_first_axis", "1d", "3d", "grouped_2d"])
def test_empty_input_never_reaches_mfma(T, case, cl, dtype):
    """An input with a spatial size of 0 but a non-empty output (bias alone) with C/group
    >= 16 must not be routed to the MFMA kernels, whose operand loads read through x's
    base pointer (README Files: the empty-input case has a route of its own)."""
    xs, ws, attrs = case
    ys, _ = T.convtranspose_output_shape(xs, ws, **attrs)
    assert int(np.prod(ys)) > 0
    assert _select(T, dtype, xs, ws, cl, **attrs) == "direct"


@pytest.mark.parametrize("dtype", [0, 1], ids=["f32", "f16"])
@pytest.mark.parametrize("cl", [0, 1], ids=["nc", "cl"])
def test_empty_input_forward_convolution_not_mfma(T, cl, dtype):
    """The stride-1 forward convolution with an empty spatial input and padding (a bias-only
    output) is refused by the MFMA path before any launch (CT_EUNSUPPORTED when forced)."""
    lib = T.load_library()
    vp = ctypes.c_void_p
    xs, ws, attrs = (1, 16, 0, 6), (32, 16, 3, 3), dict(pads=[2, 1, 2, 1])
    ys = T.convolution_output_shape(xs, ws, **attrs)[0]
    assert int(np.prod(ys)) > 0
    st = lib.convolution_nd(3, dtype, 2, cl, vp(256), T._i64(xs), vp(512), T._i64(ws), None, vp(1024),
                            T._i64(ys), *T._conv_attr_args(2, **attrs), None)
    assert st == 3, T.convtranspose_last_error()


def test_igemm_tile_control(T):
    """The block-shape override of the float16 MFMA kernel: validated, read back, and
    honoured by the dispatcher (host-side planning only; nothing is launched)."""
    lib = T.load_library()

    def pick(wl, cl=0):
        at = T._attr_args(wl.nsp, **wl.attrs)
        k = lib.convtranspose_select_kernel(1, wl.nsp, cl, ctypes.c_void_p(256), T._i64(wl.x_shape),
                                            ctypes.c_void_p(256), T._i64(wl.w_shape), ctypes.c_void_p(256),
                                            ctypes.c_void_p(256), *at)
        return T.convtranspose_kernel_name(k)

    assert lib.convtranspose_igemm_tile() == -1
    for bad in (-2, len(T.IGEMM_TILES)):
        assert lib.convtranspose_set_igemm_tile(bad) == 1 and "tile" in T.convtranspose_last_error()
        assert lib.convtranspose_igemm_tile() == -1
    try:
        for t, name in enumerate(T.IGEMM_TILES):
            T.set_igemm_tile(name)
            assert lib.convtranspose_igemm_tile() == t and T.igemm_tile() == name
        # C5 stride 1 (J = 34 x 34 output planes): the 256 x 256 tile's input halo does not
        # fit one block's loads, the automatic choice and the 64 x 128 tile serve it
        T.set_igemm_tile("256x256")
        assert pick(W.C5_S1) != "igemm"
        T.set_igemm_tile("64x128")
        assert pick(W.C5_S1) == "igemm"
    finally:
        T.set_igemm_tile(None)
    assert pick(W.C5_S1) == "igemm" and T.igemm_tile() is None


def test_igemm_channels_first_row_widths(T):
    """Channels-first input rows of any even width go to the MFMA kernel (16-byte loads
    when the width is a multiple of 8, 4-byte loads otherwise); odd widths do not."""
    lib = T.load_library()
    for width, ok in ((32, True), (34, True), (18, True), (6, True), (33, False), (7, False)):
        wl = W.C5_S1.with_(x_shape=(2, 64, 18, 34, width), w_shape=(64, 128, 3, 3, 3))
        at = T._attr_args(wl.nsp, **wl.attrs)
        k = lib.convtranspose_select_kernel(1, wl.nsp, 0, ctypes.c_void_p(256), T._i64(wl.x_shape),
                                            ctypes.c_void_p(256), T._i64(wl.w_shape), ctypes.c_void_p(256),
                                            ctypes.c_void_p(256), *at)
        assert (T.convtranspose_kernel_name(k) == "igemm") == ok, (width, T.convtranspose_kernel_name(k))


def test_qlinear_validation_launches_nothing(T):
    """Argument checks of the quantized entry point, all before any launch (the fake
    device pointers are never dereferenced), and an empty output that launches nothing."""
    lib = T.load_library()
    P = ctypes.c_void_p(256)
    U8, I8 = 3, 2

    def call(xt=U8, wt=I8, yt=U8, xs=(1, 4, 3, 3), ws=(4, 2, 3, 3), ys=(1, 2, 7, 7), x_scale=0.1, x_zp=128,
             y_scale=0.2, y_zp=0, wq=1, kernel=0, strides=(2, 2)):
        at = T._attr_args(2, strides=list(strides))
        return lib.qlinear_convtranspose_nd(kernel, 2, 0, P, xt, T._i64(xs), x_scale, x_zp, P, wt, T._i64(ws), P, P,
                                            wq, None, P, yt, T._i64(ys), y_scale, y_zp, *at, None)

    assert call(xt=1) == 3 and "CT_UINT8 or CT_INT8" in T.convtranspose_last_error()
    assert call(yt=0) == 3
    assert call(kernel=3) == 3                                     # C = 4: the int8 MFMA kernel needs 16
    assert call(x_scale=0.0) == 1 and call(x_scale=float("inf")) == 1 and call(y_scale=-1.0) == 1
    assert call(x_zp=256) == 1 and call(xt=I8, x_zp=128) == 1 and call(yt=I8, y_zp=-129) == 1
    assert call(wq=3) == 1 and "length 1 or M" in T.convtranspose_last_error()
    assert call(ys=(1, 2, 6, 7)) == 2                              # y_shape differs from the resolved shape
    assert call(xs=(0, 4, 3, 3), ys=(0, 2, 7, 7)) == 0             # empty output: nothing launched
    assert T.convtranspose_last_error() == ""


def test_random_cases_resolve_identically(T):
    rng = np.random.default_rng(5)
    for t in range(300):
        x, w, b, attrs = pins.random_case(rng, auto=(t % 3 == 0))
        assert T.convtranspose_output_shape(x.shape, w.shape, **attrs) == \
            tuple(tuple(v) for v in O.output_shape(x.shape, w.shape, **attrs))


def test_noalloc_rejects_oversized_workspace(T):
    """The allocation-free entry point refuses, before touching any device, a call whose
    workspace exceeds its fixed array (and names the limit)."""
    lib = T.load_library()
    assert lib.convtranspose_noalloc_max_workspace() == 16 << 20
    xs, ws, attrs = (1, 1024, 4, 4), (1024, 1024, 4, 4), dict(strides=[2, 2])
    ys, _ = T.convtranspose_output_shape(xs, ws, **attrs)
    at = T._attr_args(2, **attrs)
    P = ctypes.c_void_p(256)
    st = lib.convtranspose_nd_noalloc(0, 1, 2, 0, P, T._i64(xs), P, T._i64(ws), None, P, T._i64(ys), *at, None)
    assert st == 1 and "16777216" in T.convtranspose_last_error()
    # invalid arguments: the status the call itself gives, nothing launched
    st = lib.convtranspose_nd_noalloc(0, 1, 2, 0, P, T._i64(xs), P, T._i64((1000, 1024, 4, 4)), None, P,
                                      T._i64(ys), *at, None)
    assert st == 1


def test_out_of_range_enum_arguments_are_refused(T):
    """Enum arguments arrive from C as any int: values outside each enum are refused with
    a status (unknown element type: CT_EUNSUPPORTED; other enums: CT_EINVAL) before
    anything else happens (nothing launched)."""
    lib = T.load_library()
    P = ctypes.c_void_p(256)
    xs, ws, ys = (1, 4, 5, 5), (4, 2, 3, 3), (1, 2, 11, 11)

    def nd(kernel=0, dtype=1, auto_pad=0, act=0):
        at = list(T._attr_args(2, strides=[2, 2]))
        at[0] = auto_pad
        return lib.convtranspose_nd_fused(kernel, dtype, 2, 0, P, T._i64(xs), P, T._i64(ws), None, P, T._i64(ys),
                                          *at, act, 0.0, 0.0, None, 0, None)

    for kw, want in ((dict(kernel=9), 1), (dict(kernel=-3), 1), (dict(dtype=-1), 3), (dict(dtype=77), 3),
                     (dict(auto_pad=99), 1), (dict(auto_pad=-2), 1), (dict(act=8), 1), (dict(act=-1), 1)):
        assert nd(**kw) == want, kw
        assert T.convtranspose_last_error()
    at = list(T._attr_args(2, strides=[2, 2]))
    at[0] = 42
    out = (ctypes.c_int64 * 4)()
    assert lib.convtranspose_output_shape(2, T._i64(xs), T._i64(ws), *at, out, None) == 1
    assert lib.convtranspose_select_kernel(5, 2, 0, P, T._i64(xs), P, T._i64(ws), None, P,
                                           *T._attr_args(2, strides=[2, 2])) == -1
