"""MI355X-native N-D transposed convolution (ONNX ConvTranspose).

This package is a thin Python binding over ``libconvtranspose.so``, whose C ABI is
declared in ``include/convtranspose.h``.  The binding only marshals arguments: it
resolves the output shape through the library, allocates Y with torch (torch supplies
device memory and the stream) and passes raw pointers.  Every step of the operator
runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library raises.

Operator: webgpu-kernels "ai.onnx.ConvTranspose" README (Description, Inputs,
Outputs, Attributes, Type constraints); channels-last input/output as on the ClikaRT
"conv_transpose" API page.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch  # first: the library then binds to the HIP runtime torch has loaded

__all__ = [
    "ConvTransposeError", "ConvTransposePlan", "convtranspose_nd", "convtranspose_profile_events", "convtranspose_output_shape",
    "convtranspose_useful_macs", "convtranspose_select_kernel", "convtranspose_last_error",
    "convtranspose_kernel_name", "library_path", "load_library", "channels_last_empty",
    "to_channels_last", "KERNELS", "ACTIVATIONS", "convolution_nd", "convolution_output_shape",
    "IGEMM_TILES", "set_igemm_tile", "igemm_tile", "qlinear_convtranspose_nd", "PreparedCall",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# CT_LIBRARY_PATH selects another build of the same library (e.g. one with host-side
# sanitizers); it must exist like the default one -- there is no fallback.
_LIB_PATH = os.environ.get("CT_LIBRARY_PATH") or os.path.join(_HERE, "libconvtranspose.so")
AUTO_PAD = {"NOTSET": 0, "SAME_UPPER": 1, "SAME_LOWER": 2, "VALID": 3}
KERNELS = {"auto": 0, "direct": 1, "grouped": 2, "igemm": 3, "none": 4}
# output activation fused into the kernels' output stage (ct_activation), with the number
# of parameters each takes: leaky_relu (slope,), clip (lower, upper)
ACTIVATIONS = {"identity": (0, 0), "relu": (1, 0), "leaky_relu": (2, 1), "clip": (3, 2)}
_DTYPES = {torch.float32: 0, torch.float16: 1}
_STATUS = {0: "CT_OK", 1: "CT_EINVAL", 2: "CT_ESHAPE", 3: "CT_EUNSUPPORTED", 4: "CT_EDEVICE"}
_lib = None


class ConvTransposeError(RuntimeError):
    """A library call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libconvtranspose.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(_LIB_PATH)
    i64p = ctypes.POINTER(ctypes.c_int64)
    vp = ctypes.c_void_p
    attrs = [ctypes.c_int, i64p, i64p, i64p, i64p, i64p, i64p, ctypes.c_int64]
    lib.convtranspose_output_shape.argtypes = [ctypes.c_int, i64p, i64p] + attrs + [i64p, i64p]
    lib.convtranspose_useful_macs.argtypes = [ctypes.c_int, i64p, i64p] + attrs + [
        ctypes.POINTER(ctypes.c_double)]
    call = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64p, vp, i64p, vp, vp, i64p] + attrs
    lib.convtranspose_nd.argtypes = call + [vp]
    lib.convtranspose_nd_with_kernel.argtypes = [ctypes.c_int] + call + [vp, ctypes.c_size_t, vp]
    lib.convtranspose_nd_fused.argtypes = [ctypes.c_int] + call + [ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                                                   vp, ctypes.c_size_t, vp]
    lib.convtranspose_nd_noalloc.argtypes = [ctypes.c_int] + call + [vp]
    lib.convtranspose_nd_noalloc.restype = ctypes.c_int
    lib.convtranspose_noalloc_max_workspace.argtypes = []
    lib.convtranspose_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.convtranspose_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                                 i64p, i64p] + attrs + [ctypes.POINTER(ctypes.c_size_t)]
    lib.convtranspose_select_kernel.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64p,
                                                vp, i64p, vp, vp] + attrs
    for fn in ("convtranspose_output_shape", "convtranspose_useful_macs", "convtranspose_nd",
               "convtranspose_nd_with_kernel", "convtranspose_nd_fused", "convtranspose_select_kernel",
               "convtranspose_workspace_size"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.convtranspose_last_error.restype = ctypes.c_char_p
    lib.convtranspose_last_error.argtypes = []
    lib.convtranspose_kernel_name.restype = ctypes.c_char_p
    lib.convtranspose_kernel_name.argtypes = [ctypes.c_int]
    cattrs = [ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int64]  # forward convolution attributes
    lib.convolution_output_shape.argtypes = [ctypes.c_int, i64p, i64p] + cattrs + [i64p, i64p]
    lib.convolution_output_shape.restype = ctypes.c_int
    lib.convolution_nd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64p, vp, i64p, vp,
                                   vp, i64p] + cattrs + [vp]
    lib.convolution_nd.restype = ctypes.c_int
    lib.convtranspose_profile_events.argtypes = [vp, vp]
    lib.convtranspose_profile_events.restype = ctypes.c_int
    c_i32, c_f32 = ctypes.c_int32, ctypes.c_float
    lib.qlinear_convtranspose_nd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, i64p, c_f32,
                                             c_i32, vp, ctypes.c_int, i64p, vp, vp, ctypes.c_int64, vp, vp,
                                             ctypes.c_int, i64p, c_f32, c_i32] + attrs + [vp]
    lib.qlinear_convtranspose_nd.restype = ctypes.c_int
    lib.convtranspose_set_igemm_tile.argtypes = [ctypes.c_int]
    lib.convtranspose_set_igemm_tile.restype = ctypes.c_int
    lib.convtranspose_igemm_tile.argtypes = []
    lib.convtranspose_igemm_tile.restype = ctypes.c_int
    _lib = lib
    return lib


def convtranspose_last_error() -> str:
    return load_library().convtranspose_last_error().decode(errors="replace")


def convtranspose_kernel_name(kernel: int) -> str:
    return load_library().convtranspose_kernel_name(int(kernel)).decode()


def _i64(v: Optional[Sequence[int]]):
    if v is None:
        return None
    v = [int(t) for t in v]
    return (ctypes.c_int64 * max(1, len(v)))(*v)


def _attr_args(nsp, auto_pad="NOTSET", strides=None, dilations=None, pads=None, output_padding=None,
               output_shape=None, kernel_shape=None, group=1):
    lens = dict(strides=nsp, dilations=nsp, pads=2 * nsp, output_padding=nsp, output_shape=nsp,
                kernel_shape=nsp)
    vals = dict(strides=strides, dilations=dilations, pads=pads, output_padding=output_padding,
                output_shape=output_shape, kernel_shape=kernel_shape)
    for k, v in vals.items():
        if v is not None and len(v) != lens[k]:
            raise ConvTransposeError(1, f"{k} must have {lens[k]} entries")
    if auto_pad not in AUTO_PAD:
        raise ConvTransposeError(1, f"unknown auto_pad {auto_pad!r}")
    return [AUTO_PAD[auto_pad]] + [_i64(vals[k]) for k in
                                   ("strides", "dilations", "pads", "output_padding", "output_shape",
                                    "kernel_shape")] + [int(group)]


def _raise(st: int):
    raise ConvTransposeError(st, convtranspose_last_error())


def convtranspose_output_shape(x_shape, w_shape, **attrs) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """Resolved Y shape (N, M, O1..On) and applied pads (begins, then ends)."""
    lib = load_library()
    nsp = len(x_shape) - 2
    if len(w_shape) != len(x_shape):
        raise ConvTransposeError(1, "W must have the same rank as X")
    ys = (ctypes.c_int64 * (nsp + 2))()
    pd = (ctypes.c_int64 * max(1, 2 * nsp))()
    st = lib.convtranspose_output_shape(nsp, _i64(x_shape), _i64(w_shape), *_attr_args(nsp, **attrs),
                                        ys, pd)
    if st:
        _raise(st)
    return tuple(ys), tuple(pd[: 2 * nsp])


def convtranspose_useful_macs(x_shape, w_shape, **attrs) -> int:
    """Useful MACs: in-range (input sample, tap) pairs times N * C/group * M."""
    lib = load_library()
    nsp = len(x_shape) - 2
    out = ctypes.c_double(0.0)
    st = lib.convtranspose_useful_macs(nsp, _i64(x_shape), _i64(w_shape), *_attr_args(nsp, **attrs),
                                       ctypes.byref(out))
    if st:
        _raise(st)
    return int(out.value)


def _expected_cl_strides(shape):
    """Strides of a dense channels-last tensor with logical shape (N, C, D1..Dn)."""
    N, C, sp = shape[0], shape[1], list(shape[2:])
    st = [0] * len(shape)
    st[1] = 1
    acc = C
    for a in range(len(sp) - 1, -1, -1):
        st[2 + a] = acc
        acc *= sp[a]
    st[0] = acc
    return st


def _dense(t: torch.Tensor, channels_last: bool) -> bool:
    if t.numel() == 0:
        return True  # nothing is read or written
    if not channels_last:
        return t.is_contiguous()
    want = _expected_cl_strides(t.shape)
    return all(sz <= 1 or s == w for sz, s, w in zip(t.shape, t.stride(), want))


def channels_last_empty(shape, dtype, device) -> torch.Tensor:
    """Uninitialised tensor of logical shape (N, C, D..) stored (N, D.., C)."""
    nsp = len(shape) - 2
    phys = torch.empty((shape[0],) + tuple(shape[2:]) + (shape[1],), dtype=dtype, device=device)
    return phys.permute(0, nsp + 1, *range(1, nsp + 1))


def to_channels_last(t: torch.Tensor) -> torch.Tensor:
    """Dense channels-last copy of a logical (N, C, D..) tensor."""
    nsp = t.dim() - 2
    return t.permute(0, *range(2, nsp + 2), 1).contiguous().permute(0, nsp + 1, *range(1, nsp + 1))


def _check_tensor(name, t, device, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ConvTransposeError(1, f"{name} must be on a HIP device (got {t.device})")
    if t.device != device:
        raise ConvTransposeError(1, f"{name} is on {t.device}, x is on {device}")
    if t.dtype != dtype:
        raise ConvTransposeError(3, f"{name} has dtype {t.dtype}, x has {dtype}")


def _call_args(x, w, bias, y, attrs):
    nsp = x.dim() - 2
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    return nsp, ptr(x), _i64(x.shape), ptr(w), _i64(w.shape), ptr(bias), ptr(y), _attr_args(nsp, **attrs)


def convtranspose_select_kernel(x, w, bias=None, *, channels_last=False, **attrs) -> str:
    """Name of the kernel family the dispatcher would run for these tensors."""
    lib = load_library()
    if x.dtype not in _DTYPES:
        raise ConvTransposeError(3, f"dtype {x.dtype} is not served")
    nsp, xp, xs, wp, ws, bp, _, at = _call_args(x, w, bias, None, attrs)
    yshape, _ = convtranspose_output_shape(tuple(x.shape), tuple(w.shape), **attrs)
    # alignment of y is that of a fresh torch allocation (256 B)
    k = lib.convtranspose_select_kernel(_DTYPES[x.dtype], nsp, int(channels_last), xp, xs, wp, ws, bp,
                                        ctypes.c_void_p(256), *at)
    if k < 0:
        raise ConvTransposeError(1, convtranspose_last_error())
    return convtranspose_kernel_name(k)


class ConvTransposePlan:
    """One ConvTranspose with its arguments resolved and marshalled once.

    Construction validates the tensors, resolves Y's shape, allocates Y (unless ``out``
    is given) and the implicit-GEMM scratch, and builds the C argument list; each call
    then enqueues the operation on ``stream`` (default: torch's current stream of x's
    device at construction) with a single C call.  Repeated calls reuse Y and the
    scratch, so they must be ordered on one stream.
    """

    def __init__(self, x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                 auto_pad: str = "NOTSET", strides=None, dilations=None, pads=None,
                 output_padding=None, output_shape=None, kernel_shape=None, group: int = 1,
                 channels_last: bool = False, out: Optional[torch.Tensor] = None,
                 kernel: str = "auto", stream: Optional[torch.cuda.Stream] = None,
                 activation: str = "identity", act_params: Sequence[float] = ()):
        lib = load_library()
        if activation not in ACTIVATIONS:
            raise ConvTransposeError(1, f"unknown activation {activation!r}")
        act_kind, act_n = ACTIVATIONS[activation]
        if len(act_params) != act_n:
            raise ConvTransposeError(1, f"{activation} takes {act_n} parameter(s)")
        act_p = [float(v) for v in act_params] + [0.0] * (2 - act_n)
        if x.dtype not in _DTYPES:
            raise ConvTransposeError(3, f"dtype {x.dtype} is not served (float32, float16)")
        if x.dim() < 3 or x.dim() > 5:
            raise ConvTransposeError(1, "x must have rank 3, 4 or 5")
        dev = x.device
        _check_tensor("x", x, dev, x.dtype)
        _check_tensor("w", w, dev, x.dtype)
        if w.dim() != x.dim():
            raise ConvTransposeError(1, "W must have the same rank as X")
        if bias is not None:
            _check_tensor("bias", bias, dev, x.dtype)
            if bias.dim() != 1 or not bias.is_contiguous():
                raise ConvTransposeError(1, "bias must be a dense 1-D tensor")
            if bias.shape[0] != w.shape[1] * int(group):
                raise ConvTransposeError(1, "bias length must equal M = W.shape[1] * group")
        if not _dense(x, channels_last):
            raise ConvTransposeError(1, "x is not dense in the requested layout")
        if not w.is_contiguous():
            raise ConvTransposeError(1, "w must be contiguous")
        if kernel not in KERNELS:
            raise ConvTransposeError(1, f"unknown kernel {kernel!r}")
        attrs = dict(auto_pad=auto_pad, strides=strides, dilations=dilations, pads=pads,
                     output_padding=output_padding, output_shape=output_shape,
                     kernel_shape=kernel_shape, group=group)
        yshape, _ = convtranspose_output_shape(tuple(x.shape), tuple(w.shape), **attrs)
        if out is None:
            out = (channels_last_empty(yshape, x.dtype, dev) if channels_last
                   else torch.empty(yshape, dtype=x.dtype, device=dev))
        else:
            _check_tensor("out", out, dev, x.dtype)
            if tuple(out.shape) != tuple(yshape):
                raise ConvTransposeError(2, f"out has shape {tuple(out.shape)}, expected {yshape}")
            if not _dense(out, channels_last):
                raise ConvTransposeError(1, "out is not dense in the requested layout")
        nsp, xp, xs, wp, ws, bp, yp, at = _call_args(x, w, bias, out, attrs)
        nbytes = ctypes.c_size_t(0)
        st = lib.convtranspose_workspace_size(KERNELS[kernel], _DTYPES[x.dtype], nsp, int(channels_last), xp,
                                              xs, ws, *at, ctypes.byref(nbytes))
        if st:
            _raise(st)
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        self.scratch = None
        if nbytes.value:
            with torch.cuda.stream(self.stream):
                self.scratch = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
        self.out = out
        self.device = dev
        self._keep = (x, w, bias)  # the pointers below stay valid while the plan lives
        self._fn = lib.convtranspose_nd_fused
        self._args = (KERNELS[kernel], _DTYPES[x.dtype], nsp, int(channels_last), xp, xs, wp, ws, bp, yp,
                      _i64(yshape), *at, act_kind, act_p[0], act_p[1],
                      ctypes.c_void_p(self.scratch.data_ptr()) if self.scratch is not None else None,
                      nbytes.value, ctypes.c_void_p(self.stream.cuda_stream))

    def __call__(self) -> torch.Tensor:
        with torch.cuda.device(self.device):
            st = self._fn(*self._args)
        if st:
            _raise(st)
        return self.out


def convtranspose_nd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                     auto_pad: str = "NOTSET", strides=None, dilations=None, pads=None,
                     output_padding=None, output_shape=None, kernel_shape=None, group: int = 1,
                     channels_last: bool = False, out: Optional[torch.Tensor] = None,
                     kernel: str = "auto", stream: Optional[torch.cuda.Stream] = None,
                     activation: str = "identity", act_params: Sequence[float] = ()) -> torch.Tensor:
    """Y = ConvTranspose(X, W, bias) on the GPU, enqueued on ``stream`` (default: torch's
    current stream of x's device).

    x: logical (N, C, D1..Dn) float32/float16 on a HIP device; dense NC.. storage, or
    dense N..C storage when ``channels_last`` (see ``to_channels_last``).
    w: (C, M/group, k1..kn) dense.  bias: (M,) or None.  Y is allocated (or ``out`` is
    used) with the same layout convention as x.  ``kernel`` forces a kernel family.
    ``activation`` ("identity", "relu", "leaky_relu" with ``act_params=(slope,)``, "clip"
    with ``act_params=(lower, upper)``) is applied to every output in float32, after the
    bias and before the one rounding, inside the kernel that computes it.
    """
    return ConvTransposePlan(x, w, bias, auto_pad=auto_pad, strides=strides, dilations=dilations,
                             pads=pads, output_padding=output_padding, output_shape=output_shape,
                             kernel_shape=kernel_shape, group=group, channels_last=channels_last,
                             out=out, kernel=kernel, stream=stream, activation=activation,
                             act_params=act_params)()


def convtranspose_nd_noalloc(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                             out: torch.Tensor, auto_pad: str = "NOTSET", strides=None, dilations=None, pads=None,
                             output_padding=None, output_shape=None, kernel_shape=None, group: int = 1,
                             channels_last: bool = False, kernel: str = "auto",
                             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """The C entry point ``convtranspose_nd_noalloc``: Y = ConvTranspose(X, W, bias) into the
    caller's ``out`` with the library's fixed device workspace, so nothing is allocated
    (neither here nor in the library).  Arguments as for ``convtranspose_nd``; ``out`` is
    required.  Calls on one device share the workspace: order them on one stream."""
    lib = load_library()
    if x.dtype not in _DTYPES:
        raise ConvTransposeError(3, f"dtype {x.dtype} is not served (float32, float16)")
    if kernel not in KERNELS:
        raise ConvTransposeError(1, f"unknown kernel {kernel!r}")
    dev = x.device
    for name, t in (("x", x), ("w", w), ("out", out)) + ((("bias", bias),) if bias is not None else ()):
        _check_tensor(name, t, dev, x.dtype)
    if not _dense(x, channels_last) or not _dense(out, channels_last) or not w.is_contiguous():
        raise ConvTransposeError(1, "x, out and w must be dense in the requested layout")
    attrs = dict(auto_pad=auto_pad, strides=strides, dilations=dilations, pads=pads,
                 output_padding=output_padding, output_shape=output_shape,
                 kernel_shape=kernel_shape, group=group)
    nsp, xp, xs, wp, ws, bp, yp, at = _call_args(x, w, bias, out, attrs)
    st_ = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = lib.convtranspose_nd_noalloc(KERNELS[kernel], _DTYPES[x.dtype], nsp, int(channels_last), xp, xs, wp, ws,
                                          bp, yp, _i64(tuple(out.shape)), *at, ctypes.c_void_p(st_.cuda_stream))
    if st:
        _raise(st)
    return out


IGEMM_TILES = ("256x256", "128x256", "64x512", "64x256", "64x128", "allphase", "tapsplit")


def set_igemm_tile(tile: Optional[str]) -> None:
    """Force one block shape of the float16 MFMA kernel (a name from IGEMM_TILES, output
    channels x output pixels), or None for the automatic choice.  Process-wide."""
    lib = load_library()
    st = lib.convtranspose_set_igemm_tile(-1 if tile is None else IGEMM_TILES.index(tile))
    if st:
        _raise(st)


def igemm_tile() -> Optional[str]:
    """The forced block shape of the float16 MFMA kernel, or None (automatic)."""
    t = load_library().convtranspose_igemm_tile()
    return None if t < 0 else IGEMM_TILES[t]


def convtranspose_profile_events(before: Optional[torch.cuda.Event], after: Optional[torch.cuda.Event]):
    """Have later calls on this thread record ``before``/``after`` around their dominant
    kernel (timing events created with ``enable_timing=True``); None, None turns it off."""
    lib = load_library()
    handles = []
    for ev in (before, after):
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:
            ev.record()  # torch creates the HIP event on first record
        handles.append(ctypes.c_void_p(ev.cuda_event))
    st = lib.convtranspose_profile_events(*handles)
    if st:
        _raise(st)


# ------------------------------------------------------------------------------------
# The forward convolution with the same W (the adjoint of the transposed convolution)
# ------------------------------------------------------------------------------------
def _conv_attr_args(nsp, auto_pad="NOTSET", strides=None, dilations=None, pads=None, kernel_shape=None, group=1):
    lens = dict(strides=nsp, dilations=nsp, pads=2 * nsp, kernel_shape=nsp)
    vals = dict(strides=strides, dilations=dilations, pads=pads, kernel_shape=kernel_shape)
    for k, v in vals.items():
        if v is not None and len(v) != lens[k]:
            raise ConvTransposeError(1, f"{k} must have {lens[k]} entries")
    if auto_pad not in AUTO_PAD:
        raise ConvTransposeError(1, f"unknown auto_pad {auto_pad!r}")
    return [AUTO_PAD[auto_pad], _i64(strides), _i64(dilations), _i64(pads), _i64(kernel_shape), int(group)]


def convolution_output_shape(x_shape, w_shape, **attrs) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    """Forward convolution: resolved Y shape (N, M, O1..On) and applied pads."""
    lib = load_library()
    nsp = len(x_shape) - 2
    if len(w_shape) != len(x_shape):
        raise ConvTransposeError(1, "W must have the same rank as X")
    ys = (ctypes.c_int64 * (nsp + 2))()
    pd = (ctypes.c_int64 * max(1, 2 * nsp))()
    st = lib.convolution_output_shape(nsp, _i64(x_shape), _i64(w_shape), *_conv_attr_args(nsp, **attrs), ys, pd)
    if st:
        _raise(st)
    return tuple(ys), tuple(pd[: 2 * nsp])


def convolution_nd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                   auto_pad: str = "NOTSET", strides=None, dilations=None, pads=None, kernel_shape=None,
                   group: int = 1, channels_last: bool = False, out: Optional[torch.Tensor] = None,
                   kernel: str = "auto", stream: Optional[torch.cuda.Stream] = None,
                   _prepare_only: bool = False) -> torch.Tensor:
    """Y = Conv(X, W, bias) on the GPU (ONNX Conv; W is (M, C/group, k1..kn)), the adjoint of
    ``convtranspose_nd`` with the same W.  ``kernel``: "auto", "direct" or "igemm" (the
    MFMA path: stride 1, or strided with dilation 1 through the input phases)."""
    lib = load_library()
    if x.dtype not in _DTYPES:
        raise ConvTransposeError(3, f"dtype {x.dtype} is not served (float32, float16)")
    if x.dim() < 3 or x.dim() > 5 or w.dim() != x.dim():
        raise ConvTransposeError(1, "x and w must have the same rank, 3 to 5")
    dev = x.device
    _check_tensor("x", x, dev, x.dtype)
    _check_tensor("w", w, dev, x.dtype)
    if bias is not None:
        _check_tensor("bias", bias, dev, x.dtype)
        if bias.dim() != 1 or not bias.is_contiguous() or bias.shape[0] != w.shape[0]:
            raise ConvTransposeError(1, "bias must be a dense 1-D tensor of length M = W.shape[0]")
    if not _dense(x, channels_last) or not w.is_contiguous():
        raise ConvTransposeError(1, "x (in the requested layout) and w must be dense")
    if kernel not in ("auto", "direct", "igemm"):
        raise ConvTransposeError(1, f"unknown kernel {kernel!r}")
    attrs = dict(auto_pad=auto_pad, strides=strides, dilations=dilations, pads=pads, kernel_shape=kernel_shape,
                 group=group)
    yshape, _ = convolution_output_shape(tuple(x.shape), tuple(w.shape), **attrs)
    if out is None:
        out = (channels_last_empty(yshape, x.dtype, dev) if channels_last
               else torch.empty(yshape, dtype=x.dtype, device=dev))
    else:
        _check_tensor("out", out, dev, x.dtype)
        if tuple(out.shape) != tuple(yshape) or not _dense(out, channels_last):
            raise ConvTransposeError(2, f"out must be dense with shape {yshape}")
    stream = stream if stream is not None else torch.cuda.current_stream(dev)
    nsp = x.dim() - 2
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    args = (KERNELS[kernel], _DTYPES[x.dtype], nsp, int(channels_last), ptr(x), _i64(x.shape), ptr(w), _i64(w.shape),
            ptr(bias), ptr(out), _i64(yshape), *_conv_attr_args(nsp, **attrs), ctypes.c_void_p(stream.cuda_stream))
    if _prepare_only:
        return lib.convolution_nd, args, out
    with torch.cuda.device(dev):
        st = lib.convolution_nd(*args)
    if st:
        _raise(st)
    return out


_QTYPES = {torch.int8: 2, torch.uint8: 3}


def qlinear_convtranspose_nd(x: torch.Tensor, x_scale: float, x_zero_point: int, w: torch.Tensor,
                             w_scale: torch.Tensor, w_zero_point: torch.Tensor, y_scale: float, y_zero_point: int,
                             y_dtype: torch.dtype = torch.uint8, bias: Optional[torch.Tensor] = None, *,
                             auto_pad: str = "NOTSET", strides=None, dilations=None, pads=None, output_padding=None,
                             output_shape=None, kernel_shape=None, group: int = 1, channels_last: bool = False,
                             out: Optional[torch.Tensor] = None, kernel: str = "auto",
                             stream: Optional[torch.cuda.Stream] = None, _prepare_only: bool = False) -> torch.Tensor:
    """Quantized ConvTranspose (QLinear scheme) on the GPU: uint8/int8 x, w and y; x and y
    quantized per tensor (host scalars), w per tensor or per output channel (w_scale
    float32 and w_zero_point of w's dtype, 1 or M values, on x's device); bias int32."""
    lib = load_library()
    for name, t in (("x", x), ("w", w), ("w_zero_point", w_zero_point)):
        if t.dtype not in _QTYPES:
            raise ConvTransposeError(3, f"{name} must be uint8 or int8 (got {t.dtype})")
    if y_dtype not in _QTYPES:
        raise ConvTransposeError(3, f"y_dtype must be uint8 or int8 (got {y_dtype})")
    if w_zero_point.dtype != w.dtype:
        raise ConvTransposeError(3, "w_zero_point must have w's dtype")
    if x.dim() < 3 or x.dim() > 5 or w.dim() != x.dim():
        raise ConvTransposeError(1, "x and w must have the same rank, 3 to 5")
    dev = x.device
    _check_tensor("x", x, dev, x.dtype)
    _check_tensor("w", w, dev, w.dtype)
    _check_tensor("w_scale", w_scale, dev, torch.float32)
    _check_tensor("w_zero_point", w_zero_point, dev, w.dtype)
    if w_scale.dim() != 1 or w_zero_point.dim() != 1 or w_scale.numel() != w_zero_point.numel() \
            or not w_scale.is_contiguous() or not w_zero_point.is_contiguous():
        raise ConvTransposeError(1, "w_scale and w_zero_point must be dense 1-D tensors of the same length")
    if bias is not None:
        _check_tensor("bias", bias, dev, torch.int32)
        if bias.dim() != 1 or not bias.is_contiguous():
            raise ConvTransposeError(1, "bias must be a dense 1-D int32 tensor")
    if not _dense(x, channels_last) or not w.is_contiguous():
        raise ConvTransposeError(1, "x (in the requested layout) and w must be dense")
    if kernel not in KERNELS:
        raise ConvTransposeError(1, f"unknown kernel {kernel!r}")
    attrs = dict(auto_pad=auto_pad, strides=strides, dilations=dilations, pads=pads, output_padding=output_padding,
                 output_shape=output_shape, kernel_shape=kernel_shape, group=group)
    yshape, _ = convtranspose_output_shape(tuple(x.shape), tuple(w.shape), **attrs)
    if out is None:
        out = (channels_last_empty(yshape, y_dtype, dev) if channels_last
               else torch.empty(yshape, dtype=y_dtype, device=dev))
    else:
        _check_tensor("out", out, dev, y_dtype)
        if tuple(out.shape) != tuple(yshape) or not _dense(out, channels_last):
            raise ConvTransposeError(2, f"out must be dense with shape {yshape}")
    stream = stream if stream is not None else torch.cuda.current_stream(dev)
    nsp = x.dim() - 2
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    args = (KERNELS[kernel], nsp, int(channels_last), ptr(x), _QTYPES[x.dtype], _i64(x.shape), float(x_scale),
            int(x_zero_point), ptr(w), _QTYPES[w.dtype], _i64(w.shape), ptr(w_scale), ptr(w_zero_point),
            w_scale.numel(), ptr(bias), ptr(out), _QTYPES[y_dtype], _i64(yshape), float(y_scale), int(y_zero_point),
            *_attr_args(nsp, **attrs), ctypes.c_void_p(stream.cuda_stream))
    if _prepare_only:
        return lib.qlinear_convtranspose_nd, args, out
    with torch.cuda.device(dev):
        st = lib.qlinear_convtranspose_nd(*args)
    if st:
        _raise(st)
    return out


class PreparedCall:
    """One call of ``convolution_nd`` or ``qlinear_convtranspose_nd`` with its arguments
    validated and marshalled once: ``PreparedCall(convolution_nd, x, w, ...)`` takes the
    function's own arguments; each call then enqueues the operation with a single C
    call, writing the same output tensor (``.out``).  Repeated calls must be ordered on
    one stream; the tensors must outlive the object."""

    def __init__(self, fn, *args, **kwargs):
        if fn not in (convolution_nd, qlinear_convtranspose_nd):
            raise TypeError("PreparedCall serves convolution_nd and qlinear_convtranspose_nd")
        self._fn, self._args, self.out = fn(*args, _prepare_only=True, **kwargs)
        self._keep = (args, kwargs)  # the pointers stay valid while the object lives
        self.device = self.out.device

    def __call__(self) -> torch.Tensor:
        with torch.cuda.device(self.device):
            st = self._fn(*self._args)
        if st:
            _raise(st)
        return self.out
