"""Python face of the fp64 ConvTranspose oracle (``ct_oracle.c``).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares nothing with
the HIP library and imports nothing from it.

The arithmetic lives in ``ct_oracle.c`` (the scatter definition of the transposed
convolution from the webgpu-kernels "ai.onnx.ConvTranspose" README, sections
Description, Inputs, Attributes and Outputs).  This file only builds that library,
widens inputs exactly to fp64 and passes pointers.  Inputs are in the logical
(N, C, D1..Dn) layout; callers holding channels-last data permute first.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ct_oracle.c")
_LIB = os.path.join(_HERE, "libctoracle.so")
AUTO_PAD = {"NOTSET": 0, "SAME_UPPER": 1, "SAME_LOWER": 2, "VALID": 3}
_lib = None


class OracleError(ValueError):
    """The oracle rejected the attributes or shapes."""


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    # CT_ORACLE_LIB: another build of ct_oracle.c (e.g. with sanitizers) as the default
    env = os.environ.get("CT_ORACLE_LIB") if path is None else None
    p = path or env or _LIB
    if path is None and not env and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(p)
    i64p = ctypes.POINTER(ctypes.c_int64)
    f64p = ctypes.POINTER(ctypes.c_double)
    attrs = [ctypes.c_int, i64p, i64p, i64p, i64p, i64p, i64p, ctypes.c_int64]
    lib.oracle_output_shape.argtypes = [ctypes.c_int, i64p, i64p] + attrs + [
        i64p, i64p, ctypes.c_char_p, ctypes.c_int]
    lib.oracle_useful_macs.argtypes = [ctypes.c_int, i64p, i64p] + attrs + [
        f64p, ctypes.c_char_p, ctypes.c_int]
    lib.oracle_convtranspose_f64.argtypes = [ctypes.c_int, i64p, f64p, i64p, f64p, f64p] + attrs + [
        f64p, ctypes.c_int64, ctypes.c_char_p, ctypes.c_int]
    lib.oracle_convtranspose_at.argtypes = [ctypes.c_int, i64p, f64p, i64p, f64p, f64p] + attrs + [
        i64p, ctypes.c_int64, f64p, ctypes.c_char_p, ctypes.c_int]
    cattrs = [ctypes.c_int, i64p, i64p, i64p, i64p, ctypes.c_int64]  # forward convolution
    lib.oracle_conv_output_shape.argtypes = [ctypes.c_int, i64p, i64p] + cattrs + [
        i64p, i64p, ctypes.c_char_p, ctypes.c_int]
    lib.oracle_conv_f64.argtypes = [ctypes.c_int, i64p, f64p, i64p, f64p, f64p] + cattrs + [
        f64p, ctypes.c_int64, ctypes.c_char_p, ctypes.c_int]
    i32p = ctypes.POINTER(ctypes.c_int32)
    f32p = ctypes.POINTER(ctypes.c_float)
    c_i32, c_f32 = ctypes.c_int32, ctypes.c_float
    lib.oracle_qconvtranspose.argtypes = [ctypes.c_int, i64p, i32p, c_i32, c_f32, i64p, i32p, i32p, f32p,
                                          ctypes.c_int64, i32p, c_f32, c_i32, c_i32, c_i32] + attrs + [
        i64p, i32p, ctypes.c_int64, ctypes.c_char_p, ctypes.c_int]
    lib.oracle_requantize.argtypes = [i64p, ctypes.c_int64, c_f32, f32p, i64p, c_f32, c_i32, c_i32, c_i32, i32p]
    for fn in ("oracle_output_shape", "oracle_useful_macs", "oracle_convtranspose_f64",
               "oracle_convtranspose_at", "oracle_threads", "oracle_conv_output_shape", "oracle_conv_f64",
               "oracle_qconvtranspose", "oracle_requantize"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    if path is None:
        _lib = lib
    return lib


def threads(lib=None) -> int:
    """OpenMP threads the oracle's loops run on."""
    return int((lib or load()).oracle_threads())


def _i64(v: Optional[Sequence[int]]):
    if v is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(v, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _f64(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(a).astype(np.float64))  # exact widening of f16/f32
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _attr_args(auto_pad="NOTSET", strides=None, dilations=None, pads=None, output_padding=None,
               output_shape=None, kernel_shape=None, group=1):
    keep = []
    out = [AUTO_PAD[auto_pad]]
    for v in (strides, dilations, pads, output_padding, output_shape, kernel_shape):
        arr, ptr = _i64(v)
        keep.append(arr)
        out.append(ptr)
    out.append(int(group))
    return out, keep


def _check(rc: int, err) -> None:
    if rc != 0:
        raise OracleError(err.value.decode(errors="replace"))


def output_shape(x_shape, w_shape, lib=None, **attrs):
    """Resolved Y shape (N, M, O1..On) and the applied pads [b1..bn, e1..en]."""
    lib = lib or load()
    nsp = len(x_shape) - 2
    if len(w_shape) != len(x_shape):
        raise OracleError("W must have the same rank as X")
    xs, xp = _i64(x_shape)
    ws, wp = _i64(w_shape)
    args, keep = _attr_args(**attrs)
    ys = np.zeros(nsp + 2, dtype=np.int64)
    pd = np.zeros(2 * nsp, dtype=np.int64)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_output_shape(nsp, xp, wp, *args,
                                 ys.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 pd.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), err, 256)
    _check(rc, err)
    return tuple(int(v) for v in ys), [int(v) for v in pd]


def useful_macs(x_shape, w_shape, lib=None, **attrs) -> int:
    """(input sample, tap) pairs landing inside Y, times N * C/group * M."""
    lib = lib or load()
    nsp = len(x_shape) - 2
    xs, xp = _i64(x_shape)
    ws, wp = _i64(w_shape)
    args, keep = _attr_args(**attrs)
    out = ctypes.c_double(0)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_useful_macs(nsp, xp, wp, *args, ctypes.byref(out), err, 256)
    _check(rc, err)
    return int(out.value)


def convtranspose(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray] = None, lib=None,
                  **attrs) -> np.ndarray:
    """Whole Y in fp64 by the scatter definition (logical NC.. layout)."""
    lib = lib or load()
    x64, xp = _f64(x)
    w64, wp = _f64(w)
    b64, bp = _f64(bias)
    yshape, _ = output_shape(x64.shape, w64.shape, lib=lib, **attrs)
    if b64 is not None and b64.shape != (yshape[1],):
        raise OracleError("bias must be 1-D of length M")
    y = np.zeros(yshape, dtype=np.float64)
    args, keep = _attr_args(**attrs)
    xs, xsp = _i64(x64.shape)
    ws, wsp = _i64(w64.shape)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_convtranspose_f64(x64.ndim - 2, xsp, xp, wsp, wp, bp, *args,
                                      y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                      y.size, err, 256)
    _check(rc, err)
    return y


def convtranspose_at(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray], points: np.ndarray,
                     lib=None, **attrs) -> np.ndarray:
    """Y at the given output positions (rows of (n, m, o1..on)), fp64."""
    lib = lib or load()
    x64, xp = _f64(x)
    w64, wp = _f64(w)
    b64, bp = _f64(bias)
    pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64))
    out = np.zeros(len(pts), dtype=np.float64)
    args, keep = _attr_args(**attrs)
    xs, xsp = _i64(x64.shape)
    ws, wsp = _i64(w64.shape)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_convtranspose_at(x64.ndim - 2, xsp, xp, wsp, wp, bp, *args,
                                     pts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     len(pts), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                     err, 256)
    _check(rc, err)
    return out


ACTIVATIONS = ("identity", "relu", "leaky_relu", "clip")


def activation(y: np.ndarray, kind: str = "identity", params: Sequence[float] = ()) -> np.ndarray:
    """The output activation applied elementwise, in fp64, to Y (bias included).

    ClikaRT "conv_transpose" API page: the call takes an ``activation`` argument whose
    default is Identity; the page does not list the other members, so each one here is
    the elementwise function of its usual definition:
      relu        v if v > 0, else 0
      leaky_relu  v if v >= 0, else slope * v            (params = (slope,))
      clip        lower if v < lower, upper if v > upper, else v   (params = (lower, upper))
    """
    y = np.asarray(y, dtype=np.float64)
    p = [float(v) for v in params]
    if kind == "identity" and not p:
        return y.copy()
    if kind == "relu" and not p:
        return np.where(y > 0.0, y, 0.0)
    if kind == "leaky_relu" and len(p) == 1 and np.isfinite(p[0]):
        return np.where(y >= 0.0, y, p[0] * y)
    if kind == "clip" and len(p) == 2 and np.all(np.isfinite(p)) and p[0] <= p[1]:
        return np.where(y < p[0], p[0], np.where(y > p[1], p[1], y))
    raise OracleError(f"activation {kind!r} with parameters {params!r} is not defined")


# ------------------------------------------------------------------------------------
# Forward convolution (ONNX Conv with the same W layout (M, C/group, k..)): the adjoint
# of the transposed convolution.  Arithmetic in ct_oracle.c (oracle_conv_f64).
# ------------------------------------------------------------------------------------
def _conv_attr_args(auto_pad="NOTSET", strides=None, dilations=None, pads=None, kernel_shape=None, group=1):
    keep = []
    out = [AUTO_PAD[auto_pad]]
    for v in (strides, dilations, pads, kernel_shape):
        arr, ptr = _i64(v)
        keep.append(arr)
        out.append(ptr)
    out.append(int(group))
    return out, keep


def conv_output_shape(x_shape, w_shape, lib=None, **attrs):
    """Resolved forward-convolution output shape (N, M, O1..On) and the applied pads."""
    lib = lib or load()
    nsp = len(x_shape) - 2
    if len(w_shape) != len(x_shape):
        raise OracleError("W must have the same rank as X")
    xs, xp = _i64(x_shape)
    ws, wp = _i64(w_shape)
    args, keep = _conv_attr_args(**attrs)
    ys = np.zeros(nsp + 2, dtype=np.int64)
    pd = np.zeros(2 * nsp, dtype=np.int64)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_conv_output_shape(nsp, xp, wp, *args,
                                      ys.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      pd.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), err, 256)
    _check(rc, err)
    return tuple(int(v) for v in ys), [int(v) for v in pd]


def conv(x: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray] = None, lib=None, **attrs) -> np.ndarray:
    """Whole forward-convolution output in fp64 by the gather definition (NC.. layout)."""
    lib = lib or load()
    x64, xp = _f64(x)
    w64, wp = _f64(w)
    b64, bp = _f64(bias)
    yshape, _ = conv_output_shape(x64.shape, w64.shape, lib=lib, **attrs)
    if b64 is not None and b64.shape != (yshape[1],):
        raise OracleError("bias must be 1-D of length M")
    y = np.zeros(yshape, dtype=np.float64)
    args, keep = _conv_attr_args(**attrs)
    xs, xsp = _i64(x64.shape)
    ws, wsp = _i64(w64.shape)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_conv_f64(x64.ndim - 2, xsp, xp, wsp, wp, bp, *args,
                             y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), y.size, err, 256)
    _check(rc, err)
    return y


# --------------------------------------------------------------------------------------
# quantized transposed convolution (QLinear scale / zero-point scheme)
# --------------------------------------------------------------------------------------
QRANGE = {"uint8": (0, 255), "int8": (-128, 127)}


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a).astype(np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _f32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32).reshape(-1))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def qconvtranspose(x: np.ndarray, w: np.ndarray, x_scale: float, x_zero_point: int, w_scale, w_zero_point,
                   y_scale: float, y_zero_point: int, y_type: str = "uint8", bias: Optional[np.ndarray] = None,
                   return_acc: bool = False, lib=None, **attrs):
    """Quantized transposed convolution (NC.. layout): the exact integer scatter sum of
    zero-point-shifted operands plus the int32 bias, requantized in float32 to y_type.
    w_scale / w_zero_point: one value or one per output channel M.  Returns y (int32
    array of y_type values), and the exact accumulators too with ``return_acc``."""
    lib = lib or load()
    x32, xp = _i32(x)
    w32, wp = _i32(w)
    ws32, wsp = _f32(w_scale)
    wz32, wzp = _i32(np.asarray(w_zero_point).reshape(-1))
    if ws32.size != wz32.size:
        raise OracleError("w_scale and w_zero_point must have the same length")
    b32, bp = _i32(bias) if bias is not None else (None, None)
    yshape, _ = output_shape(x32.shape, w32.shape, lib=lib, **attrs)
    if b32 is not None and b32.shape != (yshape[1],):
        raise OracleError("bias must be 1-D of length M")
    lo, hi = QRANGE[y_type]
    y = np.zeros(yshape, dtype=np.int32)
    acc = np.zeros(yshape, dtype=np.int64) if return_acc else None
    args, keep = _attr_args(**attrs)
    xs, xsp = _i64(x32.shape)
    wsh, wshp = _i64(w32.shape)
    err = ctypes.create_string_buffer(256)
    rc = lib.oracle_qconvtranspose(x32.ndim - 2, xsp, xp, int(x_zero_point), float(x_scale), wshp, wp, wzp, wsp,
                                   ws32.size, bp, float(y_scale), int(y_zero_point), lo, hi, *args,
                                   acc.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if acc is not None else None,
                                   y.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), y.size, err, 256)
    _check(rc, err)
    return (y, acc) if return_acc else y


def requantize(acc, x_scale: float, w_scale, channel, y_scale: float, y_zero_point: int, y_type: str = "uint8",
               lib=None) -> np.ndarray:
    """The requantization step alone: acc (int64 values) of output channels ``channel``."""
    lib = lib or load()
    a = np.ascontiguousarray(np.asarray(acc, dtype=np.int64).reshape(-1))
    ch = np.ascontiguousarray(np.broadcast_to(np.asarray(channel, dtype=np.int64), a.shape))
    ws32, wsp = _f32(w_scale)
    lo, hi = QRANGE[y_type]
    y = np.zeros(a.shape, dtype=np.int32)
    lib.oracle_requantize(a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), a.size, float(x_scale), wsp,
                          ch.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), float(y_scale), int(y_zero_point),
                          lo, hi, y.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return y.reshape(np.shape(acc))
