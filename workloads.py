"""Seeded synthetic workloads for the N-D transposed convolution (ONNX ConvTranspose).

This module only *draws numbers*: it names the benchmark shapes, their attribute
sets and value distributions, and produces the input tensors from a seed.  It holds
none of the operator's arithmetic (no output-size rule, no padding rule, no sum), so
both the fp64 oracle side and the HIP side can take their inputs from here without
sharing any of the method.

Distributions: ``N(mu, sigma)`` means mean ``mu`` and standard deviation ``sigma``
(numpy ``rng.normal(loc, scale)``); ``U(a, b)`` is ``rng.uniform(a, b)``.  Every
tensor is drawn in fp64 from ``numpy.random.default_rng(seed)`` in the order X, W,
bias, then rounded once (round-to-nearest-even, numpy ``astype``) to the config's
element type.  Integer-valued variants draw X and W uniformly from {-2..2} and bias
from {-4..4} with ``seed + 100``; every partial sum of such inputs is an integer far
below 2**24, so fp32 accumulation of them is exact.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

DTYPES = {"f32": np.float32, "f16": np.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One ConvTranspose problem: shapes, ONNX attributes and value recipe."""

    name: str
    dtype: str                      # "f32" or "f16" (element type T of X, W, bias, Y)
    x_shape: Tuple[int, ...]        # logical (N, C, D1..Dn)
    w_shape: Tuple[int, ...]        # (C, M/group, k1..kn), ONNX layout
    has_bias: bool
    attrs: dict                     # ONNX attributes (strides, pads, ...); absent => default
    x_dist: Tuple[str, float, float]
    w_dist: Tuple[str, float, float]
    b_dist: Tuple[str, float, float]
    seed: int
    channels_last: bool = False
    note: str = ""

    @property
    def nsp(self) -> int:
        return len(self.x_shape) - 2

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _draw(rng: np.random.Generator, dist: Tuple[str, float, float], shape) -> np.ndarray:
    kind, a, b = dist
    if kind == "N":
        return rng.normal(a, b, size=shape)
    if kind == "U":
        return rng.uniform(a, b, size=shape)
    if kind == "I":  # integers, inclusive range [a, b]
        return rng.integers(int(a), int(b) + 1, size=shape).astype(np.float64)
    raise ValueError(f"unknown distribution {kind!r}")


def make_inputs(wl: Workload, integer: bool = False, seed: Optional[int] = None):
    """Return (x, w, bias) as numpy arrays of the workload's dtype, logical NC.. layout.

    ``integer=True`` gives the small-integer variant (X, W in {-2..2}, bias in {-4..4},
    seed + 100) used for bit-exact checks.  bias is None when the workload has none.
    """
    dt = DTYPES[wl.dtype]
    s = wl.seed if seed is None else seed
    if integer:
        rng = np.random.default_rng(s + 100)
        xd, wd, bd = ("I", -2, 2), ("I", -2, 2), ("I", -4, 4)
    else:
        rng = np.random.default_rng(s)
        xd, wd, bd = wl.x_dist, wl.w_dist, wl.b_dist
    x = _draw(rng, xd, wl.x_shape).astype(dt)
    w = _draw(rng, wd, wl.w_shape).astype(dt)
    m = wl.w_shape[1] * int(wl.attrs.get("group", 1))
    b = _draw(rng, bd, (m,)).astype(dt) if wl.has_bias else None
    return x, w, b


def make_points(y_shape: Sequence[int], count: int, seed: int) -> np.ndarray:
    """``count`` seeded output multi-indices (int64, shape [count, rank]) inside y_shape.

    The first rows are the corners of the output box (every coordinate at 0 or at its
    maximum), so borders and the ragged ends are always sampled.
    """
    rank = len(y_shape)
    corners = []
    for bits in range(1 << rank):
        corners.append([(y_shape[a] - 1) if (bits >> a) & 1 else 0 for a in range(rank)])
    rng = np.random.default_rng(seed)
    rnd = np.stack([rng.integers(0, y_shape[a], size=count) for a in range(rank)], axis=1)
    pts = np.concatenate([np.array(corners, dtype=np.int64), rnd.astype(np.int64)], axis=0)
    return pts[:max(count, len(corners))]


# The five benchmark configurations of the dense/grouped/1-D/3-D ConvTranspose study.
# Where the recipe gives no bias distribution, bias is N(0, 1) like X.
C1 = Workload(
    "c1_2d_f32_s2_op1", "f32", (1, 4, 8, 8), (4, 4, 3, 3), True,
    dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1], dilations=[1, 1], group=1),
    ("U", -1.0, 1.0), ("U", -1.0, 1.0), ("U", -1.0, 1.0), seed=1)
C2 = Workload(
    "c2_1d_f32_s3_d2", "f32", (4, 64, 256), (64, 32, 5), True,
    dict(strides=[3], dilations=[2], pads=[2, 2], output_padding=[1], group=1),
    ("N", 0.0, 1.0), ("N", 0.0, 1.0 / math.sqrt(64 * 5)), ("N", 0.0, 1.0), seed=2)
C3 = Workload(
    "c3_2d_f16_depthwise_s2", "f16", (16, 256, 56, 56), (256, 1, 4, 4), False,
    dict(strides=[2, 2], pads=[1, 1, 1, 1], group=256),
    ("N", 0.0, 1.0), ("N", 0.0, 0.25), ("N", 0.0, 1.0), seed=3)
C4 = Workload(
    "c4_2d_f16_decoder_s2", "f16", (8, 512, 64, 64), (512, 256, 4, 4), True,
    dict(strides=[2, 2], pads=[1, 1, 1, 1], group=1),
    ("N", 0.0, 1.0), ("N", 0.0, 1.0 / math.sqrt(512 * 16)), ("N", 0.0, 1.0), seed=4)
C3_NHWC = C3.with_(name="c3_2d_f16_depthwise_s2_nhwc", channels_last=True)
C4_NHWC = C4.with_(name="c4_2d_f16_decoder_s2_nhwc", channels_last=True)
C5_S1 = Workload(
    "c5_3d_f16_s1", "f16", (2, 128, 16, 32, 32), (128, 64, 3, 3, 3), True,
    dict(strides=[1, 1, 1], group=1),
    ("N", 0.0, 1.0), ("N", 0.0, 1.0 / math.sqrt(128 * 27)), ("N", 0.0, 1.0), seed=5,
    note="stride 1 takes default pads 0: output_padding 1 is not allowed at stride 1")
C5_S1_P1 = C5_S1.with_(name="c5_3d_f16_s1_p1", attrs=dict(strides=[1, 1, 1], pads=[1] * 6, group=1))
C5_S2 = C5_S1.with_(
    name="c5_3d_f16_s2_op1",
    attrs=dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1], group=1), note="")

CONFIGS = {w.name: w for w in (C1, C2, C3, C3_NHWC, C4, C4_NHWC, C5_S1, C5_S1_P1, C5_S2)}

# Extra shapes (not benchmark configurations): the decoder tensors of C4 with kernels no
# longer than the stride, where every output receives at most one tap per axis.
F2_K2S2 = C4.with_(name="f2_2d_f16_k2_s2", w_shape=(512, 256, 2, 2),
                   attrs=dict(strides=[2, 2], pads=[0, 0, 0, 0], group=1),
                   w_dist=("N", 0.0, 1.0 / math.sqrt(512 * 4)), seed=6)
F2_1X1 = C4.with_(name="f2_2d_f16_1x1", w_shape=(512, 256, 1, 1), attrs=dict(strides=[1, 1], group=1),
                  w_dist=("N", 0.0, 1.0 / math.sqrt(512)), seed=7)
# A 3-D depthwise call on C5's input tensors (the grouped family's rank-3 path).
G3_DW = C5_S2.with_(name="g3_3d_f16_depthwise_s2", w_shape=(128, 1, 3, 3, 3), has_bias=False,
                    attrs=dict(strides=[2, 2, 2], pads=[1] * 6, output_padding=[1, 1, 1], group=128),
                    w_dist=("N", 0.0, 0.25), seed=8)
# C3's shapes as a grouped call with 2 channels per group, channels-first and channels-last
G2_NCHW = C3.with_(name="g2_2d_f16_grouped2_s2", w_shape=(256, 2, 4, 4), attrs=dict(C3.attrs, group=128), seed=9)
G2_NHWC = G2_NCHW.with_(name="g2_2d_f16_grouped2_s2_nhwc", channels_last=True)
EXTRAS = {w.name: w for w in (F2_K2S2, F2_1X1, G3_DW, G2_NCHW, G2_NHWC)}


# --------------------------------------------------------------------------------------
# quantized problems (QLinear scale / zero-point scheme)
# --------------------------------------------------------------------------------------
QRANGE = {"uint8": (0, 255), "int8": (-128, 127)}


@dataclasses.dataclass(frozen=True)
class QWorkload:
    """A quantized ConvTranspose: shapes, attributes, element types and the recipe of the
    quantization parameters.  x and w are drawn uniformly over their types' whole range;
    the weight zero point is 0 for int8 weights and 128 for uint8 ones (symmetric
    weights), one per output channel when ``per_channel``; w_scale is U(0.8, 1.2) times
    ``w_scale`` per channel; bias is uniform in [-bias_max, bias_max]."""

    name: str
    x_shape: Tuple[int, ...]
    w_shape: Tuple[int, ...]
    attrs: dict
    x_type: str
    w_type: str
    y_type: str
    x_scale: float
    x_zero_point: int
    w_scale: float
    y_scale: float
    y_zero_point: int
    per_channel: bool
    bias_max: int
    seed: int
    channels_last: bool = False

    @property
    def nsp(self) -> int:
        return len(self.x_shape) - 2

    def with_(self, **kw) -> "QWorkload":
        return dataclasses.replace(self, **kw)


def make_qinputs(qw: QWorkload) -> dict:
    """Keyword arguments of a quantized call (numpy arrays; NC.. layout), drawn from
    ``default_rng(seed)`` in the order x, w, w_scale, bias."""
    rng = np.random.default_rng(qw.seed)
    npt = {"uint8": np.uint8, "int8": np.int8}
    lo, hi = QRANGE[qw.x_type]
    x = rng.integers(lo, hi + 1, size=qw.x_shape).astype(npt[qw.x_type])
    lo, hi = QRANGE[qw.w_type]
    w = rng.integers(lo, hi + 1, size=qw.w_shape).astype(npt[qw.w_type])
    M = qw.w_shape[1] * int(qw.attrs.get("group", 1))
    nq = M if qw.per_channel else 1
    w_scale = (qw.w_scale * rng.uniform(0.8, 1.2, size=nq)).astype(np.float32)
    w_zp = np.full(nq, 0 if qw.w_type == "int8" else 128).astype(npt[qw.w_type])
    bias = rng.integers(-qw.bias_max, qw.bias_max + 1, size=M).astype(np.int32) if qw.bias_max > 0 else None
    return dict(x=x, w=w, x_scale=np.float32(qw.x_scale), x_zero_point=qw.x_zero_point, w_scale=w_scale,
                w_zero_point=w_zp, y_scale=np.float32(qw.y_scale), y_zero_point=qw.y_zero_point, y_type=qw.y_type,
                bias=bias)


# The C4 decoder shapes quantized: uint8 activations (zero point 128), int8 weights with
# per-channel scales, uint8 output, channels-last; the scales put the output's spread at
# about 50 codes.
F4_C4 = QWorkload("f4_2d_int8_decoder_s2_nhwc", (8, 512, 64, 64), (512, 256, 4, 4),
                  dict(strides=[2, 2], pads=[1, 1, 1, 1], group=1), "uint8", "int8", "uint8",
                  x_scale=0.02, x_zero_point=128, w_scale=0.001, y_scale=0.1, y_zero_point=128,
                  per_channel=True, bias_max=50000, seed=8, channels_last=True)
QCONFIGS = {F4_C4.name: F4_C4}
