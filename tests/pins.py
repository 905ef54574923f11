"""Independent checks ("pins") of the fp64 ConvTranspose oracle.

Each ``pin_*`` function takes an oracle library handle (``oracle.load(path)``) and
raises AssertionError when the oracle disagrees with something fixed outside it:
hand-derived worked examples, a library routine (PyTorch's CPU conv_transpose /
conv in float64, numpy's convolve), a brute-force gather written as a different
loop nest, the zero-insertion ("fractionally strided") construction, the adjoint
identity with the forward convolution that uses the same W, the stride-1
flipped-kernel identity, and invariants (group split, linearity, translation).
The same functions run against deliberately broken copies of the oracle in
``test_oracle_mutants.py`` to show that each plausible mistake is caught.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")

_CT = {1: F.conv_transpose1d, 2: F.conv_transpose2d, 3: F.conv_transpose3d}
_CV = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}


# ----------------------------------------------------------------------------------
# random tiny problems
# ----------------------------------------------------------------------------------
def random_case(rng: np.random.Generator, nsp=None, auto=False, max_L=5):
    """A random small problem with explicit (NOTSET) pads, or an auto_pad mode."""
    while True:
        n = int(nsp or rng.integers(1, 4))
        group = int(rng.choice([1, 1, 2, 3]))
        Cg, Mg = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 3))
        Ls = [int(rng.integers(1, max_L + 1)) for _ in range(n)]
        Ks = [int(rng.integers(1, 5)) for _ in range(n)]
        s = [int(rng.integers(1, 4)) for _ in range(n)]
        d = [int(rng.integers(1, 4)) for _ in range(n)]
        op = [int(rng.integers(0, max(si, di))) for si, di in zip(s, d)]
        attrs = dict(strides=s, dilations=d, output_padding=op, group=group)
        if auto:
            attrs["auto_pad"] = str(rng.choice(["SAME_UPPER", "SAME_LOWER", "VALID"]))
        else:
            attrs["pads"] = [int(rng.integers(0, 3)) for _ in range(2 * n)]
        x = rng.normal(size=(N, Cg * group, *Ls))
        w = rng.normal(size=(Cg * group, Mg, *Ks))
        b = rng.normal(size=(Mg * group,)) if rng.random() < 0.7 else None
        try:
            O.output_shape(x.shape, w.shape, **attrs)
        except O.OracleError:
            continue  # e.g. a negative output size; draw again
        return x, w, b, attrs


def _crop_full(y_full: np.ndarray, nsp: int, b, O_sizes) -> np.ndarray:
    """Y[o] = y_full[o + b] where that index exists, else 0 (per spatial axis)."""
    out = np.zeros(y_full.shape[:2] + tuple(O_sizes), dtype=y_full.dtype)
    src, dst = [slice(None), slice(None)], [slice(None), slice(None)]
    for a in range(nsp):
        Fa = y_full.shape[2 + a]
        lo = max(0, -b[a])
        hi = min(O_sizes[a], Fa - b[a])
        if hi <= lo:
            return out
        dst.append(slice(lo, hi))
        src.append(slice(lo + b[a], hi + b[a]))
    out[tuple(dst)] = y_full[tuple(src)]
    return out


def torch_reference(x, w, bias, attrs, lib):
    """PyTorch CPU float64 conv_transpose with no padding (the whole footprint), then the
    resolved pads applied as a crop / zero extension, then bias."""
    nsp = x.ndim - 2
    yshape, pads = O.output_shape(x.shape, w.shape, lib=lib, **attrs)
    s = attrs.get("strides") or [1] * nsp
    d = attrs.get("dilations") or [1] * nsp
    full = _CT[nsp](torch.from_numpy(x), torch.from_numpy(w), stride=tuple(s), padding=0,
                    output_padding=0, groups=int(attrs.get("group", 1)), dilation=tuple(d)).numpy()
    y = _crop_full(full, nsp, pads[:nsp], yshape[2:])
    if bias is not None:
        y = y + bias.reshape((1, -1) + (1,) * nsp)
    return y


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, f"shape {a.shape} != {b.shape}"
    if a.size:
        err = np.max(np.abs(a - b) / (1.0 + np.abs(b)))
        assert err <= tol, f"max rel err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------------
def pin_golden(lib):
    """Hand-derived worked examples (tests/golden/worked_examples.json), exact."""
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float64)
        w = np.array(c["w"], dtype=np.float64)
        b = None if c["bias"] is None else np.array(c["bias"], dtype=np.float64)
        y = O.convtranspose(x, w, b, lib=lib, **c["attrs"])
        want = np.array(c["y"], dtype=np.float64)
        assert y.shape == want.shape, (c["name"], y.shape, want.shape)
        assert np.array_equal(y, want), (c["name"], y.tolist())


def pin_benchmark_shapes(lib):
    """Output shapes stated with the benchmark problems, and SAME => O = L * stride
    (README, Attributes: auto_pad)."""
    stated = [
        ((1, 4, 8, 8), (4, 4, 3, 3), dict(strides=[2, 2], pads=[1, 1, 1, 1], output_padding=[1, 1]),
         (1, 4, 16, 16)),
        ((16, 256, 56, 56), (256, 1, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1], group=256),
         (16, 256, 112, 112)),
        ((8, 512, 64, 64), (512, 256, 4, 4), dict(strides=[2, 2], pads=[1, 1, 1, 1]),
         (8, 256, 128, 128)),
    ]
    for xs, ws, at, want in stated:
        got, _ = O.output_shape(xs, ws, lib=lib, **at)
        assert got == want, (xs, got, want)
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 4))
        L = [int(v) for v in rng.integers(0, 7, size=n)]
        K = [int(v) for v in rng.integers(1, 6, size=n)]
        s = [int(v) for v in rng.integers(1, 4, size=n)]
        d = [int(v) for v in rng.integers(1, 4, size=n)]
        mode = str(rng.choice(["SAME_UPPER", "SAME_LOWER"]))
        got, pads = O.output_shape((1, 2) + tuple(L), (2, 3) + tuple(K), lib=lib, strides=s,
                                   dilations=d, auto_pad=mode)
        assert list(got[2:]) == [Li * si for Li, si in zip(L, s)], (L, s, got)
        for a in range(n):
            b, e = pads[a], pads[a + n]
            tot = s[a] * (L[a] - 1) + d[a] * (K[a] - 1) + 1 - L[a] * s[a]
            assert b + e == tot
            # the odd part of the total goes to the end (UPPER) / the beginning (LOWER)
            big, small = (e, b) if mode == "SAME_UPPER" else (b, e)
            assert big - small in ((0, 1) if tot >= 0 else (0, -1)), (mode, tot, b, e)


def pin_torch_library(lib, count=160, seed=11):
    """Random 1-D/2-D/3-D problems (strides, dilations, pads, output_padding, groups,
    bias, auto_pad) against PyTorch's float64 CPU conv_transpose."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        x, w, b, attrs = random_case(rng, auto=(t % 4 == 3))
        got = O.convtranspose(x, w, b, lib=lib, **attrs)
        _close(got, torch_reference(x, w, b, attrs, lib))


def pin_brute_force_gather(lib, count=40, seed=12):
    """A different loop nest: for every output element search every (c, i, k) whose
    scatter target it is.  Pads here are explicit, so O comes from the footprint."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        x, w, b, attrs = random_case(rng, max_L=3)
        nsp = x.ndim - 2
        s, d, pads, op = attrs["strides"], attrs["dilations"], attrs["pads"], attrs["output_padding"]
        G = attrs["group"]
        N, C = x.shape[:2]
        Mg = w.shape[1]
        Ks = w.shape[2:]
        Osz = [s[a] * (x.shape[2 + a] - 1) + op[a] + d[a] * (Ks[a] - 1) + 1 - pads[a] - pads[a + nsp]
               for a in range(nsp)]
        if min(Osz) < 0:
            continue
        y = np.zeros((N, Mg * G, *Osz))
        for n_, m in itertools.product(range(N), range(Mg * G)):
            g, mm = divmod(m, Mg)
            Cg = C // G
            for o in itertools.product(*[range(v) for v in Osz]):
                acc = b[m] if b is not None else 0.0
                for c in range(g * Cg, (g + 1) * Cg):
                    for i in itertools.product(*[range(v) for v in x.shape[2:]]):
                        for k in itertools.product(*[range(v) for v in Ks]):
                            if all(o[a] == i[a] * s[a] - pads[a] + k[a] * d[a] for a in range(nsp)):
                                acc += x[(n_, c) + i] * w[(c, mm) + k]
                y[(n_, m) + o] = acc
        _close(O.convtranspose(x, w, b, lib=lib, **attrs), y)


def pin_zero_insertion(lib, count=60, seed=13):
    """The 'fractionally strided' construction: insert s-1 zeros between input samples,
    pad d(K-1)-b before and d(K-1)-e+op after (negative = crop), then a stride-1
    correlation at dilation d with the tap-reversed, channel-swapped filter."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        x, w, b, attrs = random_case(rng)
        nsp = x.ndim - 2
        s, d, pads, op = attrs["strides"], attrs["dilations"], attrs["pads"], attrs["output_padding"]
        G = attrs["group"]
        N, C = x.shape[:2]
        Cg, Mg = C // G, w.shape[1]
        Ks = w.shape[2:]
        up = np.zeros((N, C) + tuple(s[a] * (x.shape[2 + a] - 1) + 1 for a in range(nsp)))
        up[(slice(None), slice(None)) + tuple(slice(None, None, s[a]) for a in range(nsp))] = x
        for a in range(nsp):  # pad / crop axis a
            before = d[a] * (Ks[a] - 1) - pads[a]
            after = d[a] * (Ks[a] - 1) - pads[a + nsp] + op[a]
            ax = 2 + a
            if before < 0:
                up = np.take(up, range(-before, up.shape[ax]), axis=ax)
                before = 0
            if after < 0:
                up = np.take(up, range(0, up.shape[ax] + after), axis=ax)
                after = 0
            pw = [(0, 0)] * up.ndim
            pw[ax] = (before, after)
            up = np.pad(up, pw)
        Osz = [up.shape[2 + a] - d[a] * (Ks[a] - 1) for a in range(nsp)]
        if min(Osz) < 0:
            continue
        y = np.zeros((N, Mg * G, *Osz))
        for g in range(G):
            xs = up[:, g * Cg:(g + 1) * Cg]
            for k in itertools.product(*[range(v) for v in Ks]):
                win = xs[(slice(None), slice(None)) +
                         tuple(slice(k[a] * d[a], k[a] * d[a] + Osz[a]) for a in range(nsp))]
                flip = tuple(Ks[a] - 1 - k[a] for a in range(nsp))
                wk = w[(slice(g * Cg, (g + 1) * Cg), slice(None)) + flip]  # [Cg, Mg]
                y[:, g * Mg:(g + 1) * Mg] += np.einsum("nc...,cm->nm...", win, wk)
        if b is not None:
            y += b.reshape((1, -1) + (1,) * nsp)
        _close(O.convtranspose(x, w, b, lib=lib, **attrs), y)


def pin_numpy_convolve(lib, count=60, seed=14):
    """1-D, one channel: the footprint is numpy.convolve of the zero-inserted signal with
    the dilated filter (the polynomial identity sum_o y[o] z^(o+b) = x(z^s) w(z^d))."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        L, K = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        s, d = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        op = int(rng.integers(0, max(s, d)))
        pads = [int(rng.integers(0, 4)), int(rng.integers(0, 4))]
        x, w = rng.normal(size=L), rng.normal(size=K)
        bias = float(rng.normal())
        xu = np.zeros(s * (L - 1) + 1)
        xu[::s] = x
        wd = np.zeros(d * (K - 1) + 1)
        wd[::d] = w
        full = np.convolve(xu, wd)
        On = len(full) + op - pads[0] - pads[1]
        if On < 0:
            continue
        want = np.zeros(On)
        for o in range(On):
            q = o + pads[0]
            if 0 <= q < len(full):
                want[o] = full[q]
        got = O.convtranspose(x.reshape(1, 1, L), w.reshape(1, 1, K), np.array([bias]), lib=lib,
                              strides=[s], dilations=[d], pads=pads, output_padding=[op])
        _close(got.reshape(-1), want + bias)


def forward_conv_adjoint(a, w, attrs, in_sizes, pads_begin):
    """ONNX forward Conv that reads the same W as (C out, M/group in, k..): maps a Y-shaped
    tensor back to X's shape, out[n,c,i] = sum_{m,k} a[n,m,i*s-b+k*d] W[c,m',k]."""
    nsp = a.ndim - 2
    s = attrs.get("strides") or [1] * nsp
    d = attrs.get("dilations") or [1] * nsp
    Ks = w.shape[2:]
    t = torch.from_numpy(a)
    for ax in range(nsp):  # pad/crop so that index q = o + b starts at 0 and is long enough
        b = pads_begin[ax]
        dim = 2 + ax
        if b < 0:
            t = t.narrow(dim, -b, t.shape[dim] + b) if t.shape[dim] + b > 0 else t.narrow(dim, 0, 0)
            b = 0
        need = (in_sizes[ax] - 1) * s[ax] + d[ax] * (Ks[ax] - 1) + 1
        after = max(0, need - (t.shape[dim] + b))
        shape_b = list(t.shape)
        shape_b[dim] = b
        shape_a = list(t.shape)
        shape_a[dim] = after
        t = torch.cat([torch.zeros(shape_b, dtype=t.dtype), t, torch.zeros(shape_a, dtype=t.dtype)], dim)
    out = _CV[nsp](t, torch.from_numpy(w), stride=tuple(s), dilation=tuple(d),
                   groups=int(attrs.get("group", 1)))
    sl = (slice(None), slice(None)) + tuple(slice(0, in_sizes[ax]) for ax in range(nsp))
    return out[sl].numpy()


def pin_adjoint(lib, count=80, seed=15):
    """<Conv_W(a), x> == <a, ConvT_W(x)> with no bias, Conv_W the forward convolution
    using the same W, strides, dilations and begin pads."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        x, w, _, attrs = random_case(rng, auto=(t % 3 == 2))
        nsp = x.ndim - 2
        y = O.convtranspose(x, w, None, lib=lib, **attrs)
        _, pads = O.output_shape(x.shape, w.shape, lib=lib, **attrs)
        a = rng.normal(size=y.shape)
        lhs = float(np.sum(forward_conv_adjoint(a, w, attrs, x.shape[2:], pads[:nsp]) * x))
        rhs = float(np.sum(a * y))
        assert abs(lhs - rhs) <= 1e-10 * (1.0 + abs(lhs)), (lhs, rhs, attrs)


def pin_stride1_forward(lib, count=60, seed=16):
    """At stride 1 the transposed convolution is a forward convolution of X with the
    tap-reversed, channel-swapped filter, begin pad d(K-1)-b and end pad d(K-1)-e+op."""
    rng = np.random.default_rng(seed)
    done = 0
    while done < count:
        x, w, b, attrs = random_case(rng)
        nsp = x.ndim - 2
        attrs["strides"] = [1] * nsp
        d = attrs["dilations"]
        attrs["output_padding"] = [int(rng.integers(0, di)) for di in d]
        pads = attrs["pads"]
        G = attrs["group"]
        C, Mg = w.shape[0], w.shape[1]
        Cg = C // G
        Ks = w.shape[2:]
        try:
            O.output_shape(x.shape, w.shape, lib=lib, **attrs)
        except O.OracleError:
            continue
        wt = torch.from_numpy(w).reshape(G, Cg, Mg, *Ks).transpose(1, 2).reshape(G * Mg, Cg, *Ks)
        wt = torch.flip(wt, dims=list(range(2, 2 + nsp)))
        t = torch.from_numpy(x)
        for ax in range(nsp):
            pb = d[ax] * (Ks[ax] - 1) - pads[ax]
            pe = d[ax] * (Ks[ax] - 1) - pads[ax + nsp] + attrs["output_padding"][ax]
            t = _pad_or_crop(t, 2 + ax, pb, pe)
            if t is None:
                break
        if t is None or any(t.shape[2 + ax] < d[ax] * (Ks[ax] - 1) + 1 for ax in range(nsp)):
            continue  # everything cropped away; covered by the other pins
        want = _CV[nsp](t, wt, dilation=tuple(d), groups=G).numpy()
        if b is not None:
            want = want + b.reshape((1, -1) + (1,) * nsp)
        _close(O.convtranspose(x, w, b, lib=lib, **attrs), want)
        done += 1


def _pad_or_crop(t, dim, before, after):
    """Zero-pad (positive) or crop (negative) a tensor along dim; None if nothing is left."""
    if t.shape[dim] + min(before, 0) + min(after, 0) <= 0:
        return None
    if before < 0:
        t = t.narrow(dim, -before, t.shape[dim] + before)
        before = 0
    if after < 0:
        t = t.narrow(dim, 0, t.shape[dim] + after)
        after = 0
    zb = list(t.shape)
    zb[dim] = before
    ze = list(t.shape)
    ze[dim] = after
    return torch.cat([torch.zeros(zb, dtype=t.dtype), t, torch.zeros(ze, dtype=t.dtype)], dim)


def pin_pointwise_matmul(lib, count=30, seed=17):
    """1x..x1 kernel, stride 1, no pads: a per-group channel matmul at every pixel."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        nsp = int(rng.integers(1, 4))
        G = int(rng.integers(1, 4))
        Cg, Mg = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        sp = tuple(int(v) for v in rng.integers(1, 5, size=nsp))
        x = rng.normal(size=(2, G * Cg) + sp)
        w = rng.normal(size=(G * Cg, Mg) + (1,) * nsp)
        b = rng.normal(size=G * Mg)
        want = np.concatenate([
            np.einsum("nc...,cm->nm...", x[:, g * Cg:(g + 1) * Cg],
                      w[g * Cg:(g + 1) * Cg].reshape(Cg, Mg)) for g in range(G)], axis=1)
        want += b.reshape((1, -1) + (1,) * nsp)
        _close(O.convtranspose(x, w, b, lib=lib, group=G), want)


def pin_group_split(lib, count=40, seed=18):
    """A group-G result equals G independent group-1 results on the channel slices."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        x, w, b, attrs = random_case(rng)
        G = attrs["group"]
        if G == 1:
            continue
        Cg, Mg = x.shape[1] // G, w.shape[1]
        whole = O.convtranspose(x, w, b, lib=lib, **attrs)
        parts = []
        for g in range(G):
            a1 = dict(attrs, group=1)
            parts.append(O.convtranspose(x[:, g * Cg:(g + 1) * Cg], w[g * Cg:(g + 1) * Cg],
                                         None if b is None else b[g * Mg:(g + 1) * Mg], lib=lib, **a1))
        _close(whole, np.concatenate(parts, axis=1), tol=0.0)


def pin_linearity_translation(lib, count=30, seed=19):
    """Linear in X; bias adds per channel; shifting X by one sample along an axis shifts
    the (unpadded) output by one stride."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        x, w, b, attrs = random_case(rng)
        nsp = x.ndim - 2
        x2 = rng.normal(size=x.shape)
        y1 = O.convtranspose(x, w, None, lib=lib, **attrs)
        y2 = O.convtranspose(x2, w, None, lib=lib, **attrs)
        y12 = O.convtranspose(2.0 * x - 3.0 * x2, w, None, lib=lib, **attrs)
        _close(y12, 2.0 * y1 - 3.0 * y2, tol=1e-11)
        if b is not None:
            yb = O.convtranspose(x, w, b, lib=lib, **attrs)
            _close(yb - y1, np.broadcast_to(b.reshape((1, -1) + (1,) * nsp), y1.shape), tol=1e-12)
        plain = dict(strides=attrs["strides"], dilations=attrs["dilations"], group=attrs["group"])
        ax = int(rng.integers(0, nsp))
        s = attrs["strides"][ax]
        shifted = np.concatenate([np.zeros_like(np.take(x, [0], axis=2 + ax)), x], axis=2 + ax)
        ya = O.convtranspose(x, w, None, lib=lib, **plain)
        yb = O.convtranspose(shifted, w, None, lib=lib, **plain)
        assert yb.shape[2 + ax] == ya.shape[2 + ax] + s
        _close(np.take(yb, range(s, yb.shape[2 + ax]), axis=2 + ax), ya, tol=0.0)
        assert not np.any(np.take(yb, range(0, s), axis=2 + ax))


def pin_useful_macs(lib, count=60, seed=20):
    """The useful-MAC count equals the sum of Y for all-ones X and W without bias
    (each useful (n, c, m, i, k) term contributes exactly 1)."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        x, w, _, attrs = random_case(rng, auto=(t % 3 == 1))
        ones_y = O.convtranspose(np.ones_like(x), np.ones_like(w), None, lib=lib, **attrs)
        assert O.useful_macs(x.shape, w.shape, lib=lib, **attrs) == int(round(ones_y.sum()))


def pin_points_match_whole(lib, count=30, seed=21):
    """Selected-output evaluation equals the whole-output routine bit for bit."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        x, w, b, attrs = random_case(rng)
        y = O.convtranspose(x, w, b, lib=lib, **attrs)
        if y.size == 0:
            continue
        pts = np.stack([rng.integers(0, v, size=25) for v in y.shape], axis=1)
        got = O.convtranspose_at(x, w, b, pts, lib=lib, **attrs)
        assert np.array_equal(got, y[tuple(pts.T)])


def pin_rejects_invalid(lib):
    """Attribute and shape errors are refused (README Attributes table; ClikaRT page:
    inconsistent channel/group arithmetic or span length raises)."""
    xs, ws = (1, 4, 5, 5), (4, 3, 3, 3)
    bad = [
        dict(strides=[0, 1]),
        dict(dilations=[1, 0]),
        dict(group=0),
        dict(group=3),                                  # C=4 not divisible
        dict(output_padding=[2, 0], strides=[2, 2]),    # op >= max(s, d)
        dict(output_padding=[1, 0]),                    # op >= 1 at s=d=1
        dict(pads=[-1, 0, 0, 0]),
        dict(pads=[1, 1, 1, 1], auto_pad="SAME_UPPER"),
        dict(kernel_shape=[3, 2]),
        dict(output_shape=[7, 8], pads=[0, 0, 0, 0]),  # pads disagree with output_shape
        dict(pads=[5, 5, 5, 5]),                        # negative output size
    ]
    for at in bad:
        try:
            O.output_shape(xs, ws, lib=lib, **at)
        except O.OracleError:
            continue
        raise AssertionError(f"accepted invalid attributes {at}")
    for xs2, ws2 in [((1, 4, 5, 5), (3, 3, 3, 3)), ((1, 4, 5), (4, 3, 3, 3)), ((1, 4, 5, 5, 5, 5), (4, 3, 1, 1, 1, 1))]:
        try:
            O.output_shape(xs2, ws2, lib=lib)
        except O.OracleError:
            continue
        raise AssertionError(f"accepted mismatched shapes {xs2} {ws2}")


def pin_activation_closed_forms(lib, seed=22):
    """The output activations against closed forms built from |v| (not from the
    comparisons the oracle uses): relu(v) = (v + |v|) / 2, leaky(v) = relu(v) - a relu(-v),
    clip(v) = lo + relu(v - lo) - relu(v - hi); identity leaves Y alone; undefined
    parameter sets are refused."""
    rng = np.random.default_rng(seed)
    v = np.concatenate([rng.normal(size=500) * 3, [0.0, -0.0, 1.5, -1.5, 2.0, -2.0]])
    relu = lambda t: (t + np.abs(t)) / 2
    assert np.array_equal(O.activation(v, "identity"), v)
    assert np.allclose(O.activation(v, "relu"), relu(v), rtol=0, atol=1e-15)
    for a in (0.0, 0.01, 0.25, 1.0, -0.5, 3.0):
        assert np.allclose(O.activation(v, "leaky_relu", (a,)), relu(v) - a * relu(-v), rtol=0, atol=1e-14)
    for lo, hi in ((-1.0, 1.0), (0.0, 6.0), (-2.0, -2.0), (-0.5, 4.0)):
        assert np.allclose(O.activation(v, "clip", (lo, hi)), lo + relu(v - lo) - relu(v - hi), rtol=0, atol=1e-14)
    # applied to a transposed convolution: elementwise on the whole output
    x = rng.normal(size=(2, 3, 5))
    w = rng.normal(size=(3, 2, 3))
    b = rng.normal(size=2)
    y = O.convtranspose(x, w, b, lib=lib, strides=[2], pads=[1, 0])
    assert np.allclose(O.activation(y, "relu"), relu(y), rtol=0, atol=1e-14)
    for kind, params in (("relu", (1.0,)), ("leaky_relu", ()), ("leaky_relu", (np.inf,)),
                         ("clip", (1.0, 0.0)), ("clip", (0.0,)), ("gelu", ())):
        try:
            O.activation(y, kind, params)
        except O.OracleError:
            continue
        raise AssertionError(f"activation {kind} {params} accepted")


# ------------------------------------------------------------------------------------
# Forward convolution (ONNX Conv, the adjoint of the transposed convolution)
# ------------------------------------------------------------------------------------
def random_conv_case(rng: np.random.Generator, nsp=None, auto=False, max_L=7):
    """A random small forward-convolution problem (W is (M, C/group, k..))."""
    while True:
        n = int(nsp or rng.integers(1, 4))
        group = int(rng.choice([1, 1, 2, 3]))
        Cg, Mg = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 3))
        Ls = [int(rng.integers(1, max_L + 1)) for _ in range(n)]
        Ks = [int(rng.integers(1, 4)) for _ in range(n)]
        s = [int(rng.integers(1, 4)) for _ in range(n)]
        d = [int(rng.integers(1, 3)) for _ in range(n)]
        attrs = dict(strides=s, dilations=d, group=group)
        if auto:
            attrs["auto_pad"] = str(rng.choice(["SAME_UPPER", "SAME_LOWER", "VALID"]))
        else:
            attrs["pads"] = [int(rng.integers(0, 3)) for _ in range(2 * n)]
        x = rng.normal(size=(N, Cg * group, *Ls))
        w = rng.normal(size=(Mg * group, Cg, *Ks))
        b = rng.normal(size=(Mg * group,)) if rng.random() < 0.7 else None
        try:
            ys, _ = O.conv_output_shape(x.shape, w.shape, **attrs)
        except O.OracleError:
            continue
        if min(ys) == 0:
            continue
        return x, w, b, attrs


def pin_conv_torch_library(lib, count=120, seed=31):
    """The forward convolution against PyTorch's CPU convolution in float64 on the input
    zero-padded by the applied pads (PyTorch takes symmetric padding only)."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        x, w, b, attrs = random_conv_case(rng, auto=(t % 4 == 3))
        nsp = x.ndim - 2
        ys, pads = O.conv_output_shape(x.shape, w.shape, lib=lib, **attrs)
        fpad = []
        for a in reversed(range(nsp)):  # F.pad takes the last axis first
            fpad += [pads[a], pads[nsp + a]]
        for a in range(nsp):  # a padded axis shorter than the dilated kernel has no output
            if x.shape[2 + a] + pads[a] + pads[nsp + a] < attrs["dilations"][a] * (w.shape[2 + a] - 1) + 1:
                raise AssertionError(f"outputs {ys} where no window fits the padded input: {attrs}")
        xt = F.pad(torch.from_numpy(x), fpad)
        ref = _CV[nsp](xt, torch.from_numpy(w), None if b is None else torch.from_numpy(b),
                       stride=tuple(attrs["strides"]), dilation=tuple(attrs["dilations"]),
                       groups=attrs["group"]).numpy()
        got = O.conv(x, w, b, lib=lib, **attrs)
        assert got.shape == ref.shape == tuple(ys), (got.shape, ref.shape, attrs)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), attrs
    # SAME_UPPER at stride 1 is PyTorch's padding="same" (extra pad at the end)
    for t in range(30):
        x, w, b, attrs = random_conv_case(rng)
        attrs = dict(strides=[1] * (x.ndim - 2), dilations=attrs["dilations"], group=attrs["group"],
                     auto_pad="SAME_UPPER")
        got = O.conv(x, w, b, lib=lib, **attrs)
        ref = _CV[x.ndim - 2](torch.from_numpy(x), torch.from_numpy(w), None if b is None else torch.from_numpy(b),
                              dilation=tuple(attrs["dilations"]), groups=attrs["group"], padding="same").numpy()
        assert got.shape == ref.shape and np.allclose(got, ref, rtol=1e-12, atol=1e-12), attrs
    # SAME keeps ceil(L / s) outputs (QLinearConv Attributes, auto_pad)
    for t in range(60):
        x, w, b, attrs = random_conv_case(rng)
        for mode in ("SAME_UPPER", "SAME_LOWER"):
            a2 = dict(strides=attrs["strides"], dilations=attrs["dilations"], group=attrs["group"], auto_pad=mode)
            ys, _ = O.conv_output_shape(x.shape, w.shape, lib=lib, **a2)
            assert list(ys[2:]) == [-(-L // s) for L, s in zip(x.shape[2:], attrs["strides"])]


def pin_conv_brute_force(lib, count=40, seed=32):
    """Tiny problems by a different loop nest: every input sample is sent to the outputs
    o with o*s - b + k*d equal to its index (a scatter, where the oracle gathers)."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        x, w, b, attrs = random_conv_case(rng, max_L=5)
        nsp = x.ndim - 2
        ys, pads = O.conv_output_shape(x.shape, w.shape, lib=lib, **attrs)
        s, d, G = attrs["strides"], attrs["dilations"], attrs["group"]
        Mg, Cg = w.shape[0] // G, w.shape[1]
        y = np.zeros(ys)
        if b is not None:
            y += b.reshape((1, -1) + (1,) * nsp)
        for idx in np.ndindex(*x.shape):
            n, c, i = idx[0], idx[1], idx[2:]
            g = c // Cg
            for k in np.ndindex(*w.shape[2:]):
                o = []
                for a in range(nsp):
                    q = i[a] + pads[a] - k[a] * d[a]
                    if q < 0 or q % s[a] or q // s[a] >= ys[2 + a]:
                        break
                    o.append(q // s[a])
                else:
                    for mm in range(Mg):
                        m = g * Mg + mm
                        y[(n, m) + tuple(o)] += x[idx] * w[(m, c - g * Cg) + k]
        assert np.allclose(O.conv(x, w, b, lib=lib, **attrs), y, rtol=1e-12, atol=1e-12), attrs


def pin_conv_adjoint(lib, count=80, seed=33):
    """<ConvT_W(x), a> == <x, Conv_W(a)>: the forward convolution with the same W,
    strides, dilations and begin pads, and end pads e - output_padding, is the adjoint
    of the (separately pinned) transposed convolution."""
    rng = np.random.default_rng(seed)
    done = 0
    while done < count:
        x, w, _, attrs = random_case(rng)
        nsp = x.ndim - 2
        _, pads = O.output_shape(x.shape, w.shape, lib=lib, **attrs)
        op = attrs["output_padding"]
        ends = [pads[nsp + a] - op[a] for a in range(nsp)]
        if min(ends) < 0 or min(pads[:nsp]) < 0:
            continue
        y = O.convtranspose(x, w, None, lib=lib, **attrs)
        a = rng.normal(size=y.shape)
        cattrs = dict(strides=attrs["strides"], dilations=attrs["dilations"], group=attrs["group"],
                      pads=list(pads[:nsp]) + ends)
        back = O.conv(a, w, None, lib=lib, **cattrs)
        assert back.shape == x.shape, (back.shape, x.shape, attrs)
        lhs, rhs = float(np.sum(a * y)), float(np.sum(x * back))
        assert abs(lhs - rhs) <= 1e-10 * (1.0 + abs(lhs)), (lhs, rhs, attrs)
        done += 1


def pin_conv_rejects_invalid(lib):
    x, w = np.zeros((1, 4, 6, 6)), np.zeros((6, 2, 3, 3))
    bad = [dict(group=3), dict(group=2, strides=[0, 1]), dict(group=2, dilations=[1, 0]),
           dict(group=2, pads=[1, 1, -1, 0]), dict(group=2, pads=[1, 1, 1, 1], auto_pad="VALID"),
           dict(group=2, kernel_shape=[3, 2])]
    for attrs in bad:
        try:
            O.conv(x, w, None, lib=lib, **attrs)
        except O.OracleError:
            continue
        raise AssertionError(f"accepted {attrs}")
    O.conv(x, w, None, lib=lib, group=2)  # the valid base case


# ----------------------------------------------------------------------------------
# quantized transposed convolution (QLinear scheme of the "ai.onnx.QLinearConv" README)
# ----------------------------------------------------------------------------------
QT = {"uint8": (0, 255), "int8": (-128, 127)}


def random_qcase(rng: np.random.Generator, auto=False, margin=0):
    """A random small quantized problem: uint8 / int8 operands and output, per-tensor or
    per-output-channel weight parameters, optional int32 bias.  ``margin`` keeps values
    that far inside their type's range."""
    x, w, _, attrs = random_case(rng, auto=auto)
    tx, tw, ty = (str(rng.choice(["uint8", "int8"])) for _ in range(3))
    M = w.shape[1] * attrs.get("group", 1)
    nq = M if rng.random() < 0.5 else 1
    draw = lambda t, size=None: rng.integers(QT[t][0] + margin, QT[t][1] - margin + 1, size=size)  # noqa: E731
    q = dict(x=draw(tx, x.shape), w=draw(tw, w.shape), x_scale=np.float32(rng.uniform(0.005, 0.05)),
             x_zero_point=int(draw(tx)), w_scale=rng.uniform(0.002, 0.05, size=nq).astype(np.float32),
             w_zero_point=draw(tw, nq), y_scale=np.float32(rng.uniform(0.02, 1.0)), y_zero_point=int(draw(ty)),
             y_type=ty, bias=rng.integers(-20000, 20001, size=M) if rng.random() < 0.7 else None)
    return q, attrs, (tx, tw)


def _shifted_operands(q):
    """x - x_zp and w[c, m', k] - w_zp[group(c) * Mg + m'] as float64 (exact integers)."""
    x, w = q["x"], q["w"]
    C, Mg = w.shape[:2]
    M = q["bias"].shape[0] if q["bias"] is not None else None
    wz = np.asarray(q["w_zero_point"]).reshape(-1)
    G = 1 if wz.size == 1 else wz.size // Mg
    if wz.size == 1:
        wzc = np.full((C, Mg), wz[0])
    else:
        Cg = C // G
        m_of = (np.arange(C) // Cg)[:, None] * Mg + np.arange(Mg)[None, :]
        wzc = wz[m_of]
    del M
    return (x - q["x_zero_point"]).astype(np.float64), (w - wzc.reshape((C, Mg) + (1,) * (w.ndim - 2))).astype(np.float64)


def pin_qconv_accumulator(lib, count=120, seed=41):
    """The exact integer sums against PyTorch's float64 conv_transpose of the
    zero-point-shifted operands plus the bias (exact: every value is a small integer)."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        q, attrs, _ = random_qcase(rng, auto=(t % 4 == 3))
        _, acc = O.qconvtranspose(**q, return_acc=True, lib=lib, **attrs)
        xs, ws = _shifted_operands(q)
        ref = torch_reference(xs, ws, None if q["bias"] is None else q["bias"].astype(np.float64), attrs, lib)
        assert np.array_equal(ref, np.round(ref))
        assert np.array_equal(acc, ref.astype(np.int64)), f"case {t}: accumulators differ {attrs}"


def pin_qconv_dequantized(lib, count=120, seed=42):
    """Quantized outputs against the real-valued result: PyTorch's float64
    conv_transpose of the dequantized operands ((q - zero point) * scale) plus the
    dequantized bias, divided by y_scale, rounded half to even, shifted by y_zp and
    saturated.  The float32 requantization may differ from this float64 value only by
    one step, and only next to a rounding tie."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        q, attrs, _ = random_qcase(rng, auto=(t % 4 == 3))
        y = O.qconvtranspose(**q, lib=lib, **attrs)
        xs, ws = _shifted_operands(q)
        M = y.shape[1]
        wsc = np.broadcast_to(np.asarray(q["w_scale"], dtype=np.float64).reshape(-1), (M,))
        Mg, C = q["w"].shape[1], q["w"].shape[0]
        G = attrs.get("group", 1)
        wsc_c = wsc[((np.arange(C) // (C // G))[:, None] * Mg + np.arange(Mg)[None, :])]
        xr = xs * float(q["x_scale"])
        wr = ws * wsc_c.reshape((C, Mg) + (1,) * (ws.ndim - 2))
        br = None if q["bias"] is None else q["bias"] * float(q["x_scale"]) * wsc
        real = torch_reference(xr, wr, br, attrs, lib) / float(q["y_scale"])
        lo, hi = QT[q["y_type"]]
        want = np.clip(np.rint(real) + q["y_zero_point"], lo, hi)
        diff = np.abs(y - want)
        frac = np.abs(real - np.floor(real) - 0.5)
        near_tie = frac < 1e-4 * np.maximum(1.0, np.abs(real))
        assert np.all(diff <= 1) and np.all(near_tie[diff == 1]), \
            f"case {t}: {int((diff > 0).sum())} outputs differ from the dequantized result"


def pin_requantize_definition(lib):
    """Values fixed by the definition of the requantization step: round half to even,
    the zero point added after rounding, saturation to the output type, and the int32
    accumulator taken modulo 2^32."""
    acc = np.arange(-5, 6)
    # multiplier 1 * 0.5 / 1 = 0.5 exactly: -2.5 .. 2.5 in steps of 0.5
    want = np.array([-2, -2, -2, -1, 0, 0, 0, 1, 2, 2, 2])
    assert np.array_equal(O.requantize(acc, 1.0, [0.5], 0, 1.0, 0, "int8", lib=lib), want)
    assert np.array_equal(O.requantize(acc, 1.0, [0.5], 0, 1.0, 10, "uint8", lib=lib), want + 10)
    # multiplier 0.5 * 0.5 / 1 = 0.25: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -1.5 -> -2
    assert np.array_equal(O.requantize([2, 6, 10, -6], 0.5, [0.5], 0, 1.0, 0, "int8", lib=lib), [0, 2, 2, -2])
    # per-channel multipliers: channel 1 has w_scale 2 (multiplier 2)
    assert np.array_equal(O.requantize([3, 3], 1.0, [0.5, 2.0], [0, 1], 1.0, 0, "int8", lib=lib), [2, 6])
    # saturation after the zero point
    assert np.array_equal(O.requantize([1000, -1000, 490, 500], 1.0, [0.5], 0, 1.0, 10, "uint8", lib=lib),
                          [255, 0, 255, 255])
    assert np.array_equal(O.requantize([1000, -1000, 234, 236], 1.0, [0.5], 0, 1.0, 10, "int8", lib=lib),
                          [127, -128, 127, 127])
    assert np.array_equal(O.requantize([-276, -278], 1.0, [0.5], 0, 1.0, 10, "int8", lib=lib), [-128, -128])
    assert np.array_equal(O.requantize([-274], 1.0, [0.5], 0, 1.0, 10, "int8", lib=lib), [-127])
    # int32 accumulator: 2^32 + 3 wraps to 3, 2^31 wraps to -2^31
    assert np.array_equal(O.requantize([2 ** 32 + 3], 1.0, [1.0], 0, 1.0, 0, "int8", lib=lib), [3])
    assert np.array_equal(O.requantize([2 ** 31], 1.0, [1.0], 0, 1.0, 0, "int8", lib=lib), [-128])


def pin_qconv_zero_point_shifts(lib, count=40, seed=43):
    """Moving x (or w) and its zero point by the same amount leaves every output
    unchanged; per-channel parameters that are all equal act like per-tensor ones."""
    rng = np.random.default_rng(seed)
    for t in range(count):
        q, attrs, (tx, tw) = random_qcase(rng, margin=8)
        y = O.qconvtranspose(**q, lib=lib, **attrs)
        dx, dw = int(rng.integers(-8, 9)), int(rng.integers(-8, 9))
        q2 = dict(q, x=q["x"] + dx, x_zero_point=q["x_zero_point"] + dx, w=q["w"] + dw,
                  w_zero_point=np.asarray(q["w_zero_point"]) + dw)
        assert np.array_equal(O.qconvtranspose(**q2, lib=lib, **attrs), y), f"case {t}: zero-point shift"
        M = y.shape[1]
        q3 = dict(q, w_scale=np.full(M, q["w_scale"][0], np.float32),
                  w_zero_point=np.full(M, np.asarray(q["w_zero_point"]).reshape(-1)[0]))
        q4 = dict(q, w_scale=q["w_scale"][:1], w_zero_point=np.asarray(q["w_zero_point"]).reshape(-1)[:1])
        assert np.array_equal(O.qconvtranspose(**q3, lib=lib, **attrs), O.qconvtranspose(**q4, lib=lib, **attrs))


ALL_PINS = [pin_activation_closed_forms, pin_golden, pin_benchmark_shapes, pin_torch_library, pin_brute_force_gather,
            pin_zero_insertion, pin_numpy_convolve, pin_adjoint, pin_stride1_forward,
            pin_pointwise_matmul, pin_group_split, pin_linearity_translation, pin_useful_macs,
            pin_points_match_whole, pin_rejects_invalid, pin_conv_torch_library, pin_conv_brute_force,
            pin_conv_adjoint, pin_conv_rejects_invalid, pin_qconv_accumulator, pin_qconv_dequantized,
            pin_requantize_definition, pin_qconv_zero_point_shifts]
