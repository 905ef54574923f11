"""Planted mistakes in copies of the oracle: each one must make some pin fail.

Every mutant is a textual edit of ct_oracle.c compiled into a temporary library and
checked in a subprocess, so the oracle source itself carries no mutation hooks.  Each
edit keeps every memory access in bounds."""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "begin_pad_sign": ("* g.s[a] - g.b[a] + kc[a] * g.d[a];", "* g.s[a] + g.b[a] + kc[a] * g.d[a];"),
    "end_pad_for_begin": ("* g.s[a] - g.b[a] + kc[a] * g.d[a];", "* g.s[a] - g.e[a] + kc[a] * g.d[a];"),
    "stride_dilation_swapped": ("icoord[a] * g.s[a] - g.b[a] + kc[a] * g.d[a];",
                                "icoord[a] * g.d[a] - g.b[a] + kc[a] * g.s[a];"),
    "dilation_ignored": ("+ kc[a] * g.d[a];", "+ kc[a];"),
    "weight_read_as_M_C": ("w + (c * g.Mg + mm) * taps", "w + (mm * g.C + c) * taps"),
    "taps_reversed": ("yp[flat] += xv * wp[kk];", "yp[flat] += xv * wp[taps - 1 - kk];"),
    "bias_dropped": ("bias ? bias[m] : 0.0", "0.0"),
    "output_padding_dropped": ("full = s * (L - 1) + op + d * (K - 1) + 1;",
                               "full = s * (L - 1) + d * (K - 1) + 1;"),
    "footprint_off_by_one": ("full = s * (L - 1) + op + d * (K - 1) + 1;",
                             "full = s * (L - 1) + op + d * (K - 1);"),
    "same_sides_swapped": ("            if (auto_pad == OR_SAME_UPPER) {",
                           "            if (auto_pad == OR_SAME_LOWER) {"),
    "same_split_floor": ("            if (auto_pad == OR_SAME_UPPER) {\n                b = tot / 2;",
                         "            if (auto_pad == OR_SAME_UPPER) {\n                b = tot >= 0 ? tot / 2 : (tot - 1) / 2;"),
    "output_shape_extra_at_begin": ("} else if (auto_pad == OR_SAME_LOWER) {",
                                    "} else if (auto_pad != OR_SAME_LOWER) {"),
    "group_of_out_channel": ("int64_t grp = m / g.Mg, mm = m % g.Mg;",
                             "int64_t grp = m % g.group, mm = m / g.group;"),
    "group_channels_interleaved": ("int64_t c = grp * g.Cg + cc;", "int64_t c = cc * g.group + grp;"),
    "points_pad_sign": ("if (i * g.s[a] - g.b[a] + k * g.d[a] == o) {",
                        "if (i * g.s[a] + g.b[a] + k * g.d[a] == o) {"),
    "useful_macs_upper_bound_inclusive": ("if (o >= 0 && o < g.O[a])\n                    hits++;",
                                          "if (o >= 0 && o <= g.O[a])\n                    hits++;"),
    # forward convolution
    "conv_pad_sign": ("int64_t i = ocoord[a] * g.s[a] - g.b[a] + kc[a] * g.d[a];",
                      "int64_t i = ocoord[a] * g.s[a] + g.b[a] + kc[a] * g.d[a];"),
    "conv_dilation_ignored": ("int64_t i = ocoord[a] * g.s[a] - g.b[a] + kc[a] * g.d[a];",
                              "int64_t i = ocoord[a] * g.s[a] - g.b[a] + kc[a];"),
    "conv_group_channels": ("x + (n * g.C + grp * g.Cg + cc) * in_plane", "x + (n * g.C + cc) * in_plane"),
    "conv_output_size_rounded_up": ("g->O[a] = num >= 0 ? num / s + 1 : 0;",
                                    "g->O[a] = num >= 0 ? (num + s - 1) / s + 1 : 0;"),
    "conv_same_total_off_by_one": ("tot = (O - 1) * s + d * (K - 1) + 1 - L;", "tot = (O - 1) * s + d * (K - 1) - L;"),
    "conv_weight_read_transposed": ("const double *wp = w + (m * g.Cg + cc) * taps;",
                                    "const double *wp = w + (cc * g.M + m) * taps;"),
    # quantized transposed convolution
    "q_x_zero_point_dropped": ("int64_t xv = (int64_t)xp[ii] - x_zp;", "int64_t xv = (int64_t)xp[ii];"),
    "q_w_zero_point_per_tensor": ("acc[flat] += xv * ((int64_t)wp[kk] - w_zp[q]);",
                                  "acc[flat] += xv * ((int64_t)wp[kk] - w_zp[0]);"),
    "q_w_scale_per_tensor": ("float mult = or_requant_mult(x_scale, w_scale[q], y_scale);",
                             "float mult = or_requant_mult(x_scale, w_scale[0], y_scale);"),
    "q_bias_dropped": ("acc[p] = bias ? bias[m] : 0;", "acc[p] = 0;"),
    "q_round_half_away": ("float r = rintf(v);", "float r = roundf(v);"),
    "q_round_truncate": ("float r = rintf(v);", "float r = truncf(v);"),
    "q_no_upper_saturation": ("    if (q > (double)y_hi)\n        return y_hi;\n", ""),
    "q_y_zero_point_dropped": ("double q = (double)r + (double)y_zp;", "double q = (double)r;"),
    "q_y_zero_point_before_rounding": ("volatile float v = (float)acc32 * mult;",
                                       "volatile float v = (float)acc32 * mult + (float)y_zp;"),
    "q_multiplier_inverted": ("volatile float mult = xw / y_scale;", "volatile float mult = xw * y_scale;"),
    "q_accumulator_not_wrapped": ("volatile float v = (float)acc32 * mult;", "volatile float v = (float)acc * mult;"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(O.__file__), "ct_oracle.c")).read()
    assert old in src, f"mutant {name}: pattern not found in ct_oracle.c"
    path_c = os.path.join(tmp, f"{name}.c")
    path_so = os.path.join(tmp, f"lib{name}.so")
    open(path_c, "w").write(src.replace(old, new))
    O.build(path_c, path_so)
    r = subprocess.run([sys.executable, os.path.join(HERE, "_mutant_runner.py"), path_so, name],
                       capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=6) as ex:
            res = dict(zip(MUTANTS, ex.map(lambda n: _run_mutant(n, tmp), MUTANTS)))
    missed = {n: out for n, (rc, out) in res.items() if rc != 0}
    assert not missed, f"mutants not caught by any pin: {missed}"


ACT_MUTANTS = {
    # plausible slips in the activation, each planted into a wrapper of the oracle's own
    "relu_keeps_negatives": lambda f: lambda y, k="identity", p=(): (
        np.abs(np.asarray(y, dtype=np.float64)) if k == "relu" else f(y, k, p)),
    "leaky_slope_on_positive_side": lambda f: lambda y, k="identity", p=(): (
        np.where(np.asarray(y) >= 0, p[0] * np.asarray(y), np.asarray(y)) if k == "leaky_relu" else f(y, k, p)),
    "clip_bounds_swapped": lambda f: lambda y, k="identity", p=(): (
        np.minimum(np.maximum(np.asarray(y, dtype=np.float64), p[1]), p[0]) if k == "clip" and len(p) == 2 and p[0] <= p[1]
        else f(y, k, p)),
    "clip_upper_only": lambda f: lambda y, k="identity", p=(): (
        np.minimum(np.asarray(y, dtype=np.float64), p[1]) if k == "clip" and len(p) == 2 and p[0] <= p[1]
        else f(y, k, p)),
}


@pytest.mark.parametrize("name", sorted(ACT_MUTANTS))
def test_activation_mistakes_are_caught(name, monkeypatch):
    import pins
    monkeypatch.setattr(O, "activation", ACT_MUTANTS[name](O.activation))
    with pytest.raises(AssertionError):
        pins.pin_activation_closed_forms(O.load())
