/*
 * ct_oracle.c -- plain fp64 reference for the N-D transposed convolution
 * (ONNX ConvTranspose).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library.  It shares no code, header, table or helper
 * with the HIP library; it has its own attribute resolver.
 *
 * What it computes (webgpu-kernels "ai.onnx.ConvTranspose" README):
 *   - Description: the transpose of a convolution ("fractionally strided convolution",
 *     "deconvolution") of X by filter W plus an optional bias B, with grouping.
 *   - Inputs: X is (N, C, D1..Dn); W is (C, M/group, k1..kn); bias has length M.
 *   - Attributes: auto_pad, dilations, group, kernel_shape, output_padding,
 *     output_shape, pads (all begins, then all ends), strides.
 *   - Outputs: Y has X's rank; spatial sizes follow from input size, kernel, strides,
 *     dilations and padding.
 * The ClikaRT "conv_transpose" API page states the same weight convention
 * (input-channel first, C_out = weight[1]*groups) and that output_padding grows only
 * the high side of each output axis.
 *
 * Definition used (the scatter form of the transposed convolution): every input sample
 * X[n,c,i] is sent through every tap k of its group's filter to output position
 *     o_a = i_a*s_a - b_a + k_a*d_a      on each spatial axis a,
 * and added there when 0 <= o_a < O_a on all axes; out channel m = g*Mg + m' receives
 * from input channels c of group g = c / Cg through W[c, m', k].  Y starts at bias[m]
 * (or 0), so output positions no sample reaches hold the bias.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - output_padding must satisfy 0 <= op < max(stride, dilation);
 *   - strides and dilations are >= 1; explicit pads are >= 0;
 *   - explicit pads together with an auto_pad other than NOTSET are an error;
 *   - SAME_UPPER / SAME_LOWER give O = L*s; the total padding
 *     tot = s*(L-1) + op + d*(K-1) + 1 - O is split with C's truncating division,
 *     the odd extra going to the end (UPPER) or the beginning (LOWER);
 *   - output_shape, when given, sets O; tot is split as above (extra at the
 *     beginning only for SAME_LOWER); explicit pads given as well must sum to tot;
 *   - kernel_shape, when given, must equal W's spatial dims.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC ct_oracle.c -o libctoracle.so
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_INVALID 1

#define OR_NOTSET 0
#define OR_SAME_UPPER 1
#define OR_SAME_LOWER 2
#define OR_VALID 3

typedef struct {
    int nsp;
    int64_t N, C, M, group, Cg, Mg;
    int64_t L[3], K[3], s[3], d[3], b[3], e[3], op[3], O[3];
} or_geom;

static int or_fail(char *err, int errlen, const char *msg)
{
    if (err && errlen > 0) {
        strncpy(err, msg, (size_t)errlen - 1);
        err[errlen - 1] = 0;
    }
    return OR_INVALID;
}

/* Attribute defaults, validation, padding and output size (README, Attributes table). */
static int or_resolve(int nsp, const int64_t *xs, const int64_t *ws, int auto_pad,
                      const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                      const int64_t *output_padding, const int64_t *output_shape,
                      const int64_t *kernel_shape, int64_t group, or_geom *g,
                      char *err, int errlen)
{
    int a;
    if (nsp < 1 || nsp > 3)
        return or_fail(err, errlen, "spatial rank must be 1, 2 or 3");
    if (auto_pad < OR_NOTSET || auto_pad > OR_VALID)
        return or_fail(err, errlen, "unknown auto_pad");
    if (group < 1)
        return or_fail(err, errlen, "group must be >= 1");
    for (a = 0; a < nsp + 2; a++) {
        if (xs[a] < 0)
            return or_fail(err, errlen, "negative input dimension");
    }
    if (ws[0] != xs[1])
        return or_fail(err, errlen, "W.shape[0] must equal C");
    if (ws[1] < 1)
        return or_fail(err, errlen, "W.shape[1] (M/group) must be >= 1");
    if (xs[1] % group != 0)
        return or_fail(err, errlen, "C must be divisible by group");
    if (pads && auto_pad != OR_NOTSET)
        return or_fail(err, errlen, "explicit pads cannot be combined with auto_pad");

    g->nsp = nsp;
    g->N = xs[0];
    g->C = xs[1];
    g->group = group;
    g->Cg = xs[1] / group;
    g->Mg = ws[1];
    g->M = ws[1] * group;

    for (a = 0; a < nsp; a++) {
        int64_t L = xs[2 + a], K = ws[2 + a];
        int64_t s = strides ? strides[a] : 1;
        int64_t d = dilations ? dilations[a] : 1;
        int64_t op = output_padding ? output_padding[a] : 0;
        int64_t full, O, b, e, tot;
        if (K < 1)
            return or_fail(err, errlen, "kernel dimensions must be >= 1");
        if (kernel_shape && kernel_shape[a] != K)
            return or_fail(err, errlen, "kernel_shape must match W's spatial dims");
        if (s < 1)
            return or_fail(err, errlen, "strides must be >= 1");
        if (d < 1)
            return or_fail(err, errlen, "dilations must be >= 1");
        if (op < 0 || op >= (s > d ? s : d))
            return or_fail(err, errlen, "output_padding must be in [0, max(stride, dilation))");
        if (pads && (pads[a] < 0 || pads[a + nsp] < 0))
            return or_fail(err, errlen, "explicit pads must be >= 0");

        /* Size of the whole scatter footprint including output_padding. */
        full = s * (L - 1) + op + d * (K - 1) + 1;
        if (output_shape) {
            O = output_shape[a];
            if (O < 0)
                return or_fail(err, errlen, "output_shape entries must be >= 0");
            tot = full - O;
            if (pads) {
                if (pads[a] + pads[a + nsp] != tot)
                    return or_fail(err, errlen, "pads disagree with output_shape");
                b = pads[a];
                e = pads[a + nsp];
            } else if (auto_pad == OR_SAME_LOWER) {
                e = tot / 2;
                b = tot - e;
            } else {
                b = tot / 2;
                e = tot - b;
            }
        } else if (auto_pad == OR_SAME_UPPER || auto_pad == OR_SAME_LOWER) {
            O = L * s;
            tot = full - O;
            if (auto_pad == OR_SAME_UPPER) {
                b = tot / 2;
                e = tot - b;
            } else {
                e = tot / 2;
                b = tot - e;
            }
        } else if (auto_pad == OR_VALID) {
            b = 0;
            e = 0;
            O = full;
        } else {
            b = pads ? pads[a] : 0;
            e = pads ? pads[a + nsp] : 0;
            O = full - b - e;
        }
        if (O < 0)
            return or_fail(err, errlen, "resolved output size is negative");
        g->L[a] = L;
        g->K[a] = K;
        g->s[a] = s;
        g->d[a] = d;
        g->b[a] = b;
        g->e[a] = e;
        g->op[a] = op;
        g->O[a] = O;
    }
    return OR_OK;
}

static int64_t or_prod(const int64_t *v, int n)
{
    int64_t p = 1;
    int a;
    for (a = 0; a < n; a++)
        p *= v[a];
    return p;
}

/* Row-major decode of a flat index into per-axis coordinates (last axis fastest). */
static void or_decode(int64_t flat, const int64_t *dims, int n, int64_t *coord)
{
    int a;
    for (a = n - 1; a >= 0; a--) {
        coord[a] = flat % dims[a];
        flat /= dims[a];
    }
}

/* Threads the parallel loops below use (for reporting a timing's core count). */
int oracle_threads(void)
{
    return omp_get_max_threads();
}

/* Resolved shape of Y = (N, M, O1..On) and the begin/end pads actually applied. */
int oracle_output_shape(int nsp, const int64_t *x_shape, const int64_t *w_shape, int auto_pad,
                        const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                        const int64_t *output_padding, const int64_t *output_shape,
                        const int64_t *kernel_shape, int64_t group, int64_t *y_shape,
                        int64_t *pads_out, char *err, int errlen)
{
    or_geom g;
    int a, rc;
    rc = or_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, output_padding,
                    output_shape, kernel_shape, group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    y_shape[0] = g.N;
    y_shape[1] = g.M;
    for (a = 0; a < nsp; a++) {
        y_shape[2 + a] = g.O[a];
        if (pads_out) {
            pads_out[a] = g.b[a];
            pads_out[a + nsp] = g.e[a];
        }
    }
    return OR_OK;
}

/* Useful multiply-accumulates: (input sample, tap) pairs that land inside Y, times
 * N * Cg * M.  Counted by enumeration of every (i, k) pair on each axis. */
int oracle_useful_macs(int nsp, const int64_t *x_shape, const int64_t *w_shape, int auto_pad,
                       const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                       const int64_t *output_padding, const int64_t *output_shape,
                       const int64_t *kernel_shape, int64_t group, double *macs_out,
                       char *err, int errlen)
{
    or_geom g;
    int a, rc;
    double total;
    rc = or_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, output_padding,
                    output_shape, kernel_shape, group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    total = (double)g.N * (double)g.Cg * (double)g.M;
    for (a = 0; a < nsp; a++) {
        int64_t i, k, hits = 0;
        for (i = 0; i < g.L[a]; i++)
            for (k = 0; k < g.K[a]; k++) {
                int64_t o = i * g.s[a] - g.b[a] + k * g.d[a];
                if (o >= 0 && o < g.O[a])
                    hits++;
            }
        total *= (double)hits;
    }
    *macs_out = total;
    return OR_OK;
}

/* Whole output by the scatter definition.  y has N*M*prod(O) doubles (NCHW order).
 * Threads split the (n, m) output planes, which are written by one thread each; the
 * sum inside a plane runs c, then input index i, then tap k, all ascending, so the
 * result does not depend on the thread count. */
int oracle_convtranspose_f64(int nsp, const int64_t *x_shape, const double *x,
                             const int64_t *w_shape, const double *w, const double *bias,
                             int auto_pad, const int64_t *strides, const int64_t *dilations,
                             const int64_t *pads, const int64_t *output_padding,
                             const int64_t *output_shape, const int64_t *kernel_shape,
                             int64_t group, double *y, int64_t y_len, char *err, int errlen)
{
    or_geom g;
    int rc;
    int64_t in_plane, out_plane, taps, t, plane;
    int64_t *tap_coord;
    rc = or_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, output_padding,
                    output_shape, kernel_shape, group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    in_plane = or_prod(g.L, nsp);
    out_plane = or_prod(g.O, nsp);
    taps = or_prod(g.K, nsp);
    if (y_len != g.N * g.M * out_plane)
        return or_fail(err, errlen, "y buffer length does not match the resolved output");
    if (g.N * g.M * out_plane == 0)
        return OR_OK;

    tap_coord = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)(taps > 0 ? taps : 1));
    if (!tap_coord)
        return or_fail(err, errlen, "out of host memory");
    for (t = 0; t < taps; t++)
        or_decode(t, g.K, nsp, tap_coord + 3 * t);

#pragma omp parallel for schedule(dynamic, 1)
    for (plane = 0; plane < g.N * g.M; plane++) {
        int64_t n = plane / g.M, m = plane % g.M;
        int64_t grp = m / g.Mg, mm = m % g.Mg;
        double *yp = y + plane * out_plane;
        int64_t p, cc, ii, kk;
        int a;
        for (p = 0; p < out_plane; p++)
            yp[p] = bias ? bias[m] : 0.0;
        for (cc = 0; cc < g.Cg; cc++) {
            int64_t c = grp * g.Cg + cc;
            const double *xp = x + (n * g.C + c) * in_plane;
            const double *wp = w + (c * g.Mg + mm) * taps;
            for (ii = 0; ii < in_plane; ii++) {
                int64_t icoord[3];
                double xv = xp[ii];
                or_decode(ii, g.L, nsp, icoord);
                for (kk = 0; kk < taps; kk++) {
                    const int64_t *kc = tap_coord + 3 * kk;
                    int64_t flat = 0;
                    int inside = 1;
                    for (a = 0; a < nsp; a++) {
                        int64_t o = icoord[a] * g.s[a] - g.b[a] + kc[a] * g.d[a];
                        if (o < 0 || o >= g.O[a]) {
                            inside = 0;
                            break;
                        }
                        flat = flat * g.O[a] + o;
                    }
                    if (inside)
                        yp[flat] += xv * wp[kk];
                }
            }
        }
    }
    free(tap_coord);
    return OR_OK;
}

/* Selected outputs by the same definition: for each requested output position the sum
 * runs over exactly the (c, i, k) whose scatter target is that position, in the same
 * order as above (c, then i, then k), so each value equals the full routine's.
 * points holds npts rows of (n, m, o1..on). */
int oracle_convtranspose_at(int nsp, const int64_t *x_shape, const double *x,
                            const int64_t *w_shape, const double *w, const double *bias,
                            int auto_pad, const int64_t *strides, const int64_t *dilations,
                            const int64_t *pads, const int64_t *output_padding,
                            const int64_t *output_shape, const int64_t *kernel_shape,
                            int64_t group, const int64_t *points, int64_t npts, double *out,
                            char *err, int errlen)
{
    or_geom g;
    int rc;
    int64_t in_plane, taps, q;
    int bad = 0;
    rc = or_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, output_padding,
                    output_shape, kernel_shape, group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    in_plane = or_prod(g.L, nsp);
    taps = or_prod(g.K, nsp);

#pragma omp parallel for schedule(dynamic, 16)
    for (q = 0; q < npts; q++) {
        const int64_t *pt = points + q * (nsp + 2);
        int64_t n = pt[0], m = pt[1];
        int64_t grp, mm, cc;
        /* per axis: the input coordinates i and taps k with i*s - b + k*d == o */
        int64_t pi[3][64], pk[3][64], np_[3];
        int a, ok = 1;
        double acc;
        if (n < 0 || n >= g.N || m < 0 || m >= g.M)
            ok = 0;
        for (a = 0; ok && a < nsp; a++) {
            int64_t o = pt[2 + a], i, k;
            if (o < 0 || o >= g.O[a]) {
                ok = 0;
                break;
            }
            np_[a] = 0;
            for (i = 0; i < g.L[a]; i++)
                for (k = 0; k < g.K[a]; k++)
                    if (i * g.s[a] - g.b[a] + k * g.d[a] == o) {
                        if (np_[a] >= 64) {
                            ok = 0;
                            break;
                        }
                        pi[a][np_[a]] = i;
                        pk[a][np_[a]] = k;
                        np_[a]++;
                    }
        }
        if (!ok) {
#pragma omp atomic write
            bad = 1;
            out[q] = 0.0;
            continue;
        }
        grp = m / g.Mg;
        mm = m % g.Mg;
        acc = bias ? bias[m] : 0.0;
        for (cc = 0; cc < g.Cg; cc++) {
            int64_t c = grp * g.Cg + cc;
            const double *xp = x + (n * g.C + c) * in_plane;
            const double *wp = w + (c * g.Mg + mm) * taps;
            int64_t sel[3] = {0, 0, 0};
            int empty = 0;
            for (a = 0; a < nsp; a++)
                if (np_[a] == 0)
                    empty = 1;
            /* lexicographic walk over the per-axis pair lists = ascending i */
            while (!empty) {
                int64_t iflat = 0, kflat = 0;
                for (a = 0; a < nsp; a++) {
                    iflat = iflat * g.L[a] + pi[a][sel[a]];
                    kflat = kflat * g.K[a] + pk[a][sel[a]];
                }
                acc += xp[iflat] * wp[kflat];
                for (a = nsp - 1; a >= 0; a--) {
                    if (++sel[a] < np_[a])
                        break;
                    sel[a] = 0;
                }
                if (a < 0)
                    break;
            }
        }
        out[q] = acc;
    }
    if (bad)
        return or_fail(err, errlen, "a requested point lies outside Y (or has > 64 taps per axis)");
    return OR_OK;
}

/* ------------------------------------------------------------------------------------
 * Forward convolution (ONNX Conv), the adjoint of the transposed convolution with the
 * same W.  Attributes follow the webgpu-kernels "ai.onnx.QLinearConv" README (its
 * Attributes table is that of a convolution): auto_pad NOTSET / SAME_UPPER /
 * SAME_LOWER / VALID with SAME giving O = ceil(L / s), pads in ONNX order, strides,
 * dilations, group, kernel_shape; W is (M, C/group, k1..kn) (its Inputs table).
 *
 * Definition: Y[n, m, o] = bias[m] + sum over c of m's group and taps k of
 *     X[n, c, o*s - b + k*d] * W[m, c', k],   X = 0 outside [0, L) on each axis.
 * Readings (the pages print no output-size formula): the outputs are the window
 * positions that fit inside the padded input, O = floor((L + b + e - d(K-1) - 1)/s) + 1
 * (0 when no window fits); SAME's total pad is max(0, (O-1)s + d(K-1) + 1 - L), the
 * odd extra at the end (UPPER) or the beginning (LOWER); pads together with an
 * auto_pad other than NOTSET, negative pads and non-positive strides or dilations are
 * errors.
 * ---------------------------------------------------------------------------------- */
typedef struct {
    int nsp;
    int64_t N, C, M, group, Cg, Mg;
    int64_t L[3], K[3], s[3], d[3], b[3], e[3], O[3];
} or_cgeom;

static int or_conv_resolve(int nsp, const int64_t *xs, const int64_t *ws, int auto_pad,
                           const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                           const int64_t *kernel_shape, int64_t group, or_cgeom *g, char *err,
                           int errlen)
{
    int a;
    if (nsp < 1 || nsp > 3)
        return or_fail(err, errlen, "spatial rank must be 1, 2 or 3");
    if (auto_pad < OR_NOTSET || auto_pad > OR_VALID)
        return or_fail(err, errlen, "unknown auto_pad");
    if (pads && auto_pad != OR_NOTSET)
        return or_fail(err, errlen, "pads cannot be combined with an automatic padding mode");
    if (group < 1)
        return or_fail(err, errlen, "group must be >= 1");
    memset(g, 0, sizeof(*g));
    g->nsp = nsp;
    g->N = xs[0];
    g->C = xs[1];
    g->M = ws[0];
    g->group = group;
    if (g->N < 0 || g->C < 0 || g->M < 0 || ws[1] < 0)
        return or_fail(err, errlen, "negative dimension");
    if (g->C % group != 0 || g->M % group != 0)
        return or_fail(err, errlen, "C and M must be multiples of group");
    g->Cg = g->C / group;
    g->Mg = g->M / group;
    if (ws[1] != g->Cg)
        return or_fail(err, errlen, "W.shape[1] must equal C / group");
    for (a = 0; a < nsp; a++) {
        int64_t L = xs[2 + a], K = ws[2 + a], s = strides ? strides[a] : 1, d = dilations ? dilations[a] : 1;
        int64_t b = 0, e = 0, num;
        if (L < 0 || K < 1)
            return or_fail(err, errlen, "bad spatial size or kernel size");
        if (kernel_shape && kernel_shape[a] != K)
            return or_fail(err, errlen, "kernel_shape does not match W");
        if (s < 1 || d < 1)
            return or_fail(err, errlen, "strides and dilations must be >= 1");
        if (auto_pad == OR_NOTSET && pads) {
            b = pads[a];
            e = pads[nsp + a];
            if (b < 0 || e < 0)
                return or_fail(err, errlen, "pads must be >= 0");
        } else if (auto_pad == OR_SAME_UPPER || auto_pad == OR_SAME_LOWER) {
            int64_t O = (L + s - 1) / s, tot = (O - 1) * s + d * (K - 1) + 1 - L;
            if (tot < 0)
                tot = 0;
            if (auto_pad == OR_SAME_UPPER) {
                b = tot / 2;
                e = tot - b;
            } else {
                e = tot / 2;
                b = tot - e;
            }
        }
        num = L + b + e - d * (K - 1) - 1;
        g->L[a] = L;
        g->K[a] = K;
        g->s[a] = s;
        g->d[a] = d;
        g->b[a] = b;
        g->e[a] = e;
        g->O[a] = num >= 0 ? num / s + 1 : 0;
    }
    return OR_OK;
}

int oracle_conv_output_shape(int nsp, const int64_t *x_shape, const int64_t *w_shape, int auto_pad,
                             const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                             const int64_t *kernel_shape, int64_t group, int64_t *y_shape,
                             int64_t *pads_out, char *err, int errlen)
{
    or_cgeom g;
    int a, rc = or_conv_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, kernel_shape,
                                group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    y_shape[0] = g.N;
    y_shape[1] = g.M;
    for (a = 0; a < nsp; a++) {
        y_shape[2 + a] = g.O[a];
        if (pads_out) {
            pads_out[a] = g.b[a];
            pads_out[nsp + a] = g.e[a];
        }
    }
    return OR_OK;
}

/* Whole output by the gather definition (NCHW order); threads split the (n, m) planes,
 * and each output sums its group's channels c, then taps k, ascending. */
int oracle_conv_f64(int nsp, const int64_t *x_shape, const double *x, const int64_t *w_shape,
                    const double *w, const double *bias, int auto_pad, const int64_t *strides,
                    const int64_t *dilations, const int64_t *pads, const int64_t *kernel_shape,
                    int64_t group, double *y, int64_t y_len, char *err, int errlen)
{
    or_cgeom g;
    int64_t in_plane, out_plane, taps, plane;
    int rc = or_conv_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, kernel_shape,
                             group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    in_plane = or_prod(g.L, nsp);
    out_plane = or_prod(g.O, nsp);
    taps = or_prod(g.K, nsp);
    if (y_len != g.N * g.M * out_plane)
        return or_fail(err, errlen, "y buffer length does not match the resolved output");
#pragma omp parallel for schedule(dynamic, 1)
    for (plane = 0; plane < g.N * g.M; plane++) {
        int64_t n = plane / g.M, m = plane % g.M, grp = m / g.Mg;
        double *yp = y + plane * out_plane;
        int64_t p, cc, kk;
        int a;
        for (p = 0; p < out_plane; p++) {
            int64_t ocoord[3];
            double acc = bias ? bias[m] : 0.0;
            or_decode(p, g.O, nsp, ocoord);
            for (cc = 0; cc < g.Cg; cc++) {
                const double *xp = x + (n * g.C + grp * g.Cg + cc) * in_plane;
                const double *wp = w + (m * g.Cg + cc) * taps;
                for (kk = 0; kk < taps; kk++) {
                    int64_t kc[3], flat = 0;
                    int inside = 1;
                    or_decode(kk, g.K, nsp, kc);
                    for (a = 0; a < nsp; a++) {
                        int64_t i = ocoord[a] * g.s[a] - g.b[a] + kc[a] * g.d[a];
                        if (i < 0 || i >= g.L[a]) {
                            inside = 0;
                            break;
                        }
                        flat = flat * g.L[a] + i;
                    }
                    if (inside)
                        acc += xp[flat] * wp[kk];
                }
            }
            yp[p] = acc;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------------------
 * Quantized transposed convolution with the QLinear scale / zero-point scheme of the
 * webgpu-kernels "ai.onnx.QLinearConv" README (Description and Inputs table): x and y
 * are quantized per tensor (scale, zero point), w per tensor or per output channel
 * (w_scale and w_zero_point of length 1 or M), and the optional int32 bias carries scale
 * x_scale * w_scale and zero point 0.  The pages describe the scheme for the forward
 * convolution; here it is carried over to the transposed convolution unchanged.
 *
 * Definition used: the integer sum of the scatter form (the same (c, i, k) pairs as
 * oracle_convtranspose_f64) over zero-point-shifted operands,
 *     acc[n, m, o] = B[m] + sum (x[n, c, i] - x_zp) * (w[c, m', k] - w_zp[m]),
 * computed exactly (int64), then
 *     y = saturate(round_half_even(float(acc32) * mult[m]) + y_zp),
 *     mult[m] = float(float(x_scale * w_scale[m]) / y_scale),
 * where acc32 is acc reduced modulo 2^32 to int32 (the accumulator type of the bias)
 * and every floating-point step is one IEEE float32 operation.  Readings where the
 * pages are silent: the float32 order of the requantization above, round half to even,
 * saturation to [y_lo, y_hi] (0..255 for uint8, -128..127 for int8).
 *
 * x and w arrive widened to int32 (their uint8 / int8 values), NCHW order.  acc_out
 * (nullable) receives the exact sums; y_out the quantized outputs (as int32 values).
 * ---------------------------------------------------------------------------------- */
static float or_requant_mult(float x_scale, float w_scale, float y_scale)
{
    volatile float xw = x_scale * w_scale; /* one float32 product, rounded */
    volatile float mult = xw / y_scale;    /* one float32 quotient, rounded */
    return mult;
}

static int32_t or_requantize(int64_t acc, float mult, int32_t y_zp, int32_t y_lo, int32_t y_hi)
{
    int32_t acc32 = (int32_t)(uint32_t)(uint64_t)acc; /* modulo 2^32 */
    volatile float v = (float)acc32 * mult;
    float r = rintf(v); /* default rounding mode: to nearest, ties to even */
    double q = (double)r + (double)y_zp;
    if (q < (double)y_lo)
        return y_lo;
    if (q > (double)y_hi)
        return y_hi;
    return (int32_t)q;
}

int oracle_qconvtranspose(int nsp, const int64_t *x_shape, const int32_t *x, int32_t x_zp, float x_scale,
                          const int64_t *w_shape, const int32_t *w, const int32_t *w_zp, const float *w_scale,
                          int64_t wq_len, const int32_t *bias, float y_scale, int32_t y_zp, int32_t y_lo,
                          int32_t y_hi, int auto_pad, const int64_t *strides, const int64_t *dilations,
                          const int64_t *pads, const int64_t *output_padding, const int64_t *output_shape,
                          const int64_t *kernel_shape, int64_t group, int64_t *acc_out, int32_t *y_out,
                          int64_t y_len, char *err, int errlen)
{
    or_geom g;
    int rc;
    int64_t in_plane, out_plane, taps, t, plane;
    int64_t *tap_coord;
    int oom = 0;
    rc = or_resolve(nsp, x_shape, w_shape, auto_pad, strides, dilations, pads, output_padding,
                    output_shape, kernel_shape, group, &g, err, errlen);
    if (rc != OR_OK)
        return rc;
    if (wq_len != 1 && wq_len != g.M)
        return or_fail(err, errlen, "w_scale / w_zero_point must have length 1 or M");
    if (y_lo > y_hi)
        return or_fail(err, errlen, "empty output range");
    in_plane = or_prod(g.L, nsp);
    out_plane = or_prod(g.O, nsp);
    taps = or_prod(g.K, nsp);
    if (y_len != g.N * g.M * out_plane)
        return or_fail(err, errlen, "y buffer length does not match the resolved output");
    if (g.N * g.M * out_plane == 0)
        return OR_OK;

    tap_coord = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)(taps > 0 ? taps : 1));
    if (!tap_coord)
        return or_fail(err, errlen, "out of host memory");
    for (t = 0; t < taps; t++)
        or_decode(t, g.K, nsp, tap_coord + 3 * t);

#pragma omp parallel for schedule(dynamic, 1)
    for (plane = 0; plane < g.N * g.M; plane++) {
        int64_t n = plane / g.M, m = plane % g.M;
        int64_t grp = m / g.Mg, mm = m % g.Mg;
        int64_t q = wq_len == 1 ? 0 : m;
        int64_t *acc = (int64_t *)malloc(sizeof(int64_t) * (size_t)out_plane);
        float mult = or_requant_mult(x_scale, w_scale[q], y_scale);
        int64_t p, cc, ii, kk;
        int a;
        if (!acc) {
            /* reported after the loop as an error (no plane of y can be trusted then) */
#pragma omp atomic write
            oom = 1;
            continue;
        }
        for (p = 0; p < out_plane; p++)
            acc[p] = bias ? bias[m] : 0;
        for (cc = 0; cc < g.Cg; cc++) {
            int64_t c = grp * g.Cg + cc;
            const int32_t *xp = x + (n * g.C + c) * in_plane;
            const int32_t *wp = w + (c * g.Mg + mm) * taps;
            for (ii = 0; ii < in_plane; ii++) {
                int64_t icoord[3];
                int64_t xv = (int64_t)xp[ii] - x_zp;
                or_decode(ii, g.L, nsp, icoord);
                for (kk = 0; kk < taps; kk++) {
                    const int64_t *kc = tap_coord + 3 * kk;
                    int64_t flat = 0;
                    int inside = 1;
                    for (a = 0; a < nsp; a++) {
                        int64_t o = icoord[a] * g.s[a] - g.b[a] + kc[a] * g.d[a];
                        if (o < 0 || o >= g.O[a]) {
                            inside = 0;
                            break;
                        }
                        flat = flat * g.O[a] + o;
                    }
                    if (inside)
                        acc[flat] += xv * ((int64_t)wp[kk] - w_zp[q]);
                }
            }
        }
        for (p = 0; p < out_plane; p++) {
            if (acc_out)
                acc_out[plane * out_plane + p] = acc[p];
            y_out[plane * out_plane + p] = or_requantize(acc[p], mult, y_zp, y_lo, y_hi);
        }
        free(acc);
    }
    free(tap_coord);
    if (oom)
        return or_fail(err, errlen, "out of host memory");
    return OR_OK;
}

/* The requantization step alone on given accumulators (acc of length n, channel index
 * ch[i] into mult inputs), for pinning it against values fixed by its definition. */
int oracle_requantize(const int64_t *acc, int64_t n, float x_scale, const float *w_scale, const int64_t *ch,
                      float y_scale, int32_t y_zp, int32_t y_lo, int32_t y_hi, int32_t *y_out)
{
    int64_t i;
    for (i = 0; i < n; i++)
        y_out[i] = or_requantize(acc[i], or_requant_mult(x_scale, w_scale[ch[i]], y_scale), y_zp, y_lo, y_hi);
    return OR_OK;
}
