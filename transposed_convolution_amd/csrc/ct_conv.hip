// ct_conv.hip -- the forward convolution that is the adjoint of the transposed
// convolution with the same W (ONNX Conv; attributes as in the webgpu-kernels
// "ai.onnx.QLinearConv" README, Attributes table; W is (M, C/group, k1..kn) as in its
// Inputs table, which is the transposed convolution's (C, M/group, k..) read the other
// way round).
//
//   Y[n, m, o] = bias[m] + sum over c of m's group, taps k of X[n, c, o*s - b + k*d] W[m, c', k]
//
// with X = 0 outside [0, L).  Output size: the window positions that fit inside the
// padded input, O = floor((L + b + e - d(K-1) - 1) / s) + 1 (0 when none fits); SAME
// keeps ceil(L / s) outputs with the odd extra pad at the end (UPPER) or the beginning
// (LOWER).  With the transposed convolution's strides, dilations and begin pads and end
// pads e - output_padding this is its adjoint: <ConvT_W(x), y> = <x, Conv_W(y)>.
//
// Paths:
//   * stride 1 on every axis: the same correlation is a stride-1 transposed convolution
//     with W re-laid out as (C, M/group, k) and its taps reversed, begin pads
//     d(K-1) - b and end pads d(K-1) - e, so it runs on the MFMA implicit GEMM;
//   * stride s > 1 with dilation 1: split every tap k = s*k' + rho; input phase rho of
//     the zero-padded input, xs_rho[j] = X[s*j + rho - b], is read at j = o + k', so
//       Y[o] = sum over rho, k' of xs_rho[o + k'] W[s*k' + rho]
//     is a stride-1 correlation over s^n times the channels with ceil(K/s) taps (the
//     input phases become channels, "space to depth"); it runs on the path above;
//   * otherwise (and wherever the MFMA kernel does not serve the shape): a gather
//     kernel, one thread per output element, float32 accumulation.
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>

#include "ct_internal.hpp"

namespace ct {
namespace {

// Resolved forward-convolution geometry, carried on 3 axes like Geom (a rank-n problem
// puts its axes last; the leading axes have L = K = s = d = O = 1 and no pads).
struct CGeom {
    int nsp = 0;
    int64_t N = 0, C = 0, M = 0, G = 1, Cg = 0, Mg = 0;
    int64_t L[kAxes], K[kAxes], s[kAxes], d[kAxes], b[kAxes], e[kAxes], O[kAxes];
    int64_t in_pixels() const { return L[0] * L[1] * L[2]; }
    int64_t out_pixels() const { return O[0] * O[1] * O[2]; }
    int64_t taps() const { return K[0] * K[1] * K[2]; }
    int64_t y_elems() const { return N * M * out_pixels(); }
};

ct_status resolve_conv(int nsp, const int64_t *xs, const int64_t *ws, const Attrs &at, CGeom *g,
                       std::string *err)
{
    auto bad = [&](const std::string &m) {
        *err = m;
        return CT_EINVAL;
    };
    if (nsp < 1 || nsp > kAxes) return bad("spatial rank must be 1, 2 or 3");
    if (!xs || !ws) return bad("x_shape and w_shape are required");
    if (at.auto_pad != CT_NOTSET && at.auto_pad != CT_SAME_UPPER && at.auto_pad != CT_SAME_LOWER &&
        at.auto_pad != CT_VALID)
        return bad("auto_pad must be NOTSET, SAME_UPPER, SAME_LOWER or VALID");
    if (at.output_padding || at.output_shape) return bad("output_padding and output_shape are not Conv attributes");
    for (int a = 0; a < nsp + 2; ++a)
        if (xs[a] < 0 || ws[a] < 0) return bad("dimensions must be >= 0");
    if (at.group < 1) return bad("group must be >= 1");
    if (xs[1] % at.group != 0 || ws[0] % at.group != 0) return bad("C and M must be multiples of group");
    if (ws[1] != xs[1] / at.group) return bad("W.shape[1] must equal C / group");
    if (at.pads && at.auto_pad != CT_NOTSET) return bad("pads cannot be combined with auto_pad");
    g->nsp = nsp;
    g->N = xs[0];
    g->C = xs[1];
    g->M = ws[0];
    g->G = at.group;
    g->Cg = xs[1] / at.group;
    g->Mg = ws[0] / at.group;
    const int lead = kAxes - nsp;
    for (int t = 0; t < lead; ++t) {
        g->L[t] = g->K[t] = g->s[t] = g->d[t] = g->O[t] = 1;
        g->b[t] = g->e[t] = 0;
    }
    for (int a = 0; a < nsp; ++a) {
        const int t = lead + a;
        const int64_t L = xs[2 + a], K = ws[2 + a];
        const int64_t s = at.strides ? at.strides[a] : 1;
        const int64_t d = at.dilations ? at.dilations[a] : 1;
        if (K < 1) return bad("W spatial dimensions must be >= 1");
        if (at.kernel_shape && at.kernel_shape[a] != K)
            return bad("kernel_shape does not match W's spatial dimensions");
        if (s < 1 || d < 1) return bad("strides and dilations must be >= 1");
        int64_t b = 0, e = 0;
        if (at.auto_pad == CT_SAME_UPPER || at.auto_pad == CT_SAME_LOWER) {
            const int64_t O = (L + s - 1) / s;
            int64_t tot = (O - 1) * s + d * (K - 1) + 1 - L;
            if (tot < 0) tot = 0;
            if (at.auto_pad == CT_SAME_UPPER) {
                b = tot / 2;
                e = tot - b;
            } else {
                e = tot / 2;
                b = tot - e;
            }
        } else if (at.auto_pad == CT_NOTSET && at.pads) {
            b = at.pads[a];
            e = at.pads[nsp + a];
            if (b < 0 || e < 0) return bad("pads must be >= 0");
        }
        const int64_t num = L + b + e - d * (K - 1) - 1;
        const int64_t O = num >= 0 ? num / s + 1 : 0;
        if (L > INT32_MAX || O > INT32_MAX || K > INT32_MAX || s > INT32_MAX || d > INT32_MAX || b > INT32_MAX ||
            e > INT32_MAX)
            return bad("spatial sizes and attributes must fit in 32 bits");
        g->L[t] = L;
        g->K[t] = K;
        g->s[t] = s;
        g->d[t] = d;
        g->b[t] = b;
        g->e[t] = e;
        g->O[t] = O;
    }
    if (g->C > INT32_MAX || g->M > INT32_MAX || g->N > INT32_MAX)
        return bad("batch and channel counts must fit in 32 bits");
    return CT_OK;
}

struct ConvArgs {
    int64_t total;  // elements of Y
    int C, M, Cg, Mg, has_bias;
    int L[kAxes], K[kAxes], s[kAxes], d[kAxes], b[kAxes], O[kAxes];
};

// One thread per output element: the window's taps that land inside X, the group's
// input channels, float32 accumulation, one rounding into Y.
template <typename T, bool CL>
__global__ __launch_bounds__(256) void conv_direct_kernel(const T *__restrict__ x, const T *__restrict__ w,
                                                          const T *__restrict__ bias, T *__restrict__ y, ConvArgs p)
{
    const int64_t in_pix = int64_t(p.L[0]) * p.L[1] * p.L[2];
    const int taps = p.K[0] * p.K[1] * p.K[2];
    const int64_t step = int64_t(gridDim.x) * blockDim.x;
    for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < p.total; idx += step) {
        int64_t t = idx;
        int m, n, o0, o1, o2;
        if (CL) {  // y stored (N, O0, O1, O2, M)
            m = int(t % p.M);
            t /= p.M;
            o2 = int(t % p.O[2]);
            t /= p.O[2];
            o1 = int(t % p.O[1]);
            t /= p.O[1];
            o0 = int(t % p.O[0]);
            n = int(t / p.O[0]);
        } else {  // y stored (N, M, O0, O1, O2)
            o2 = int(t % p.O[2]);
            t /= p.O[2];
            o1 = int(t % p.O[1]);
            t /= p.O[1];
            o0 = int(t % p.O[0]);
            t /= p.O[0];
            m = int(t % p.M);
            n = int(t / p.M);
        }
        const int c0 = (m / p.Mg) * p.Cg;
        float acc = 0.0f;
        for (int k0 = 0; k0 < p.K[0]; ++k0) {
            const int i0 = o0 * p.s[0] - p.b[0] + k0 * p.d[0];
            if (i0 < 0 || i0 >= p.L[0]) continue;
            for (int k1 = 0; k1 < p.K[1]; ++k1) {
                const int i1 = o1 * p.s[1] - p.b[1] + k1 * p.d[1];
                if (i1 < 0 || i1 >= p.L[1]) continue;
                for (int k2 = 0; k2 < p.K[2]; ++k2) {
                    const int i2 = o2 * p.s[2] - p.b[2] + k2 * p.d[2];
                    if (i2 < 0 || i2 >= p.L[2]) continue;
                    const int64_t ipix = (int64_t(i0) * p.L[1] + i1) * p.L[2] + i2;
                    const int kflat = (k0 * p.K[1] + k1) * p.K[2] + k2;
                    const T *xp = CL ? x + (int64_t(n) * in_pix + ipix) * p.C + c0
                                     : x + (int64_t(n) * p.C + c0) * in_pix + ipix;
                    const int64_t xstep = CL ? 1 : in_pix;
                    const T *wp = w + int64_t(m) * p.Cg * taps + kflat;
                    for (int cc = 0; cc < p.Cg; ++cc) acc += float(xp[cc * xstep]) * float(wp[cc * taps]);
                }
            }
        }
        if (p.has_bias) acc += float(bias[m]);
        y[idx] = T(acc);
    }
}

template <typename T>
ct_status launch_direct_t(const CGeom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                          hipStream_t st, std::string *err)
{
    ConvArgs p;
    p.total = g.y_elems();
    p.C = int(g.C);
    p.M = int(g.M);
    p.Cg = int(g.Cg);
    p.Mg = int(g.Mg);
    p.has_bias = bias != nullptr;
    for (int a = 0; a < kAxes; ++a) {
        p.L[a] = int(g.L[a]);
        p.K[a] = int(g.K[a]);
        p.s[a] = int(g.s[a]);
        p.d[a] = int(g.d[a]);
        p.b[a] = int(g.b[a]);
        p.O[a] = int(g.O[a]);
    }
    const int block = 256;
    int64_t blocks = (p.total + block - 1) / block;
    if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride loop covers the rest
    const T *xt = static_cast<const T *>(x);
    const T *wt = static_cast<const T *>(w);
    const T *bt = static_cast<const T *>(bias);
    T *yt = static_cast<T *>(y);
    mark_before(st);
    if (cl)
        hipLaunchKernelGGL((conv_direct_kernel<T, true>), dim3(unsigned(blocks)), dim3(block), 0, st, xt, wt, bt,
                           yt, p);
    else
        hipLaunchKernelGGL((conv_direct_kernel<T, false>), dim3(unsigned(blocks)), dim3(block), 0, st, xt, wt, bt,
                           yt, p);
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("convolution kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

// Stride-1 path: the transposed-convolution geometry of the same correlation.
Geom stride1_as_transposed(const CGeom &c)
{
    Geom g;
    g.nsp = c.nsp;
    g.N = c.N;
    g.C = c.C;
    g.M = c.M;
    g.G = c.G;
    g.Cg = c.Cg;
    g.Mg = c.Mg;
    for (int a = 0; a < kAxes; ++a) {
        g.L[a] = c.L[a];
        g.K[a] = c.K[a];
        g.s[a] = 1;
        g.d[a] = c.d[a];
        g.b[a] = c.d[a] * (c.K[a] - 1) - c.b[a];  // may be negative: a crop
        g.e[a] = c.d[a] * (c.K[a] - 1) - c.e[a];
        g.op[a] = 0;
        g.O[a] = c.O[a];
    }
    return g;
}

// W (M, C/group, k) -> W' (C, M/group, k reversed): W'[g*Cg + c][m'][K-1-k] = W[g*Mg + m'][c][k].
template <typename T>
__global__ __launch_bounds__(256) void conv_w_to_transposed(const T *__restrict__ w, T *__restrict__ wt, int64_t total,
                                                            int Cg, int Mg, int K0, int K1, int K2)
{
    const int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (u >= total) return;
    const int taps = K0 * K1 * K2;
    const int k = int(u % taps);
    int64_t r = u / taps;
    const int c = int(r % Cg);
    r /= Cg;
    const int m = int(r);  // global output channel g*Mg + m'
    const int g = m / Mg, mm = m - g * Mg;
    const int k2 = k % K2, k1 = (k / K2) % K1, k0 = k / (K1 * K2);
    const int kr = ((K0 - 1 - k0) * K1 + (K1 - 1 - k1)) * K2 + (K2 - 1 - k2);
    wt[((int64_t(g) * Cg + c) * Mg + mm) * taps + kr] = w[u];
}

ct_status launch_stride1(const CGeom &c, ct_dtype dt, bool cl, const void *x, const void *w, const void *bias,
                         void *y, hipStream_t st, std::string *err)
{
    const Geom g = stride1_as_transposed(c);
    if (dt == CT_FLOAT16)  // the weight re-layout reads the convolution's W directly
        return launch_igemm(g, dt, cl, x, w, bias, y, Act{}, nullptr, 0, st, err, true);
    const size_t esz = 4;
    const int64_t wn = c.M * c.Cg * c.taps();
    const size_t ws = igemm_workspace_bytes(g, dt);
    const size_t wbytes = (size_t(wn) * esz + 255) / 256 * 256;
    void *buf = nullptr;
    hipError_t e = scratch_malloc(&buf, wbytes + ws, st);
    if (e != hipSuccess) {
        *err = std::string("scratch allocation failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    const unsigned blocks = unsigned((wn + 255) / 256);
    hipLaunchKernelGGL(conv_w_to_transposed<float>, dim3(blocks), dim3(256), 0, st, static_cast<const float *>(w),
                       static_cast<float *>(buf), wn, int(c.Cg), int(c.Mg), int(c.K[0]), int(c.K[1]), int(c.K[2]));
    ct_status s = launch_igemm(g, dt, cl, x, buf, bias, y, Act{}, ws ? static_cast<char *>(buf) + wbytes : nullptr,
                               ws, st, err);
    e = hipFreeAsync(buf, st);
    if (s == CT_OK && e != hipSuccess) {
        *err = std::string("scratch release failed: ") + hipGetErrorString(e);
        s = CT_EDEVICE;
    }
    return s;
}

// The stride-1 problem a strided, dilation-1 convolution becomes when its input phases
// are taken as channels: C' = C * P (P = product of the strides), K' = ceil(K / s),
// L' = O + K' - 1, no pads.  even_rows: the innermost L' is rounded up to an even size
// (the channels-first MFMA loads take whole 4-byte column pairs) and the extra column
// cropped by an end pad of -1.
CGeom s2d_geom(const CGeom &c, bool even_rows)
{
    CGeom q = c;
    int64_t P = 1;
    for (int a = 0; a < kAxes; ++a) P *= c.s[a];
    q.C = c.C * P;
    q.Cg = c.Cg * P;
    for (int a = 0; a < kAxes; ++a) {
        q.K[a] = (c.K[a] + c.s[a] - 1) / c.s[a];
        q.L[a] = c.O[a] + q.K[a] - 1;
        q.s[a] = 1;
        q.d[a] = 1;
        q.b[a] = q.e[a] = 0;
    }
    if (even_rows && q.L[kAxes - 1] % 2 != 0) {
        q.L[kAxes - 1] += 1;
        q.e[kAxes - 1] = -1;
    }
    return q;
}

struct S2dArgs {
    int64_t total;  // elements of xs
    int C, P;
    int L[kAxes], s[kAxes], b[kAxes], J[kAxes];
};

// xs[n][c * P + rho][j] = X[n][c][s * j + rho - b] (0 outside X); rho is the flattened
// per-axis phase (rho0 * s1 + rho1) * s2 + rho2.  Channels-last tensors keep their
// layout: xs[n][j][c * P + rho].  One thread makes 8 consecutive elements of xs (along
// the innermost axis, or along the channels for channels-last); 32-bit indices (the
// plan keeps xs below 2^31 elements).
// Eight consecutive values as 16-byte stores (dst 16-byte aligned), built from the values
// themselves: a reinterpreted local array would be placed in scratch memory.
template <typename T>
__device__ __forceinline__ void store8(T *dst, const T (&v)[8])
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(T) == 2) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = unsigned(__builtin_bit_cast(unsigned short, v[2 * k])) |
                   (unsigned(__builtin_bit_cast(unsigned short, v[2 * k + 1])) << 16);
        *reinterpret_cast<u32x4 *>(dst) = o;
    } else {
        static_assert(sizeof(T) == 4, "16- or 32-bit values");
        const u32x4 o0 = {__builtin_bit_cast(unsigned, v[0]), __builtin_bit_cast(unsigned, v[1]),
                          __builtin_bit_cast(unsigned, v[2]), __builtin_bit_cast(unsigned, v[3])};
        const u32x4 o1 = {__builtin_bit_cast(unsigned, v[4]), __builtin_bit_cast(unsigned, v[5]),
                          __builtin_bit_cast(unsigned, v[6]), __builtin_bit_cast(unsigned, v[7])};
        reinterpret_cast<u32x4 *>(dst)[0] = o0;
        reinterpret_cast<u32x4 *>(dst)[1] = o1;
    }
}

template <typename T, bool CL>
__global__ __launch_bounds__(256) void s2d_kernel(const T *__restrict__ x, T *__restrict__ xs, S2dArgs p)
{
    const int Cp = p.C * p.P;
    const int inner = CL ? Cp : p.J[2];  // the run a thread's 8 elements lie in
    const int g8 = (inner + 7) / 8;
    const int rows = int(p.total / inner);
    const int u = int(blockIdx.x) * int(blockDim.x) + int(threadIdx.x);
    if (u >= rows * g8) return;
    int row = u / g8;
    const int e0 = (u - row * g8) * 8;
    const int in_pix = p.L[0] * p.L[1] * p.L[2];
    int n, cp = 0, j0, j1, j2 = 0;
    if (CL) {  // row = ((n * J0 + j0) * J1 + j1) * J2 + j2
        j2 = row % p.J[2];
        row /= p.J[2];
        j1 = row % p.J[1];
        row /= p.J[1];
        j0 = row % p.J[0];
        n = row / p.J[0];
    } else {   // row = ((n * Cp + cp) * J0 + j0) * J1 + j1
        j1 = row % p.J[1];
        row /= p.J[1];
        j0 = row % p.J[0];
        row /= p.J[0];
        cp = row % Cp;
        n = row / Cp;
    }
    T *const dst = xs + size_t(u / g8) * inner;
    // every load is issued unconditionally from a valid address and masked afterwards, so
    // the eight loads are in flight together (loads under bounds branches were waited for
    // one at a time).  An empty input (padding alone can still give a phase copy) has no
    // valid address: then nothing is loaded and the copy is zeros.
    T vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vals[e] = T(0);
    if (in_pix > 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = min(e0 + e, inner - 1);  // j2 (channels-first) or cp (channels-last)
        const int cpe = CL ? k : cp, j2e = CL ? j2 : k;
        const int c = cpe / p.P, rho = cpe - c * p.P;
        const int r2 = rho % p.s[2], r1 = (rho / p.s[2]) % p.s[1], r0 = rho / (p.s[2] * p.s[1]);
        const int i0 = p.s[0] * j0 + r0 - p.b[0], i1 = p.s[1] * j1 + r1 - p.b[1], i2 = p.s[2] * j2e + r2 - p.b[2];
        const bool ok = e0 + e < inner && i0 >= 0 && i0 < p.L[0] && i1 >= 0 && i1 < p.L[1] && i2 >= 0 && i2 < p.L[2];
        const int ipix = (i0 * p.L[1] + i1) * p.L[2] + i2;
        const size_t off = !ok ? 0 : CL ? (size_t(n) * in_pix + ipix) * p.C + c : (size_t(n) * p.C + c) * in_pix + ipix;
        const T v = x[off];
        vals[e] = ok ? v : T(0);
    }
    if (inner % 8 == 0) {
        // whole runs of 8 (the scratch copy is 256-byte aligned): one 16-byte store per
        // 16 bytes instead of one store per element
        store8(dst + e0, vals);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e0 + e < inner) dst[e0 + e] = vals[e];
    }
}

// W'[m][cc * P + rho][k'] = W[m][cc][s * k' + rho] (0 where s * k' + rho >= K).
template <typename T>
__global__ __launch_bounds__(256) void s2d_w_kernel(const T *__restrict__ w, T *__restrict__ wq, int64_t total,
                                                    int Cg, int P, S2dArgs p, int K0, int K1, int K2, int Q0, int Q1,
                                                    int Q2)
{
    // 8 consecutive outputs per thread (one 16-byte store per 16 bytes): the index is split
    // once and then advanced with carries, not divided per element
    const int64_t u0 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
    if (u0 >= total) return;
    const int qt = Q0 * Q1 * Q2, cgp = Cg * P;
    int kq = int(u0 % qt);
    const int64_t r = u0 / qt;
    int cp = int(r % cgp);
    int64_t m = r / cgp;
    T vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        {  // unconditional load from a valid address, masked afterwards (see s2d_kernel)
            const int cc = cp / P, rho = cp - cc * P;
            const int r2 = rho % p.s[2], r1 = (rho / p.s[2]) % p.s[1], r0 = rho / (p.s[2] * p.s[1]);
            const int q2 = kq % Q2, q1 = (kq / Q2) % Q1, q0 = kq / (Q1 * Q2);
            const int k0 = p.s[0] * q0 + r0, k1 = p.s[1] * q1 + r1, k2 = p.s[2] * q2 + r2;
            const bool ok = u0 + e < total && k0 < K0 && k1 < K1 && k2 < K2;
            const T v = w[ok ? ((m * Cg + cc) * K0 + k0) * K1 * K2 + int64_t(k1) * K2 + k2 : 0];
            vals[e] = ok ? v : T(0);
        }
        if (++kq == qt) {
            kq = 0;
            if (++cp == cgp) {
                cp = 0;
                ++m;
            }
        }
    }
    if (total % 8 == 0) {  // whole runs of 8 (the scratch copy is 256-byte aligned)
        store8(wq + u0, vals);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (u0 + e < total) wq[u0 + e] = vals[e];
    }
}

ct_status launch_s2d(const CGeom &c, ct_dtype dt, bool cl, const void *x, const void *w, const void *bias, void *y,
                     hipStream_t st, std::string *err)
{
    const CGeom q = s2d_geom(c, !cl);
    const size_t esz = dt == CT_FLOAT32 ? 4 : 2;
    S2dArgs p;
    p.C = int(c.C);
    p.P = int(q.C / c.C);
    for (int a = 0; a < kAxes; ++a) {
        p.L[a] = int(c.L[a]);
        p.s[a] = int(c.s[a]);
        p.b[a] = int(c.b[a]);
        p.J[a] = int(q.L[a]);
    }
    p.total = q.N * q.C * q.in_pixels();
    const int64_t wn = q.M * q.Cg * q.taps();
    const size_t xs_bytes = (size_t(p.total) * esz + 255) / 256 * 256;
    const size_t wq_bytes = (size_t(wn) * esz + 255) / 256 * 256;
    void *buf = nullptr;
    hipError_t e = scratch_malloc(&buf, xs_bytes + wq_bytes, st);
    if (e != hipSuccess) {
        *err = std::string("scratch allocation failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    void *xs = buf;
    void *wq = static_cast<char *>(buf) + xs_bytes;
    const int64_t inner = cl ? q.C : q.L[kAxes - 1];
    const int64_t threads = inner > 0 ? p.total / inner * ((inner + 7) / 8) : 0;
    const unsigned bx = unsigned((threads + 255) / 256), bw = unsigned((wn + 8 * 256 - 1) / (8 * 256));
    const int K0 = int(c.K[0]), K1 = int(c.K[1]), K2 = int(c.K[2]);
    const int Q0 = int(q.K[0]), Q1 = int(q.K[1]), Q2 = int(q.K[2]);
    if (dt == CT_FLOAT16) {
        using T = _Float16;
        if (p.total > 0) {
            if (cl) hipLaunchKernelGGL((s2d_kernel<T, true>), dim3(bx), dim3(256), 0, st, static_cast<const T *>(x), static_cast<T *>(xs), p);
            else hipLaunchKernelGGL((s2d_kernel<T, false>), dim3(bx), dim3(256), 0, st, static_cast<const T *>(x), static_cast<T *>(xs), p);
        }
        if (wn > 0)
            hipLaunchKernelGGL(s2d_w_kernel<T>, dim3(bw), dim3(256), 0, st, static_cast<const T *>(w), static_cast<T *>(wq),
                               wn, int(c.Cg), p.P, p, K0, K1, K2, Q0, Q1, Q2);
    } else {
        using T = float;
        if (p.total > 0) {
            if (cl) hipLaunchKernelGGL((s2d_kernel<T, true>), dim3(bx), dim3(256), 0, st, static_cast<const T *>(x), static_cast<T *>(xs), p);
            else hipLaunchKernelGGL((s2d_kernel<T, false>), dim3(bx), dim3(256), 0, st, static_cast<const T *>(x), static_cast<T *>(xs), p);
        }
        if (wn > 0)
            hipLaunchKernelGGL(s2d_w_kernel<T>, dim3(bw), dim3(256), 0, st, static_cast<const T *>(w), static_cast<T *>(wq),
                               wn, int(c.Cg), p.P, p, K0, K1, K2, Q0, Q1, Q2);
    }
    ct_status s = launch_stride1(q, dt, cl, xs, wq, bias, y, st, err);
    e = hipFreeAsync(buf, st);
    if (s == CT_OK && e != hipSuccess) {
        *err = std::string("scratch release failed: ") + hipGetErrorString(e);
        s = CT_EDEVICE;
    }
    return s;
}

bool is_aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ct_status conv_fail(ct_status st, const std::string &m)
{
    set_last_error(m);
    return st;
}

Attrs conv_attrs(ct_auto_pad auto_pad, const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                 const int64_t *kernel_shape, int64_t group)
{
    Attrs at;
    at.auto_pad = auto_pad;
    at.strides = strides;
    at.dilations = dilations;
    at.pads = pads;
    at.kernel_shape = kernel_shape;
    at.group = group;
    return at;
}

// Which path convolution_nd takes (CT_KERNEL_IGEMM: the MFMA path, stride 1 directly or
// a strided convolution through its input phases, *s2d).
ct_kernel conv_choose(const CGeom &c, ct_dtype dt, bool cl, const void *x, ct_kernel want, std::string *why,
                      bool *s2d)
{
    bool s1 = true, d1 = true;
    for (int a = 0; a < kAxes; ++a) {
        s1 = s1 && c.s[a] == 1;
        d1 = d1 && c.d[a] == 1;
    }
    bool fast = false;
    *s2d = false;
    if (s1) {
        fast = c.Cg >= 16 && c.Mg >= 16 && igemm_supports(stride1_as_transposed(c), dt, cl, x, why);
    } else if (d1 && c.out_pixels() > 0) {
        const CGeom q = s2d_geom(c, !cl);
        // the phase copy is 256-byte aligned scratch, so x's own alignment does not matter
        fast = q.N * q.C * q.in_pixels() < (int64_t(1) << 31) && c.N * c.C * c.in_pixels() < (int64_t(1) << 31) &&
               q.Cg >= 16 && c.Mg >= 16 &&
               igemm_supports(stride1_as_transposed(q), dt, cl, reinterpret_cast<const void *>(256), why);
        *s2d = fast;
    } else {
        *why = "strided convolutions with dilation > 1 run on the gather kernel";
    }
    if (want == CT_KERNEL_DIRECT) return CT_KERNEL_DIRECT;
    if (want == CT_KERNEL_IGEMM) return fast ? CT_KERNEL_IGEMM : CT_KERNEL_NONE;
    return fast ? CT_KERNEL_IGEMM : CT_KERNEL_DIRECT;
}

}  // namespace
}  // namespace ct

extern "C" {

ct_status convolution_output_shape(int nsp, const int64_t *x_shape, const int64_t *w_shape, ct_auto_pad auto_pad,
                            const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                            const int64_t *kernel_shape, int64_t group, int64_t *y_shape_out, int64_t *pads_out)
{
    ct::set_last_error(std::string());
    {
        ct::EnumArgs ea;
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return ct::conv_fail(es, ee);
    }
    if (!y_shape_out) return ct::conv_fail(CT_EINVAL, "y_shape_out is NULL");
    ct::CGeom g;
    std::string err;
    const ct_status st = ct::resolve_conv(nsp, x_shape, w_shape,
                                          ct::conv_attrs(auto_pad, strides, dilations, pads, kernel_shape, group),
                                          &g, &err);
    if (st != CT_OK) return ct::conv_fail(st, err);
    const int lead = ct::kAxes - nsp;
    y_shape_out[0] = g.N;
    y_shape_out[1] = g.M;
    for (int a = 0; a < nsp; ++a) {
        y_shape_out[2 + a] = g.O[lead + a];
        if (pads_out) {
            pads_out[a] = g.b[lead + a];
            pads_out[nsp + a] = g.e[lead + a];
        }
    }
    return CT_OK;
}

ct_status convolution_nd(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last, const void *x,
                         const int64_t *x_shape, const void *w, const int64_t *w_shape, const void *bias, void *y,
                         const int64_t *y_shape, ct_auto_pad auto_pad, const int64_t *strides,
                         const int64_t *dilations, const int64_t *pads, const int64_t *kernel_shape, int64_t group,
                         void *stream)
{
    ct::set_last_error(std::string());
    {
        ct::EnumArgs ea;
        ea.kernel = ct::enum_int(kernel);
        ea.dtype = ct::enum_int(dtype);
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return ct::conv_fail(es, ee);
    }
    if (dtype != CT_FLOAT32 && dtype != CT_FLOAT16)
        return ct::conv_fail(CT_EUNSUPPORTED, "dtype must be CT_FLOAT32 or CT_FLOAT16");
    if (channels_last != 0 && channels_last != 1) return ct::conv_fail(CT_EINVAL, "channels_last must be 0 or 1");
    if (kernel != CT_KERNEL_AUTO && kernel != CT_KERNEL_DIRECT && kernel != CT_KERNEL_IGEMM)
        return ct::conv_fail(CT_EINVAL, "kernel must be CT_KERNEL_AUTO, CT_KERNEL_DIRECT or CT_KERNEL_IGEMM");
    if (!y_shape) return ct::conv_fail(CT_EINVAL, "y_shape is NULL");
    ct::CGeom g;
    std::string err;
    ct_status st = ct::resolve_conv(nsp, x_shape, w_shape,
                                    ct::conv_attrs(auto_pad, strides, dilations, pads, kernel_shape, group), &g, &err);
    if (st != CT_OK) return ct::conv_fail(st, err);
    const int lead = ct::kAxes - nsp;
    bool same = y_shape[0] == g.N && y_shape[1] == g.M;
    for (int a = 0; a < nsp; ++a) same = same && y_shape[2 + a] == g.O[lead + a];
    if (!same) return ct::conv_fail(CT_ESHAPE, "y_shape differs from the resolved output shape");
    const size_t esz = dtype == CT_FLOAT32 ? 4 : 2;
    if (!ct::is_aligned(x, esz) || !ct::is_aligned(w, esz) || !ct::is_aligned(y, esz) || !ct::is_aligned(bias, esz))
        return ct::conv_fail(CT_EINVAL, "tensor pointers must be aligned to the element size");
    if (g.y_elems() == 0) return CT_OK;
    if (!y) return ct::conv_fail(CT_EINVAL, "y is NULL");
    if (g.N * g.C * g.in_pixels() > 0 && !x) return ct::conv_fail(CT_EINVAL, "x is NULL");
    if (g.M * g.Cg * g.taps() > 0 && !w) return ct::conv_fail(CT_EINVAL, "w is NULL");
    const bool cl = channels_last != 0;
    std::string why;
    bool s2d = false;
    const ct_kernel k = ct::conv_choose(g, dtype, cl, x, kernel, &why, &s2d);
    if (k == CT_KERNEL_NONE)
        return ct::conv_fail(CT_EUNSUPPORTED, "the implicit-GEMM path cannot serve this convolution" +
                                                  (why.empty() ? std::string() : ": " + why));
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (k == CT_KERNEL_IGEMM && s2d)
        st = ct::launch_s2d(g, dtype, cl, x, w, bias, y, hs, &err);
    else if (k == CT_KERNEL_IGEMM)
        st = ct::launch_stride1(g, dtype, cl, x, w, bias, y, hs, &err);
    else if (dtype == CT_FLOAT16)
        st = ct::launch_direct_t<_Float16>(g, cl, x, w, bias, y, hs, &err);
    else
        st = ct::launch_direct_t<float>(g, cl, x, w, bias, y, hs, &err);
    if (st != CT_OK) return ct::conv_fail(st, err);
    return CT_OK;
}

}  // extern "C"
