// ct_direct.hip -- the generic gather kernel: one thread per output element.
//
// It serves every rank (1..3, carried as 3 axes), stride, dilation, pad, group,
// layout and dtype, so it is the dispatcher's fallback and the degenerate-case path
// (no input channels or no input samples: every output is the bias).
//
// For an output position o the taps that reach it on axis a are the k with
// (o + b - k*d) a non-negative multiple of s whose input i = (o + b - k*d)/s lies in
// [0, L) -- the scatter rule of the transposed convolution (webgpu-kernels
// "ai.onnx.ConvTranspose" README, Description and Attributes) read from the output
// side, so no zero-inserted input is ever formed.  Accumulation is float32 for both
// float32 and float16 inputs; the result is rounded once into Y.
#include <hip/hip_runtime.h>

#include "ct_internal.hpp"

namespace ct {
namespace {

struct DirectArgs {
    int64_t total;  // elements of Y
    int N, C, M, Cg, Mg, has_bias;
    int L[kAxes], K[kAxes], s[kAxes], d[kAxes], b[kAxes], O[kAxes];
    Act act;  // output activation
};

template <typename T, bool CL>
__global__ __launch_bounds__(256) void direct_kernel(const T *__restrict__ x, const T *__restrict__ w,
                                                     const T *__restrict__ bias, T *__restrict__ y,
                                                     DirectArgs p)
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
        const int grp = m / p.Mg, mm = m - grp * p.Mg;
        const int c0 = grp * p.Cg;
        float acc = 0.0f;
        for (int k0 = 0; k0 < p.K[0]; ++k0) {
            const int t0 = o0 + p.b[0] - k0 * p.d[0];
            if (t0 < 0) break;  // decreases with k0
            if (t0 % p.s[0] != 0) continue;
            const int i0 = t0 / p.s[0];
            if (i0 >= p.L[0]) continue;
            for (int k1 = 0; k1 < p.K[1]; ++k1) {
                const int t1 = o1 + p.b[1] - k1 * p.d[1];
                if (t1 < 0) break;
                if (t1 % p.s[1] != 0) continue;
                const int i1 = t1 / p.s[1];
                if (i1 >= p.L[1]) continue;
                for (int k2 = 0; k2 < p.K[2]; ++k2) {
                    const int t2 = o2 + p.b[2] - k2 * p.d[2];
                    if (t2 < 0) break;
                    if (t2 % p.s[2] != 0) continue;
                    const int i2 = t2 / p.s[2];
                    if (i2 >= p.L[2]) continue;
                    const int64_t ipix = (int64_t(i0) * p.L[1] + i1) * p.L[2] + i2;
                    const int kflat = (k0 * p.K[1] + k1) * p.K[2] + k2;
                    const T *xp = CL ? x + (int64_t(n) * in_pix + ipix) * p.C + c0
                                     : x + (int64_t(n) * p.C + c0) * in_pix + ipix;
                    const int64_t xstep = CL ? 1 : in_pix;
                    const T *wp = w + (int64_t(c0) * p.Mg + mm) * taps + kflat;
                    const int64_t wstep = int64_t(p.Mg) * taps;
                    for (int cc = 0; cc < p.Cg; ++cc)
                        acc += float(xp[cc * xstep]) * float(wp[cc * wstep]);
                }
            }
        }
        if (p.has_bias) acc += float(bias[m]);
        y[idx] = T(p.act(acc));
    }
}

template <typename T>
ct_status launch_t(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                   const Act &act, hipStream_t st, std::string *err)
{
    DirectArgs p;
    p.act = act;
    p.total = g.y_elems();
    p.N = int(g.N);
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
        hipLaunchKernelGGL((direct_kernel<T, true>), dim3(unsigned(blocks)), dim3(block), 0, st, xt, wt,
                           bt, yt, p);
    else
        hipLaunchKernelGGL((direct_kernel<T, false>), dim3(unsigned(blocks)), dim3(block), 0, st, xt,
                           wt, bt, yt, p);
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("direct kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace

ct_status launch_direct(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w,
                        const void *bias, void *y, const Act &act, hipStream_t st, std::string *err)
{
    if (dt == CT_FLOAT16) return launch_t<_Float16>(g, cl, x, w, bias, y, act, st, err);
    return launch_t<float>(g, cl, x, w, bias, y, act, st, err);
}

}  // namespace ct
