// ct_qlinear.hip -- quantized transposed convolution with the QLinear scale / zero-point
// scheme (webgpu-kernels "ai.onnx.QLinearConv" README, Description and Inputs table):
// uint8 / int8 x and y quantized per tensor, w per tensor or per output channel, an
// optional int32 bias with scale x_scale * w_scale[m] and zero point 0.  The pages give
// the scheme for the forward convolution; it is applied here to the transposed one.
//
//   acc[n, m, o] = B[m] + sum over the scatter pairs (c, i, k) reaching o of
//                  (x[n, c, i] - x_zp) * (w[c, m', k] - w_zp[m])      (int32, modulo 2^32)
//   y[n, m, o]   = saturate(round_half_even(float(acc) * mult[m]) + y_zp)
//   mult[m]      = float(float(x_scale * w_scale[m]) / y_scale)
//
// Every floating-point step above is one IEEE float32 operation (the multiply and the
// correctly rounded divide the compiler emits for '/'; no contraction), so the
// quantized codes are reproducible bit for bit.
#include <hip/hip_runtime.h>

#include <cmath>

#include "ct_internal.hpp"

namespace ct {
namespace {

struct QDirectArgs {
    int64_t total;  // elements of Y
    int N, C, M, Cg, Mg, wq_per_channel, has_bias;
    int L[kAxes], K[kAxes], s[kAxes], d[kAxes], b[kAxes], O[kAxes];
    int x_zp, y_zp, y_lo, y_hi;
    float x_scale, y_scale;
};

// One thread per output element (the gather form of the scatter rule, as in the float
// gather kernel); integer products of zero-point-shifted operands summed in uint32
// (two's complement wrap-around, i.e. modulo 2^32).
template <typename XT, typename WT, typename YT, bool CL>
__global__ __launch_bounds__(256) void qdirect_kernel(const XT *__restrict__ x, const WT *__restrict__ w,
                                                      const float *__restrict__ w_scale,
                                                      const WT *__restrict__ w_zp,
                                                      const int *__restrict__ bias, YT *__restrict__ y,
                                                      QDirectArgs p)
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
        const int q = p.wq_per_channel ? m : 0;
        const int wz = int(w_zp[q]);
        unsigned acc = p.has_bias ? unsigned(bias[m]) : 0u;
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
                    const XT *xp = CL ? x + (int64_t(n) * in_pix + ipix) * p.C + c0
                                      : x + (int64_t(n) * p.C + c0) * in_pix + ipix;
                    const int64_t xstep = CL ? 1 : in_pix;
                    const WT *wp = w + (int64_t(c0) * p.Mg + mm) * taps + kflat;
                    const int64_t wstep = int64_t(p.Mg) * taps;
                    for (int cc = 0; cc < p.Cg; ++cc)
                        acc += unsigned((int(xp[cc * xstep]) - p.x_zp) * (int(wp[cc * wstep]) - wz));
                }
            }
        }
        const float mult = requant_mult(p.x_scale, w_scale[q], p.y_scale);
        y[idx] = YT(requantize(acc, mult, p.y_zp, p.y_lo, p.y_hi));
    }
}

template <typename XT, typename WT, typename YT>
void launch_q3(bool cl, dim3 grid, hipStream_t st, const void *x, const void *w, const float *ws, const void *wz,
               const int *bias, void *y, const QDirectArgs &p)
{
    const XT *xt = static_cast<const XT *>(x);
    const WT *wt = static_cast<const WT *>(w);
    const WT *wzt = static_cast<const WT *>(wz);
    YT *yt = static_cast<YT *>(y);
    if (cl)
        hipLaunchKernelGGL((qdirect_kernel<XT, WT, YT, true>), grid, dim3(256), 0, st, xt, wt, ws, wzt, bias, yt, p);
    else
        hipLaunchKernelGGL((qdirect_kernel<XT, WT, YT, false>), grid, dim3(256), 0, st, xt, wt, ws, wzt, bias, yt, p);
}

template <typename XT, typename WT>
void launch_q2(ct_dtype yt, bool cl, dim3 grid, hipStream_t st, const void *x, const void *w, const float *ws,
               const void *wz, const int *bias, void *y, const QDirectArgs &p)
{
    if (yt == CT_INT8) launch_q3<XT, WT, int8_t>(cl, grid, st, x, w, ws, wz, bias, y, p);
    else launch_q3<XT, WT, uint8_t>(cl, grid, st, x, w, ws, wz, bias, y, p);
}

template <typename XT>
void launch_q1(ct_dtype wt, ct_dtype yt, bool cl, dim3 grid, hipStream_t st, const void *x, const void *w,
               const float *ws, const void *wz, const int *bias, void *y, const QDirectArgs &p)
{
    if (wt == CT_INT8) launch_q2<XT, int8_t>(yt, cl, grid, st, x, w, ws, wz, bias, y, p);
    else launch_q2<XT, uint8_t>(yt, cl, grid, st, x, w, ws, wz, bias, y, p);
}

bool is_q8(ct_dtype t) { return t == CT_INT8 || t == CT_UINT8; }
int q_lo(ct_dtype t) { return t == CT_INT8 ? -128 : 0; }
int q_hi(ct_dtype t) { return t == CT_INT8 ? 127 : 255; }

ct_status q_fail(ct_status st, const std::string &m)
{
    set_last_error(m);
    return st;
}

}  // namespace
}  // namespace ct

extern "C" {

ct_status qlinear_convtranspose_nd(ct_kernel kernel, int nsp, int channels_last, const void *x, ct_dtype x_type,
                                   const int64_t *x_shape, float x_scale, int32_t x_zero_point, const void *w,
                                   ct_dtype w_type, const int64_t *w_shape, const float *w_scale,
                                   const void *w_zero_point, int64_t wq_len, const int32_t *bias, void *y,
                                   ct_dtype y_type, const int64_t *y_shape, float y_scale, int32_t y_zero_point,
                                   ct_auto_pad auto_pad, const int64_t *strides, const int64_t *dilations,
                                   const int64_t *pads, const int64_t *output_padding, const int64_t *output_shape,
                                   const int64_t *kernel_shape, int64_t group, void *stream)
{
    using namespace ct;
    set_last_error(std::string());
    for (const int t : {enum_int(x_type), enum_int(w_type), enum_int(y_type)}) {
        EnumArgs ea;
        ea.kernel = enum_int(kernel);
        ea.dtype = t;
        ea.auto_pad = enum_int(auto_pad);
        std::string ee;
        const ct_status es = check_enum_args(ea, &ee);
        if (es != CT_OK) return q_fail(es, ee);
    }
    if (!is_q8(x_type) || !is_q8(w_type) || !is_q8(y_type))
        return q_fail(CT_EUNSUPPORTED, "x, w and y types must be CT_UINT8 or CT_INT8");
    if (kernel != CT_KERNEL_AUTO && kernel != CT_KERNEL_DIRECT && kernel != CT_KERNEL_IGEMM)
        return q_fail(CT_EUNSUPPORTED, "the quantized operation runs on the gather or the int8 implicit-GEMM kernel");
    if (channels_last != 0 && channels_last != 1) return q_fail(CT_EINVAL, "channels_last must be 0 or 1");
    if (!std::isfinite(x_scale) || !(x_scale > 0.0f) || !std::isfinite(y_scale) || !(y_scale > 0.0f))
        return q_fail(CT_EINVAL, "x_scale and y_scale must be positive and finite");
    if (x_zero_point < q_lo(x_type) || x_zero_point > q_hi(x_type))
        return q_fail(CT_EINVAL, "x_zero_point is outside the range of x's type");
    if (y_zero_point < q_lo(y_type) || y_zero_point > q_hi(y_type))
        return q_fail(CT_EINVAL, "y_zero_point is outside the range of y's type");
    if (!y_shape) return q_fail(CT_EINVAL, "y_shape is NULL");
    Attrs at;
    at.auto_pad = auto_pad;
    at.strides = strides;
    at.dilations = dilations;
    at.pads = pads;
    at.output_padding = output_padding;
    at.output_shape = output_shape;
    at.kernel_shape = kernel_shape;
    at.group = group;
    Geom g;
    std::string err;
    ct_status st = resolve(nsp, x_shape, w_shape, at, &g, &err);
    if (st != CT_OK) return q_fail(st, err);
    const int lead = kAxes - nsp;
    bool same = y_shape[0] == g.N && y_shape[1] == g.M;
    for (int a = 0; a < nsp; ++a) same = same && y_shape[2 + a] == g.O[lead + a];
    if (!same) return q_fail(CT_ESHAPE, "y_shape differs from the resolved output shape");
    if (wq_len != 1 && wq_len != g.M) return q_fail(CT_EINVAL, "w_scale / w_zero_point must have length 1 or M");
    if (reinterpret_cast<uintptr_t>(bias) % 4 != 0 || reinterpret_cast<uintptr_t>(w_scale) % 4 != 0)
        return q_fail(CT_EINVAL, "bias and w_scale must be 4-byte aligned");
    if (g.y_elems() == 0) return CT_OK;
    if (!y) return q_fail(CT_EINVAL, "y is NULL");
    if (!w_scale || !w_zero_point) return q_fail(CT_EINVAL, "w_scale and w_zero_point are required");
    if (g.x_elems() > 0 && !x) return q_fail(CT_EINVAL, "x is NULL");
    if (g.w_elems() > 0 && !w) return q_fail(CT_EINVAL, "w is NULL");

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool cl = channels_last != 0;
    std::string why;
    const bool mfma = kernel != CT_KERNEL_DIRECT && g.x_elems() > 0 && qigemm_supports(g, cl, x, &why);
    if (kernel == CT_KERNEL_IGEMM && !mfma)
        return q_fail(CT_EUNSUPPORTED, "the int8 implicit-GEMM kernel cannot serve this call: " + why);
    if (mfma) {
        QuantCall qc;
        qc.x_type = x_type;
        qc.w_type = w_type;
        qc.y_type = y_type;
        qc.x_scale = x_scale;
        qc.y_scale = y_scale;
        qc.x_zp = x_zero_point;
        qc.y_zp = y_zero_point;
        qc.w_scale = w_scale;
        qc.w_zp = w_zero_point;
        qc.wq_len = wq_len;
        qc.bias = reinterpret_cast<const int *>(bias);
        st = launch_qigemm(g, cl, x, w, y, qc, hs, &err);
        if (st != CT_OK) return q_fail(st, err);
        return CT_OK;
    }

    QDirectArgs p;
    p.total = g.y_elems();
    p.N = int(g.N);
    p.C = int(g.C);
    p.M = int(g.M);
    p.Cg = int(g.Cg);
    p.Mg = int(g.Mg);
    p.wq_per_channel = wq_len == g.M && g.M != 1 ? 1 : 0;
    p.has_bias = bias != nullptr;
    for (int a = 0; a < kAxes; ++a) {
        p.L[a] = int(g.L[a]);
        p.K[a] = int(g.K[a]);
        p.s[a] = int(g.s[a]);
        p.d[a] = int(g.d[a]);
        p.b[a] = int(g.b[a]);
        p.O[a] = int(g.O[a]);
    }
    p.x_zp = x_zero_point;
    p.y_zp = y_zero_point;
    p.y_lo = q_lo(y_type);
    p.y_hi = q_hi(y_type);
    p.x_scale = x_scale;
    p.y_scale = y_scale;
    int64_t blocks = (p.total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride loop covers the rest
    const int *bt = reinterpret_cast<const int *>(bias);
    mark_before(hs);
    if (x_type == CT_INT8)
        launch_q1<int8_t>(w_type, y_type, cl, dim3(unsigned(blocks)), hs, x, w, w_scale, w_zero_point, bt, y, p);
    else
        launch_q1<uint8_t>(w_type, y_type, cl, dim3(unsigned(blocks)), hs, x, w, w_scale, w_zero_point, bt, y, p);
    mark_after(hs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return q_fail(CT_EDEVICE, std::string("quantized kernel launch failed: ") + hipGetErrorString(e));
    return CT_OK;
}

}  // extern "C"
