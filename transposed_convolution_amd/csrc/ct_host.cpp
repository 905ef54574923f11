// ct_host.cpp -- C ABI entry points, attribute resolver, stride-phase plan and the
// shape-based dispatcher of libconvtranspose.so.
//
// Operation and attributes: webgpu-kernels "ai.onnx.ConvTranspose" README (sections
// Description, Inputs, Outputs, Attributes, Type constraints, Implementation variants:
// one implementation is chosen per call from the shapes and dtypes); ClikaRT
// "conv_transpose" API page (channels-last tensors; errors on inconsistent channel or
// group arithmetic, span lengths or an unserved dtype, with a reason string).
#include <hip/hip_runtime.h>

#include <cstring>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>

#include "ct_internal.hpp"

namespace ct {
namespace {

// Floor and ceiling division for a positive divisor (C++ '/' truncates toward zero).
inline int64_t floor_div(int64_t a, int64_t q) { return a >= 0 ? a / q : -((-a + q - 1) / q); }
inline int64_t ceil_div(int64_t a, int64_t q) { return -floor_div(-a, q); }

// Split a total pad into (begin, end): halves truncated toward zero, the remainder of
// an odd total on the requested side.
void split_total(int64_t tot, bool odd_at_begin, int64_t *b, int64_t *e)
{
    const int64_t half = tot / 2, rem = tot - 2 * half;
    *b = half + (odd_at_begin ? rem : 0);
    *e = half + (odd_at_begin ? 0 : rem);
}

}  // namespace

ct_status resolve(int nsp, const int64_t *xs, const int64_t *ws, const Attrs &at, Geom *g,
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
    for (int a = 0; a < nsp + 2; ++a)
        if (xs[a] < 0) return bad("X dimensions must be >= 0");
    if (at.group < 1) return bad("group must be >= 1");
    if (ws[0] != xs[1]) return bad("W.shape[0] must equal the input channel count C");
    if (xs[1] % at.group != 0) return bad("C must be a multiple of group");
    if (ws[1] < 1) return bad("W.shape[1] (output channels per group) must be >= 1");
    if (at.pads && at.auto_pad != CT_NOTSET) return bad("pads cannot be combined with auto_pad");

    g->nsp = nsp;
    g->N = xs[0];
    g->C = xs[1];
    g->G = at.group;
    g->Cg = xs[1] / at.group;
    g->Mg = ws[1];
    g->M = ws[1] * at.group;

    const int lead = kAxes - nsp;
    for (int t = 0; t < lead; ++t) {
        g->L[t] = g->K[t] = g->s[t] = g->d[t] = g->O[t] = 1;
        g->b[t] = g->e[t] = g->op[t] = 0;
    }
    for (int a = 0; a < nsp; ++a) {
        const int t = lead + a;
        const int64_t L = xs[2 + a], K = ws[2 + a];
        const int64_t s = at.strides ? at.strides[a] : 1;
        const int64_t d = at.dilations ? at.dilations[a] : 1;
        const int64_t op = at.output_padding ? at.output_padding[a] : 0;
        if (K < 1) return bad("W spatial dimensions must be >= 1");
        if (at.kernel_shape && at.kernel_shape[a] != K)
            return bad("kernel_shape does not match W's spatial dimensions");
        if (s < 1 || d < 1) return bad("strides and dilations must be >= 1");
        if (op < 0 || op >= (s > d ? s : d))
            return bad("output_padding must be >= 0 and smaller than max(stride, dilation)");
        // Extent of the scatter footprint with output_padding at the high end.
        const int64_t footprint = (L - 1) * s + (K - 1) * d + 1 + op;
        int64_t b = 0, e = 0, O = 0;
        if (at.output_shape) {
            O = at.output_shape[a];
            if (O < 0) return bad("output_shape entries must be >= 0");
            const int64_t tot = footprint - O;
            if (at.pads) {
                b = at.pads[a];
                e = at.pads[nsp + a];
                if (b < 0 || e < 0) return bad("pads must be >= 0");
                if (b + e != tot) return bad("pads are inconsistent with output_shape");
            } else {
                split_total(tot, at.auto_pad == CT_SAME_LOWER, &b, &e);
            }
        } else if (at.auto_pad == CT_SAME_UPPER || at.auto_pad == CT_SAME_LOWER) {
            O = L * s;
            split_total(footprint - O, at.auto_pad == CT_SAME_LOWER, &b, &e);
        } else if (at.auto_pad == CT_VALID) {
            O = footprint;
        } else {
            if (at.pads) {
                b = at.pads[a];
                e = at.pads[nsp + a];
                if (b < 0 || e < 0) return bad("pads must be >= 0");
            }
            O = footprint - b - e;
        }
        if (O < 0) return bad("the resolved output size is negative");
        if (L > INT32_MAX || O > INT32_MAX || K > INT32_MAX || s > INT32_MAX || d > INT32_MAX ||
            b > INT32_MAX || b < -INT32_MAX)
            return bad("spatial sizes and attributes must fit in 32 bits");
        g->L[t] = L;
        g->K[t] = K;
        g->s[t] = s;
        g->d[t] = d;
        g->b[t] = b;
        g->e[t] = e;
        g->op[t] = op;
        g->O[t] = O;
    }
    if (g->C > INT32_MAX || g->M > INT32_MAX || g->N > INT32_MAX)
        return bad("batch and channel counts must fit in 32 bits");
    return CT_OK;
}

double useful_macs(const Geom &g)
{
    double total = double(g.N) * double(g.Cg) * double(g.M);
    for (int t = 0; t < kAxes; ++t) {
        // For tap k, the inputs i that land inside are those with
        // ceil((b - k d)/s) <= i <= floor((O - 1 + b - k d)/s), within [0, L).
        int64_t pairs = 0;
        for (int64_t k = 0; k < g.K[t]; ++k) {
            const int64_t shift = g.b[t] - k * g.d[t];
            int64_t lo = ceil_div(shift, g.s[t]);
            int64_t hi = floor_div(g.O[t] - 1 + shift, g.s[t]);
            if (lo < 0) lo = 0;
            if (hi > g.L[t] - 1) hi = g.L[t] - 1;
            if (hi >= lo) pairs += hi - lo + 1;
        }
        total *= double(pairs);
    }
    return total;
}

bool axis_phase(const Geom &g, int a, int r, AxisPhase *ph)
{
    const int64_t s = g.s[a];
    ph->r = r;
    ph->J = r < g.O[a] ? int((g.O[a] - r + s - 1) / s) : 0;
    ph->ntaps = 0;
    for (int64_t k = 0; k < g.K[a]; ++k) {
        const int64_t num = r + g.b[a] - k * g.d[a];
        if (num - floor_div(num, s) * s != 0) continue;  // not a multiple of s
        if (ph->ntaps == kMaxPhaseTaps) return false;
        ph->k[ph->ntaps] = int(k);
        ph->beta[ph->ntaps] = int(floor_div(num, s));
        ++ph->ntaps;
    }
    return true;
}

hipError_t scratch_malloc(void **p, size_t bytes, hipStream_t st)
{
    // One memory pool per device, owned by the library and created on first use; freed
    // scratch stays in it (release threshold: never trim) so repeated calls reuse it
    // without mapping memory again.  The device's default pool is left as it is.
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipMallocAsync(p, bytes, st);
    hipMemPool_t pool = nullptr;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (!pools[dev]) {
            hipMemPoolProps props;
            std::memset(&props, 0, sizeof(props));
            props.allocType = hipMemAllocationTypePinned;
            props.handleTypes = hipMemHandleTypeNone;
            props.location.type = hipMemLocationTypeDevice;
            props.location.id = dev;
            hipMemPool_t created = nullptr;
            e = hipMemPoolCreate(&created, &props);
            if (e != hipSuccess) return e;
            uint64_t keep = UINT64_MAX;
            e = hipMemPoolSetAttribute(created, hipMemPoolAttrReleaseThreshold, &keep);
            if (e != hipSuccess) {
                (void)hipMemPoolDestroy(created);
                return e;
            }
            pools[dev] = created;
        }
        pool = pools[dev];
    }
    return hipMallocFromPoolAsync(p, bytes, pool, st);
}

ProfileEvents &profile_events()
{
    thread_local ProfileEvents ev;
    return ev;
}

}  // namespace ct

// ------------------------------------------------------------------------------------
// C ABI
// ------------------------------------------------------------------------------------
namespace {

thread_local std::string t_error;

}  // namespace

void ct::set_last_error(const std::string &msg) { t_error = msg; }

namespace {

ct_status fail(ct_status st, const std::string &msg)
{
    t_error = msg;
    return st;
}

ct::Attrs make_attrs(ct_auto_pad auto_pad, const int64_t *strides, const int64_t *dilations,
                     const int64_t *pads, const int64_t *output_padding,
                     const int64_t *output_shape, const int64_t *kernel_shape, int64_t group)
{
    ct::Attrs at;
    at.auto_pad = auto_pad;
    at.strides = strides;
    at.dilations = dilations;
    at.pads = pads;
    at.output_padding = output_padding;
    at.output_shape = output_shape;
    at.kernel_shape = kernel_shape;
    at.group = group;
    return at;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates a call and picks its kernel family.  y_shape may be NULL (selection only).
ct_status prepare(ct_kernel want, ct_dtype dt, int nsp, int cl, const void *x,
                  const int64_t *x_shape, const void *w, const int64_t *w_shape, const void *bias,
                  const void *y, const int64_t *y_shape, const ct::Attrs &at, ct::Geom *g,
                  ct_kernel *chosen)
{
    if (dt != CT_FLOAT32 && dt != CT_FLOAT16)
        return fail(CT_EUNSUPPORTED, "dtype must be CT_FLOAT32 or CT_FLOAT16");
    if (cl != 0 && cl != 1) return fail(CT_EINVAL, "channels_last must be 0 or 1");
    std::string err;
    ct_status st = ct::resolve(nsp, x_shape, w_shape, at, g, &err);
    if (st != CT_OK) return fail(st, err);
    if (y_shape) {
        const int lead = ct::kAxes - nsp;
        bool same = y_shape[0] == g->N && y_shape[1] == g->M;
        for (int a = 0; a < nsp; ++a) same = same && y_shape[2 + a] == g->O[lead + a];
        if (!same) return fail(CT_ESHAPE, "y_shape differs from the resolved output shape");
    }
    const size_t esz = dt == CT_FLOAT32 ? 4 : 2;
    if (!aligned(x, esz) || !aligned(w, esz) || !aligned(y, esz) || !aligned(bias, esz))
        return fail(CT_EINVAL, "tensor pointers must be aligned to the element size");
    if (g->y_elems() == 0) {
        *chosen = CT_KERNEL_NONE;
        return CT_OK;
    }
    if (!y) return fail(CT_EINVAL, "y is NULL");
    if (g->x_elems() > 0 && !x) return fail(CT_EINVAL, "x is NULL");
    if (g->w_elems() > 0 && !w) return fail(CT_EINVAL, "w is NULL");

    std::string why;
    switch (want) {
        case CT_KERNEL_AUTO:
            // MFMA tiles are 32 wide in output channels and 32 deep in input channels:
            // below 16 of either most of each tile would be padding.
            if (g->Cg >= 16 && g->Mg >= 16 && ct::igemm_supports(*g, dt, cl, x, &why))
                *chosen = CT_KERNEL_IGEMM;
            else if (ct::grouped_supports(*g, dt, cl, x))
                *chosen = CT_KERNEL_GROUPED;
            else
                *chosen = CT_KERNEL_DIRECT;
            return CT_OK;
        case CT_KERNEL_DIRECT:
            *chosen = CT_KERNEL_DIRECT;
            return CT_OK;
        case CT_KERNEL_GROUPED:
            if (!ct::grouped_supports(*g, dt, cl, x))
                return fail(CT_EUNSUPPORTED, "the grouped kernel cannot serve this call");
            *chosen = CT_KERNEL_GROUPED;
            return CT_OK;
        case CT_KERNEL_IGEMM:
            if (!ct::igemm_supports(*g, dt, cl, x, &why))
                return fail(CT_EUNSUPPORTED, "the implicit-GEMM kernel cannot serve this call: " + why);
            *chosen = CT_KERNEL_IGEMM;
            return CT_OK;
        default:
            return fail(CT_EINVAL, "unknown kernel family");
    }
}

}  // namespace

extern "C" {

ct_status convtranspose_output_shape(int nsp, const int64_t *x_shape, const int64_t *w_shape,
                                     ct_auto_pad auto_pad, const int64_t *strides,
                                     const int64_t *dilations, const int64_t *pads,
                                     const int64_t *output_padding, const int64_t *output_shape,
                                     const int64_t *kernel_shape, int64_t group,
                                     int64_t *y_shape_out, int64_t *pads_out)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return fail(es, ee);
    }
    if (!y_shape_out) return fail(CT_EINVAL, "y_shape_out is NULL");
    ct::Geom g;
    std::string err;
    const ct::Attrs at = make_attrs(auto_pad, strides, dilations, pads, output_padding,
                                    output_shape, kernel_shape, group);
    ct_status st = ct::resolve(nsp, x_shape, w_shape, at, &g, &err);
    if (st != CT_OK) return fail(st, err);
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

ct_status convtranspose_useful_macs(int nsp, const int64_t *x_shape, const int64_t *w_shape,
                                    ct_auto_pad auto_pad, const int64_t *strides,
                                    const int64_t *dilations, const int64_t *pads,
                                    const int64_t *output_padding, const int64_t *output_shape,
                                    const int64_t *kernel_shape, int64_t group, double *macs_out)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return fail(es, ee);
    }
    if (!macs_out) return fail(CT_EINVAL, "macs_out is NULL");
    ct::Geom g;
    std::string err;
    const ct::Attrs at = make_attrs(auto_pad, strides, dilations, pads, output_padding,
                                    output_shape, kernel_shape, group);
    ct_status st = ct::resolve(nsp, x_shape, w_shape, at, &g, &err);
    if (st != CT_OK) return fail(st, err);
    *macs_out = ct::useful_macs(g);
    return CT_OK;
}

int convtranspose_select_kernel(ct_dtype dtype, int nsp, int channels_last, const void *x,
                                const int64_t *x_shape, const void *w, const int64_t *w_shape,
                                const void *bias, const void *y, ct_auto_pad auto_pad,
                                const int64_t *strides, const int64_t *dilations,
                                const int64_t *pads, const int64_t *output_padding,
                                const int64_t *output_shape, const int64_t *kernel_shape,
                                int64_t group)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.dtype = ct::enum_int(dtype);
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return (fail(es, ee), -1);
    }
    ct::Geom g;
    ct_kernel k = CT_KERNEL_AUTO;
    const ct::Attrs at = make_attrs(auto_pad, strides, dilations, pads, output_padding,
                                    output_shape, kernel_shape, group);
    if (prepare(CT_KERNEL_AUTO, dtype, nsp, channels_last, x, x_shape, w, w_shape, bias, y,
                nullptr, at, &g, &k) != CT_OK)
        return -1;
    return int(k);
}

ct_status convtranspose_workspace_size(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last,
                                       const void *x, const int64_t *x_shape, const int64_t *w_shape,
                                       ct_auto_pad auto_pad, const int64_t *strides,
                                       const int64_t *dilations, const int64_t *pads,
                                       const int64_t *output_padding, const int64_t *output_shape,
                                       const int64_t *kernel_shape, int64_t group, size_t *bytes_out)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.kernel = ct::enum_int(kernel);
        ea.dtype = ct::enum_int(dtype);
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return fail(es, ee);
    }
    if (!bytes_out) return fail(CT_EINVAL, "bytes_out is NULL");
    ct::Geom g;
    ct_kernel k = CT_KERNEL_AUTO;
    const ct::Attrs at = make_attrs(auto_pad, strides, dilations, pads, output_padding,
                                    output_shape, kernel_shape, group);
    // w, bias and y are not inspected for the choice beyond alignment: pass aligned stand-ins
    const void *aligned_stub = reinterpret_cast<const void *>(uintptr_t(256));
    ct_status st = prepare(kernel, dtype, nsp, channels_last, x ? x : aligned_stub, x_shape,
                           aligned_stub, w_shape, nullptr, aligned_stub, nullptr, at, &g, &k);
    if (st != CT_OK) return st;
    *bytes_out = (k == CT_KERNEL_IGEMM) ? ct::igemm_workspace_bytes(g, dtype) : 0;
    return CT_OK;
}

ct_status convtranspose_nd_fused(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last,
                                 const void *x, const int64_t *x_shape, const void *w,
                                 const int64_t *w_shape, const void *bias, void *y,
                                 const int64_t *y_shape, ct_auto_pad auto_pad,
                                 const int64_t *strides, const int64_t *dilations,
                                 const int64_t *pads, const int64_t *output_padding,
                                 const int64_t *output_shape, const int64_t *kernel_shape,
                                 int64_t group, ct_activation activation, float act_p0, float act_p1,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.kernel = ct::enum_int(kernel);
        ea.dtype = ct::enum_int(dtype);
        ea.auto_pad = ct::enum_int(auto_pad);
        ea.activation = ct::enum_int(activation);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return fail(es, ee);
    }
    ct::Act act;
    act.kind = int(activation);
    act.p0 = act_p0;
    act.p1 = act_p1;
    switch (activation) {
        case CT_ACT_IDENTITY:
        case CT_ACT_RELU: break;
        case CT_ACT_LEAKY_RELU:
            if (!std::isfinite(act_p0)) return fail(CT_EINVAL, "leaky ReLU slope must be finite");
            break;
        case CT_ACT_CLIP:
            if (!std::isfinite(act_p0) || !std::isfinite(act_p1) || !(act_p0 <= act_p1))
                return fail(CT_EINVAL, "clip bounds must be finite with lower <= upper");
            break;
        default: return fail(CT_EINVAL, "unknown activation");
    }
    if (!y_shape) return fail(CT_EINVAL, "y_shape is NULL");
    if (workspace && !aligned(workspace, 16)) return fail(CT_EINVAL, "workspace must be 16-byte aligned");
    ct::Geom g;
    ct_kernel k = CT_KERNEL_AUTO;
    const ct::Attrs at = make_attrs(auto_pad, strides, dilations, pads, output_padding,
                                    output_shape, kernel_shape, group);
    ct_status st = prepare(kernel, dtype, nsp, channels_last, x, x_shape, w, w_shape, bias, y,
                           y_shape, at, &g, &k);
    if (st != CT_OK) return st;
    if (k == CT_KERNEL_NONE) return CT_OK;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    std::string err;
    const bool cl = channels_last != 0;
    switch (k) {
        case CT_KERNEL_IGEMM:
            st = ct::launch_igemm(g, dtype, cl, x, w, bias, y, act, workspace, workspace_bytes, hs, &err);
            break;
        case CT_KERNEL_GROUPED: st = ct::launch_grouped(g, dtype, cl, x, w, bias, y, act, hs, &err); break;
        default: st = ct::launch_direct(g, dtype, cl, x, w, bias, y, act, hs, &err); break;
    }
    if (st != CT_OK) return fail(st, err);
    return CT_OK;
}

ct_status convtranspose_nd_with_kernel(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last,
                                       const void *x, const int64_t *x_shape, const void *w,
                                       const int64_t *w_shape, const void *bias, void *y,
                                       const int64_t *y_shape, ct_auto_pad auto_pad,
                                       const int64_t *strides, const int64_t *dilations,
                                       const int64_t *pads, const int64_t *output_padding,
                                       const int64_t *output_shape, const int64_t *kernel_shape,
                                       int64_t group, void *workspace, size_t workspace_bytes,
                                       void *stream)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.kernel = ct::enum_int(kernel);
        ea.dtype = ct::enum_int(dtype);
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return fail(es, ee);
    }
    return convtranspose_nd_fused(kernel, dtype, nsp, channels_last, x, x_shape, w, w_shape, bias, y,
                                  y_shape, auto_pad, strides, dilations, pads, output_padding,
                                  output_shape, kernel_shape, group, CT_ACT_IDENTITY, 0.0f, 0.0f,
                                  workspace, workspace_bytes, stream);
}

ct_status convtranspose_nd(ct_dtype dtype, int nsp, int channels_last, const void *x,
                           const int64_t *x_shape, const void *w, const int64_t *w_shape,
                           const void *bias, void *y, const int64_t *y_shape,
                           ct_auto_pad auto_pad, const int64_t *strides, const int64_t *dilations,
                           const int64_t *pads, const int64_t *output_padding,
                           const int64_t *output_shape, const int64_t *kernel_shape,
                           int64_t group, void *stream)
{
    t_error.clear();
    {
        ct::EnumArgs ea;
        ea.dtype = ct::enum_int(dtype);
        ea.auto_pad = ct::enum_int(auto_pad);
        std::string ee;
        const ct_status es = ct::check_enum_args(ea, &ee);
        if (es != CT_OK) return fail(es, ee);
    }
    return convtranspose_nd_with_kernel(CT_KERNEL_AUTO, dtype, nsp, channels_last, x, x_shape, w,
                                        w_shape, bias, y, y_shape, auto_pad, strides, dilations,
                                        pads, output_padding, output_shape, kernel_shape, group,
                                        nullptr, 0, stream);
}

ct_status convtranspose_profile_events(void *before, void *after)
{
    t_error.clear();
    if ((before == nullptr) != (after == nullptr)) return fail(CT_EINVAL, "give both events or neither");
    ct::profile_events().before = static_cast<hipEvent_t>(before);
    ct::profile_events().after = static_cast<hipEvent_t>(after);
    return CT_OK;
}

ct_status convtranspose_set_igemm_tile(int tile)
{
    t_error.clear();
    if (tile < -1 || tile >= ct::igemm_tile_count())
        return fail(CT_EINVAL, "tile must be -1 (automatic) or 0.." + std::to_string(ct::igemm_tile_count() - 1));
    ct::igemm_force_tile(tile);
    return CT_OK;
}

int convtranspose_igemm_tile(void) { return ct::igemm_forced_tile(); }

const char *convtranspose_last_error(void) { return t_error.c_str(); }

const char *convtranspose_kernel_name(int kernel)
{
    switch (kernel) {
        case CT_KERNEL_AUTO: return "auto";
        case CT_KERNEL_DIRECT: return "direct";
        case CT_KERNEL_GROUPED: return "grouped";
        case CT_KERNEL_IGEMM: return "igemm";
        case CT_KERNEL_NONE: return "none";
        default: return "unknown";
    }
}

}  // extern "C"
