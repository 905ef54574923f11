// ct_noalloc.hip -- convtranspose_nd_noalloc: the transposed convolution for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// It is convtranspose_nd_with_kernel with the workspace taken from a fixed array in
// device memory that the library holds on each device until the process ends, instead
// of a caller buffer or the library's stream-ordered pool.  The only kernels that use a
// workspace are those of the float16 implicit GEMM (its re-laid-out weights, which the
// weight re-layout kernel writes completely, padding included, before the MFMA kernel
// reads them: nothing in the array has to start at zero).
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "ct_internal.hpp"

// Largest workspace served: 16 MiB (float16 weights of up to 8 Mi elements after padding,
// e.g. 512 x 512 x 4 x 4 or 512 x 256 x 3 x 3 x 3 with room to spare).
static constexpr size_t kScratchBytes = size_t(16) << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on each device, looked up once per device with that device
// current.  In host code the array's own name is not a device address.
std::mutex g_mu;
void *g_scratch_ptr[64] = {};

ct_status scratch_address(void **out, std::string *err)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = std::string("no current HIP device: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    if (dev < 0 || dev >= 64) {
        *err = "device index outside 0..63";
        return CT_EDEVICE;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = std::string("hipGetSymbolAddress of the static workspace failed: ") + hipGetErrorString(e);
            return CT_EDEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CT_OK;
}

}  // namespace

extern "C" {

size_t convtranspose_noalloc_max_workspace(void) { return kScratchBytes; }

ct_status convtranspose_nd_noalloc(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last, const void *x,
                                   const int64_t *x_shape, const void *w, const int64_t *w_shape, const void *bias,
                                   void *y, const int64_t *y_shape, ct_auto_pad auto_pad, const int64_t *strides,
                                   const int64_t *dilations, const int64_t *pads, const int64_t *output_padding,
                                   const int64_t *output_shape, const int64_t *kernel_shape, int64_t group,
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
        if (es != CT_OK) {
            ct::set_last_error(ee);
            return es;
        }
    }
    // host-side sizing first: invalid arguments and too large a workspace fail here,
    // before any device is touched
    size_t need = 0;
    ct_status st = convtranspose_workspace_size(kernel, dtype, nsp, channels_last, x, x_shape, w_shape, auto_pad,
                                                strides, dilations, pads, output_padding, output_shape,
                                                kernel_shape, group, &need);
    if (st != CT_OK) return st;
    if (need > kScratchBytes) {
        ct::set_last_error("the call needs a workspace of " + std::to_string(need) +
                           " bytes; convtranspose_nd_noalloc serves at most " + std::to_string(kScratchBytes) +
                           " (use convtranspose_nd_with_kernel with a caller workspace)");
        return CT_EINVAL;
    }
    void *ws = nullptr;
    if (need > 0) {
        std::string err;
        st = scratch_address(&ws, &err);
        if (st != CT_OK) {
            ct::set_last_error(err);
            return st;
        }
    }
    return convtranspose_nd_with_kernel(kernel, dtype, nsp, channels_last, x, x_shape, w, w_shape, bias, y, y_shape,
                                        auto_pad, strides, dilations, pads, output_padding, output_shape,
                                        kernel_shape, group, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
