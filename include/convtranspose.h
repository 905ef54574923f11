/*
 * convtranspose.h -- C ABI of libconvtranspose.so, an N-D transposed convolution
 * (ONNX ConvTranspose) for AMD Instinct MI355X (gfx950).
 *
 * Operation (webgpu-kernels "ai.onnx.ConvTranspose" README, sections Description,
 * Inputs, Outputs, Attributes and Type constraints; ClikaRT "conv_transpose" API page,
 * description):
 *   X is (N, C, D1..Dn), W is (C, M/group, k1..kn), optional bias has length M, and
 *   Y is (N, M, O1..On).  Every input sample X[n,c,i] is sent through every filter
 *   tap k of its group to output position o_a = i_a*s_a - b_a + k_a*d_a on each
 *   spatial axis a (s = stride, d = dilation, b = begin pad), and summed there when
 *   the position lies inside Y; Y starts at bias[m].  Out channel m belongs to group
 *   m / (M/group) and reads input channels c of that group through W[c, m % (M/group), k].
 *   Output size per axis: O = s*(L-1) + output_padding + d*(K-1) + 1 - b - e.
 *   Element type T is float32 or float16 for X, W, bias and Y alike; float16 inputs
 *   are accumulated in float32 and rounded once (to nearest even) into Y.
 *
 * Attribute pointers: a NULL attribute pointer means "absent" and its ONNX default
 * applies (strides 1, dilations 1, pads 0, output_padding 0; output_shape and
 * kernel_shape not given).  Per-axis arrays have nsp entries, pads has 2*nsp
 * (all begins, then all ends).  Readings where the pages leave a rule open:
 *   - 0 <= output_padding < max(stride, dilation); strides, dilations >= 1; pads >= 0;
 *   - pads together with an auto_pad other than NOTSET are rejected;
 *   - SAME_UPPER / SAME_LOWER give O = L*stride; the total pad
 *     tot = s*(L-1) + op + d*(K-1) + 1 - O is halved with truncation toward zero and
 *     the odd remainder goes to the end (UPPER) or the beginning (LOWER);
 *   - output_shape, when given, sets O and its total pad is split the same way (odd
 *     part at the beginning only for SAME_LOWER); explicit pads given with it must
 *     sum to that total;
 *   - kernel_shape, when given, must equal W's spatial dims.
 *
 * Shapes are always passed in logical ONNX order.  Buffers are owned by the caller,
 * must be dense in the stated layout and aligned to the element size; the library
 * keeps no pointer after a call returns.  The float16 implicit-GEMM path re-lays W out
 * into scratch memory: a caller workspace (convtranspose_nd_with_kernel), or else
 * stream-ordered scratch taken and released on the call's stream.  Such scratch comes
 * from a memory pool the library creates for each device on first use and keeps until
 * the process ends (freed scratch stays in that pool for later calls; the device's
 * default pool is not touched).
 *
 * Thread safety: every call is re-entrant; the error text is per host thread.
 */
#ifndef CONVTRANSPOSE_H
#define CONVTRANSPOSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CT_OK = 0,
    CT_EINVAL = 1,        /* bad attribute, shape arithmetic, pointer or alignment      */
    CT_ESHAPE = 2,        /* y_shape differs from the resolved output shape             */
    CT_EUNSUPPORTED = 3,  /* dtype not served, or a forced kernel cannot serve the call */
    CT_EDEVICE = 4        /* the HIP runtime reported an error at launch                */
} ct_status;

/* element types: the float types serve the float entry points, the 8-bit integer types
 * the quantized one (qlinear_convtranspose_nd) */
typedef enum { CT_FLOAT32 = 0, CT_FLOAT16 = 1, CT_INT8 = 2, CT_UINT8 = 3 } ct_dtype;

typedef enum { CT_NOTSET = 0, CT_SAME_UPPER = 1, CT_SAME_LOWER = 2, CT_VALID = 3 } ct_auto_pad;

/* Kernel families (for convtranspose_nd_with_kernel and convtranspose_select_kernel). */
typedef enum {
    CT_KERNEL_AUTO = 0,     /* let the shape-based dispatcher choose                     */
    CT_KERNEL_DIRECT = 1,   /* generic gather, any rank/attributes/layout/dtype          */
    CT_KERNEL_GROUPED = 2,  /* grouped/depthwise bandwidth kernel (small C/g and M/g)    */
    CT_KERNEL_IGEMM = 3,    /* stride-phase implicit GEMM on MFMA (float16 and float32)  */
    CT_KERNEL_NONE = 4      /* nothing to launch: Y is empty                             */
} ct_kernel;

/*
 * Activation applied to every output element after the bias, in the accumulation
 * precision (float32), before the one rounding into T (ClikaRT "conv_transpose" API page:
 * its `activation` argument, default Identity; the pages do not list the other values,
 * so these are the elementwise functions with a plain closed form):
 *   CT_ACT_IDENTITY    v
 *   CT_ACT_RELU        v > 0 ? v : 0
 *   CT_ACT_LEAKY_RELU  v >= 0 ? v : p0 * v          (p0 = slope, finite)
 *   CT_ACT_CLIP        v < p0 ? p0 : (v > p1 ? p1 : v)   (p0 <= p1, both finite)
 */
typedef enum {
    CT_ACT_IDENTITY = 0,
    CT_ACT_RELU = 1,
    CT_ACT_LEAKY_RELU = 2,
    CT_ACT_CLIP = 3
} ct_activation;

/*
 * Resolve the output shape (README Attributes table and Outputs section).  Host only;
 * touches no device.
 *   nsp            spatial rank n, 1..3
 *   x_shape        n+2 entries {N, C, D1..Dn}
 *   w_shape        n+2 entries {C, M/group, k1..kn}
 *   y_shape_out    receives n+2 entries {N, M, O1..On}
 *   pads_out       optional (may be NULL): receives the 2n begin/end pads applied
 *                  (these may be negative when derived from auto_pad/output_shape)
 * Returns CT_OK, or CT_EINVAL with convtranspose_last_error() describing the problem.
 */
ct_status convtranspose_output_shape(int nsp, const int64_t *x_shape, const int64_t *w_shape,
                                     ct_auto_pad auto_pad, const int64_t *strides,
                                     const int64_t *dilations, const int64_t *pads,
                                     const int64_t *output_padding, const int64_t *output_shape,
                                     const int64_t *kernel_shape, int64_t group,
                                     int64_t *y_shape_out, int64_t *pads_out);

/*
 * Number of useful multiply-accumulates of the call: the (input sample, tap) pairs
 * whose target lies inside Y, per spatial axis, multiplied over axes and by
 * N * (C/group) * M.  Zero-insertion holes and taps cropped by pads are not counted.
 * Host only.  Returns CT_OK or CT_EINVAL.
 */
ct_status convtranspose_useful_macs(int nsp, const int64_t *x_shape, const int64_t *w_shape,
                                    ct_auto_pad auto_pad, const int64_t *strides,
                                    const int64_t *dilations, const int64_t *pads,
                                    const int64_t *output_padding, const int64_t *output_shape,
                                    const int64_t *kernel_shape, int64_t group, double *macs_out);

/*
 * The transposed convolution, enqueued on a HIP stream (README Description/Inputs/
 * Outputs/Attributes; channels-last input and output as on the ClikaRT page).
 *   dtype          CT_FLOAT32 or CT_FLOAT16: the element type of x, w, bias and y
 *   nsp            spatial rank, 1..3
 *   channels_last  0: x is stored (N, C, D1..Dn) and y (N, M, O1..On), both dense
 *                  1: x is stored (N, D1..Dn, C) and y (N, O1..On, M), both dense
 *                  (W keeps the ONNX layout (C, M/group, k1..kn) either way)
 *   x, w, y        device pointers (caller-owned; y must not overlap x, w or bias)
 *   bias           device pointer to M elements, or NULL for no bias
 *   x_shape, w_shape, y_shape   logical shapes, n+2 entries each; y_shape must equal
 *                  the resolved output shape, else CT_ESHAPE
 *   auto_pad ... group          ONNX attributes as for convtranspose_output_shape
 *   stream         hipStream_t to enqueue on (NULL: the null stream)
 * All validation happens before anything is enqueued: on any error nothing is launched
 * and y is untouched.  Work is asynchronous: the call returns once the kernels are
 * enqueued.  An empty y (some dimension 0) returns CT_OK with no launch.  When the
 * dispatcher picks the float16 implicit-GEMM path, scratch for the re-laid-out weights
 * is taken from the library's pool (hipMallocFromPoolAsync) and released with
 * hipFreeAsync on `stream`.
 */
ct_status convtranspose_nd(ct_dtype dtype, int nsp, int channels_last, const void *x,
                           const int64_t *x_shape, const void *w, const int64_t *w_shape,
                           const void *bias, void *y, const int64_t *y_shape,
                           ct_auto_pad auto_pad, const int64_t *strides, const int64_t *dilations,
                           const int64_t *pads, const int64_t *output_padding,
                           const int64_t *output_shape, const int64_t *kernel_shape,
                           int64_t group, void *stream);

/*
 * As convtranspose_nd, with the kernel family forced and an optional caller workspace.
 *   kernel          CT_KERNEL_AUTO (the dispatcher's choice) or a family to force;
 *                   CT_EUNSUPPORTED (nothing launched) when that family cannot serve
 *                   the call (e.g. CT_KERNEL_GROUPED for a call with group 1).
 *   workspace       device scratch of workspace_bytes bytes, 16-byte aligned, used for
 *                   the float16 implicit-GEMM path's re-laid-out weights (the float32
 *                   path needs none); it must not be in use
 *                   by other work until this call's kernels have finished on `stream`.
 *                   NULL: the library takes stream-ordered scratch itself from its
 *                   own pool (hipMallocFromPoolAsync / hipFreeAsync on `stream`), as
 *                   convtranspose_nd does.
 *                   Too small a workspace is CT_EINVAL.
 */
ct_status convtranspose_nd_with_kernel(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last,
                                       const void *x, const int64_t *x_shape, const void *w,
                                       const int64_t *w_shape, const void *bias, void *y,
                                       const int64_t *y_shape, ct_auto_pad auto_pad,
                                       const int64_t *strides, const int64_t *dilations,
                                       const int64_t *pads, const int64_t *output_padding,
                                       const int64_t *output_shape, const int64_t *kernel_shape,
                                       int64_t group, void *workspace, size_t workspace_bytes,
                                       void *stream);

/*
 * As convtranspose_nd_with_kernel, with an activation fused into the output stage of
 * whichever kernel runs (see ct_activation): y = act(ConvTranspose(x, w, bias)), the
 * activation evaluated in float32 on the accumulated value plus bias, then one rounding
 * into T.  act_p0 / act_p1 are the activation's parameters (ignored where it has none).
 * An unknown activation, a non-finite parameter or p0 > p1 for CT_ACT_CLIP is
 * CT_EINVAL (nothing launched).  With CT_ACT_IDENTITY this is exactly
 * convtranspose_nd_with_kernel.
 */
ct_status convtranspose_nd_fused(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last,
                                 const void *x, const int64_t *x_shape, const void *w,
                                 const int64_t *w_shape, const void *bias, void *y,
                                 const int64_t *y_shape, ct_auto_pad auto_pad,
                                 const int64_t *strides, const int64_t *dilations,
                                 const int64_t *pads, const int64_t *output_padding,
                                 const int64_t *output_shape, const int64_t *kernel_shape,
                                 int64_t group, ct_activation activation, float act_p0, float act_p1,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): convtranspose_nd_with_kernel with the
 * workspace taken from a fixed 16 MiB array in device memory that the library holds on
 * each device it runs on until the process ends.  The call itself allocates nothing (no
 * hipMalloc, hipFree or pool allocation).  Arguments, layout, ownership and errors are
 * those of convtranspose_nd_with_kernel without the workspace pair.
 *   A call whose workspace (convtranspose_workspace_size) exceeds
 *   convtranspose_noalloc_max_workspace() bytes fails with CT_EINVAL before anything is
 *   enqueued; so do invalid arguments, as for convtranspose_nd_with_kernel.  CT_EDEVICE if
 *   the array's device address cannot be obtained on the current device.
 * Every call on a device shares that device's array and leaves its contents behind (the
 * weight re-layout rewrites every byte a call reads, so nothing is carried over): calls
 * whose work overlaps on one device -- on different streams, or from different host
 * threads without ordering -- race on it.  Order them on one stream.
 */
ct_status convtranspose_nd_noalloc(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last, const void *x,
                                   const int64_t *x_shape, const void *w, const int64_t *w_shape, const void *bias,
                                   void *y, const int64_t *y_shape, ct_auto_pad auto_pad, const int64_t *strides,
                                   const int64_t *dilations, const int64_t *pads, const int64_t *output_padding,
                                   const int64_t *output_shape, const int64_t *kernel_shape, int64_t group,
                                   void *stream);

/* Bytes of the fixed workspace convtranspose_nd_noalloc serves (16 MiB).  Host only. */
size_t convtranspose_noalloc_max_workspace(void);

/*
 * Workspace bytes convtranspose_nd_with_kernel needs for these arguments and kernel
 * choice (0 when the chosen family needs none).  x is inspected for alignment only and
 * may be NULL (then assumed 256-byte aligned).  Host only.  Returns CT_OK or the status
 * the call itself would return for invalid arguments.
 */
ct_status convtranspose_workspace_size(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last,
                                       const void *x, const int64_t *x_shape, const int64_t *w_shape,
                                       ct_auto_pad auto_pad, const int64_t *strides,
                                       const int64_t *dilations, const int64_t *pads,
                                       const int64_t *output_padding, const int64_t *output_shape,
                                       const int64_t *kernel_shape, int64_t group, size_t *bytes_out);

/*
 * The kernel family the dispatcher picks for these arguments (pointers are inspected
 * for alignment only, never dereferenced).  Host only.  Returns a ct_kernel value, or
 * -1 when the arguments are invalid (see convtranspose_last_error()).
 */
int convtranspose_select_kernel(ct_dtype dtype, int nsp, int channels_last, const void *x,
                                const int64_t *x_shape, const void *w, const int64_t *w_shape,
                                const void *bias, const void *y, ct_auto_pad auto_pad,
                                const int64_t *strides, const int64_t *dilations,
                                const int64_t *pads, const int64_t *output_padding,
                                const int64_t *output_shape, const int64_t *kernel_shape,
                                int64_t group);

/*
 * Measurement hook: on the calling host thread, every later call records `before`
 * (a hipEvent_t) on its stream just before launching its dominant kernel (the MFMA
 * kernel, not the weight re-layout; the bandwidth kernel; the direct kernel) and `after`
 * just after it, so hipEventElapsedTime gives that kernel's device time.  Both NULL
 * turns it off.  The events stay owned by the caller.  Returns CT_OK, or CT_EINVAL if
 * only one of the two is NULL.
 */
ct_status convtranspose_profile_events(void *before, void *after);

/*
 * The forward convolution (ONNX Conv) with the same W: the adjoint of the transposed
 * convolution (webgpu-kernels "ai.onnx.QLinearConv" README, Inputs and Attributes tables,
 * for the convolution's layout and attributes: W is (M, C/group, k1..kn), auto_pad
 * SAME_* keeps ceil(L / stride) outputs).
 *   Y[n, m, o] = bias[m] + sum over c of m's group and taps k of X[n, c, o*s - b + k*d] W[m, c', k]
 * with X = 0 outside the input.  Readings where the pages are silent: the outputs are
 * the window positions that fit inside the padded input,
 * O = floor((L + b + e - d*(K-1) - 1) / s) + 1 (0 if none fits); SAME's total pad
 * max(0, (O-1)*s + d*(K-1) + 1 - L) puts the odd part at the end (UPPER) or the beginning
 * (LOWER); pads with an auto_pad other than NOTSET, negative pads, strides or dilations
 * below 1 and a kernel_shape that differs from W are CT_EINVAL.
 * With a transposed convolution's strides, dilations, begin pads and end pads
 * e - output_padding, Conv_W is its adjoint: <ConvT_W(x), y> = <x, Conv_W(y)>.
 *
 * Host only; writes y_shape_out[nsp+2] = {N, M, O1..On} and, if pads_out is not NULL,
 * the 2*nsp applied pads.  Returns CT_OK or CT_EINVAL.
 */
ct_status convolution_output_shape(int nsp, const int64_t *x_shape, const int64_t *w_shape,
                                   ct_auto_pad auto_pad, const int64_t *strides,
                                   const int64_t *dilations, const int64_t *pads,
                                   const int64_t *kernel_shape, int64_t group, int64_t *y_shape_out,
                                   int64_t *pads_out);

/*
 * The forward convolution enqueued on `stream`.  Arguments as for convtranspose_nd,
 * except: x is (N, C, D1..Dn), w is (M, C/group, k1..kn), bias has M elements, y_shape
 * must equal convolution_output_shape's result, and there is no output_padding or
 * output_shape.
 *   kernel  CT_KERNEL_AUTO (the MFMA path where it serves the shape, else the gather
 *           kernel), CT_KERNEL_DIRECT (the gather kernel, any arguments) or
 *           CT_KERNEL_IGEMM (CT_EUNSUPPORTED when the MFMA path cannot serve the call).
 *           The MFMA path takes stride-1 convolutions with C/group and M/group of at
 *           least 16 as the stride-1 transposed convolution (the same correlation with
 *           reversed taps), and strided convolutions with dilation 1 after taking the
 *           input phases as channels: tap k = s*k' + rho reads phase rho of the padded
 *           input, xs_rho[j] = X[s*j + rho - b], at j = o + k', a stride-1 correlation
 *           over C * prod(s) channels with ceil(K / s) taps.
 * The MFMA path takes stream-ordered scratch from the library's pool
 * (hipMallocFromPoolAsync / hipFreeAsync on `stream`) for the re-laid-out weights and, for
 * strided calls, the input's phase copy.  Validation happens before anything is
 * enqueued; errors leave y untouched and are reported by convtranspose_last_error().
 */
ct_status convolution_nd(ct_kernel kernel, ct_dtype dtype, int nsp, int channels_last, const void *x,
                         const int64_t *x_shape, const void *w, const int64_t *w_shape,
                         const void *bias, void *y, const int64_t *y_shape, ct_auto_pad auto_pad,
                         const int64_t *strides, const int64_t *dilations, const int64_t *pads,
                         const int64_t *kernel_shape, int64_t group, void *stream);

/*
 * Quantized transposed convolution with the QLinear scheme of the webgpu-kernels
 * "ai.onnx.QLinearConv" README (Description and Inputs table), which the pages give for the
 * forward convolution and which is applied here to the transposed one:
 *   acc[n, m, o] = bias[m] + sum over the scatter pairs (c, i, k) that reach o (the same
 *                  pairs as convtranspose_nd) of (x[n, c, i] - x_zero_point) *
 *                  (w[c, m', k] - w_zero_point[m]),        summed in int32 modulo 2^32
 *   y[n, m, o]   = saturate(round_half_even(float(acc) * mult[m]) + y_zero_point)
 *   mult[m]      = float(float(x_scale * w_scale[m]) / y_scale)
 * Readings where the pages are silent: the float32 order of the requantization above
 * (each step one IEEE float32 operation), rounding half to even, saturation to the range
 * of y's type, and the int32 accumulator wrapping modulo 2^32.
 *
 *   kernel          CT_KERNEL_AUTO (the int8 MFMA implicit GEMM when it serves the call:
 *                   C/group a multiple of 16 and C/group x taps of a phase below 2^17;
 *                   otherwise the gather kernel), CT_KERNEL_DIRECT (the gather kernel,
 *                   every call) or CT_KERNEL_IGEMM (CT_EUNSUPPORTED when it cannot serve);
 *                   other families fail with CT_EUNSUPPORTED
 *   x, x_type       device tensor of CT_UINT8 or CT_INT8, logical shape x_shape =
 *                   {N, C, D1..Dn}, layout as in convtranspose_nd (channels_last)
 *   x_scale, x_zero_point   per-tensor parameters of x (host values); x_scale must be
 *                   positive and finite, x_zero_point inside x_type's range
 *   w, w_type       device tensor {C, M/group, k1..kn} of CT_UINT8 or CT_INT8
 *   w_scale         device float32 array of wq_len values (positive and finite; not
 *                   checked: they stay on the device)
 *   w_zero_point    device array of wq_len values of w_type
 *   wq_len          1 (per tensor) or M (per output channel)
 *   bias            device int32 array of length M (scale x_scale * w_scale[m], zero
 *                   point 0), or NULL
 *   y, y_type       device tensor of CT_UINT8 or CT_INT8 with y_shape = the resolved
 *                   {N, M, O1..On}, in x's layout
 *   y_scale, y_zero_point   per-tensor parameters of y (host values), y_scale positive
 *                   and finite, y_zero_point inside y_type's range
 *   attributes and stream   as convtranspose_nd
 * Validation happens before anything is enqueued; errors leave y untouched.  The caller
 * owns every buffer; the MFMA path takes stream-ordered scratch from the library's pool
 * (hipMallocFromPoolAsync / hipFreeAsync on stream) for the packed weights, their channel sums, the input's channel
 * sums and, for channels-first tensors, channels-last copies of x and y.
 */
ct_status qlinear_convtranspose_nd(ct_kernel kernel, int nsp, int channels_last, const void *x, ct_dtype x_type,
                                   const int64_t *x_shape, float x_scale, int32_t x_zero_point, const void *w,
                                   ct_dtype w_type, const int64_t *w_shape, const float *w_scale,
                                   const void *w_zero_point, int64_t wq_len, const int32_t *bias, void *y,
                                   ct_dtype y_type, const int64_t *y_shape, float y_scale, int32_t y_zero_point,
                                   ct_auto_pad auto_pad, const int64_t *strides, const int64_t *dilations,
                                   const int64_t *pads, const int64_t *output_padding, const int64_t *output_shape,
                                   const int64_t *kernel_shape, int64_t group, void *stream);

/*
 * Tile configuration of the float16 implicit-GEMM (MFMA) kernel, a control for tests and
 * tuning (the pages leave the kernel's blocking to the implementation).  tile = -1
 * restores the automatic choice, the default: the largest tile that pads the output
 * channels little and still gives every compute unit a block.  tile = 0..4 forces one
 * block shape (output channels x output pixels): 0 = 256 x 256, 1 = 128 x 256,
 * 2 = 64 x 512, 3 = 64 x 256, 4 = 64 x 128 (the last two run two blocks per compute unit);
 * tile = 5 forces the all-phase kernel (64 output channels x every residue class of a
 * 4 x 32 box of the phase grid; strided calls with at least 4 residue classes and C/group
 * a multiple of 32), which the automatic choice takes for such calls when M/group <= 64;
 * tile = 6 forces the tap-split kernel (64 output channels x 64 consecutive output
 * positions, the taps split over the block's waves; stride 1 on every axis, C/group a
 * multiple of 32, at most 32 taps), which the automatic choice takes for 3-D stride-1
 * calls when M/group <= 64.  A forced tile that cannot serve a call (its input halo does not fit) makes an
 * implicit-GEMM call fail with CT_EUNSUPPORTED and CT_KERNEL_AUTO choose another kernel
 * family.  The setting is process-wide and is read when a call is made; changing it
 * while another host thread makes calls gives that thread either setting.
 * Returns CT_OK, or CT_EINVAL for a tile outside -1..6.
 */
ct_status convtranspose_set_igemm_tile(int tile);

/* The current setting of convtranspose_set_igemm_tile (-1: automatic). */
int convtranspose_igemm_tile(void);

/* Text of the last error on the calling host thread ("" after a successful call).
 * The pointer stays valid until the next library call on that thread. */
const char *convtranspose_last_error(void);

/* Short name of a ct_kernel value ("direct", "grouped", "igemm", ...). */
const char *convtranspose_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* CONVTRANSPOSE_H */
