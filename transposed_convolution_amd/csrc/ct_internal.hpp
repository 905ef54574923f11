// ct_internal.hpp -- host-side geometry, stride-phase plan and kernel launch
// declarations shared by the library's translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <string>

#include "convtranspose.h"

namespace ct {

// Every problem is carried as 3 spatial axes: a rank-n problem puts its axes last and
// fills the leading ones with a unit axis (L = K = s = d = O = 1, no pads), which adds
// exactly one tap and one output position and changes nothing else.
constexpr int kAxes = 3;

// Workgroup b of a launch goes to XCD b % 8 (8 XCDs, each with its own L2); xcd_remap
// gives the workgroups of each XCD a contiguous range of the nb work indices, so the
// data neighbouring work items share stays in one L2.
__device__ __forceinline__ int xcd_remap(int b, int nb)
{
    const int q = nb >> 3, rem = nb & 7, x = b & 7, k = b >> 3;
    return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}

// Division of a non-negative int u by a wave-uniform divisor d >= 1 with one
// multiply-high instead of the GPU's long integer-division sequence: with
// m = ceil(2^32 / d), (u * m) >> 32 = floor(u / d) exactly while u * d < 2^32 (the
// rounding error of m adds less than 1/d to u / d).  Callers keep u * d below 2^32.
struct UDiv {
    unsigned m;
    int d;
    __device__ __forceinline__ explicit UDiv(int dv) : m(dv > 1 ? unsigned(0xffffffffu / unsigned(dv)) + 1u : 0u), d(dv) {}
    __device__ __forceinline__ int div(int u) const { return d > 1 ? int(__umulhi(unsigned(u), m)) : u; }
    __device__ __forceinline__ int mod(int u) const { return u - div(u) * d; }
};

// Resolved problem geometry (ONNX attribute table applied; README "Attributes").
struct Geom {
    int nsp = 0;                                  // rank as given (1..3)
    int64_t N = 0, C = 0, M = 0, G = 1, Cg = 0, Mg = 0;
    int64_t L[kAxes], K[kAxes], s[kAxes], d[kAxes], b[kAxes], e[kAxes], op[kAxes], O[kAxes];

    int64_t in_pixels() const { return L[0] * L[1] * L[2]; }
    int64_t out_pixels() const { return O[0] * O[1] * O[2]; }
    int64_t taps() const { return K[0] * K[1] * K[2]; }
    int64_t x_elems() const { return N * C * in_pixels(); }
    int64_t w_elems() const { return C * Mg * taps(); }
    int64_t y_elems() const { return N * M * out_pixels(); }
};

struct Attrs {
    ct_auto_pad auto_pad = CT_NOTSET;
    const int64_t *strides = nullptr, *dilations = nullptr, *pads = nullptr;
    const int64_t *output_padding = nullptr, *output_shape = nullptr, *kernel_shape = nullptr;
    int64_t group = 1;
};

// Defaults, validation, derived pads and output sizes.  Returns CT_OK or CT_EINVAL
// (message in *err).
ct_status resolve(int nsp, const int64_t *x_shape, const int64_t *w_shape, const Attrs &at,
                  Geom *g, std::string *err);

// Useful MACs: per axis the (i, k) pairs landing in [0, O), counted in closed form.
double useful_macs(const Geom &g);

// --- stride-phase (sub-pixel) decomposition of one axis --------------------------
// Output positions o with o % s == r form phase r: o = r + s*j, j in [0, J).  Such an
// output receives tap k exactly when (r + b - k*d) is a multiple of s, from input
// i = j + beta_k with beta_k = (r + b - k*d) / s.  Taps are listed by ascending k.
constexpr int kMaxPhaseTaps = 16;
struct AxisPhase {
    int r = 0;          // first output of the phase
    int J = 0;          // outputs in the phase
    int ntaps = 0;      // taps reaching the phase (0: only bias lands here)
    int k[kMaxPhaseTaps];
    int beta[kMaxPhaseTaps];
};
// Fills phase r of axis a; returns false when the phase has more than kMaxPhaseTaps taps.
bool axis_phase(const Geom &g, int a, int r, AxisPhase *ph);

// Stream-ordered scratch (hipMallocFromPoolAsync on st) from a memory pool the library
// creates per device on first use and keeps to the end of the process; its release
// threshold keeps freed scratch in the pool for the next call instead of unmapping and
// mapping it again.  Release with hipFreeAsync on the same stream.
hipError_t scratch_malloc(void **p, size_t bytes, hipStream_t st);

// The per-thread error text convtranspose_last_error() returns.
void set_last_error(const std::string &msg);

// Enum arguments come from C callers as plain ints and may hold any value, while C++ code
// may assume that an enum object holds one of its type's values.  Entry points therefore
// read each enum argument's int value without loading it as the enum (enum_int) and
// refuse values outside the enum (check_enum_args) before using the argument.
template <class E>
inline int enum_int(const E &v)
{
    static_assert(sizeof(E) == sizeof(int), "the C enums of the ABI are int-sized");
    int r;
    std::memcpy(&r, &v, sizeof r);
    return r;
}
struct EnumArgs {
    int kernel = CT_KERNEL_AUTO, dtype = CT_FLOAT32, auto_pad = CT_NOTSET, activation = CT_ACT_IDENTITY;
};
// CT_OK, or CT_EUNSUPPORTED for an unknown element type and CT_EINVAL for another
// unknown enum value (message in *err).
inline ct_status check_enum_args(const EnumArgs &e, std::string *err)
{
    if (e.dtype < CT_FLOAT32 || e.dtype > CT_UINT8) {
        *err = "unknown element type";
        return CT_EUNSUPPORTED;
    }
    if (e.auto_pad < CT_NOTSET || e.auto_pad > CT_VALID) {
        *err = "auto_pad must be NOTSET, SAME_UPPER, SAME_LOWER or VALID";
        return CT_EINVAL;
    }
    if (e.kernel < CT_KERNEL_AUTO || e.kernel > CT_KERNEL_NONE) {
        *err = "unknown kernel family";
        return CT_EINVAL;
    }
    if (e.activation < CT_ACT_IDENTITY || e.activation > CT_ACT_CLIP) {
        *err = "unknown activation";
        return CT_EINVAL;
    }
    return CT_OK;
}

// Events the caller asked to have recorded around the dominant kernel of each call on
// this host thread (both null: none).
struct ProfileEvents {
    hipEvent_t before = nullptr, after = nullptr;
};
ProfileEvents &profile_events();
inline void mark_before(hipStream_t st)
{
    if (profile_events().before) (void)hipEventRecord(profile_events().before, st);
}
inline void mark_after(hipStream_t st)
{
    if (profile_events().after) (void)hipEventRecord(profile_events().after, st);
}

// Activation of the output stage (see ct_activation in convtranspose.h), evaluated in
// float32 on the accumulated value plus bias, before the one rounding.
struct Act {
    int kind = CT_ACT_IDENTITY;
    float p0 = 0.0f, p1 = 0.0f;
    __host__ __device__ bool identity() const { return kind == CT_ACT_IDENTITY; }
    // Every candidate is formed and one selected: with a block-uniform kind this is a few
    // selects per element and no branches (a switch here became per-element branches).
    // Hot output loops test identity() once and skip the call.
    __host__ __device__ float operator()(float v) const
    {
        const float relu = v > 0.0f ? v : 0.0f;
        const float leaky = v >= 0.0f ? v : p0 * v;
        const float clip = v < p0 ? p0 : (v > p1 ? p1 : v);
        return kind == CT_ACT_RELU ? relu : kind == CT_ACT_LEAKY_RELU ? leaky : kind == CT_ACT_CLIP ? clip : v;
    }
};

// Calls f(fn) with fn the activation as a branch-free float -> float function, one
// instance per kind: output loops written inside f then carry no per-element dispatch.
template <typename F>
__device__ __forceinline__ void with_activation(const Act &a, F &&f)
{
    switch (a.kind) {
    case CT_ACT_RELU: f([](float v) { return v > 0.0f ? v : 0.0f; }); break;
    case CT_ACT_LEAKY_RELU: {
        const float slope = a.p0;
        f([slope](float v) { return v >= 0.0f ? v : slope * v; });
        break;
    }
    case CT_ACT_CLIP: {
        const float lo = a.p0, hi = a.p1;
        f([lo, hi](float v) { return v < lo ? lo : (v > hi ? hi : v); });
        break;
    }
    default: f([](float v) { return v; }); break;
    }
}

// Requantization of the quantized operation (QLinear scheme): the multiplier
// float(float(x_scale * w_scale) / y_scale) and saturate(round_half_even(float(acc) *
// mult) + y_zp), each step one IEEE float32 operation (no contraction; '/' is the
// correctly rounded divide).  acc is the int32 accumulator as its 32-bit pattern.
__device__ __forceinline__ float requant_mult(float x_scale, float w_scale, float y_scale)
{
#pragma clang fp contract(off)
    const float xw = x_scale * w_scale;
    return xw / y_scale;
}

__device__ __forceinline__ int requantize(unsigned acc, float mult, int y_zp, int y_lo, int y_hi)
{
#pragma clang fp contract(off)
    const float v = float(__builtin_bit_cast(int, acc)) * mult;
    const float r = rintf(v);  // to nearest, ties to even
    // saturate before converting (r may be far outside the int range)
    const float lo = float(y_lo - y_zp), hi = float(y_hi - y_zp);
    const float c = r < lo ? lo : (r > hi ? hi : r);
    return int(c) + y_zp;
}

// The quantized operation's parameters (see qlinear_convtranspose_nd).
struct QuantCall {
    ct_dtype x_type, w_type, y_type;
    float x_scale, y_scale;
    int x_zp, y_zp;
    const float *w_scale;
    const void *w_zp;
    int64_t wq_len;
    const int *bias;
};
// The quantized operation on the int8 MFMA implicit GEMM (channels-last only).
bool qigemm_supports(const Geom &g, bool cl, const void *x, std::string *why);
ct_status launch_qigemm(const Geom &g, bool cl, const void *x, const void *w, void *y, const QuantCall &qc,
                        hipStream_t st, std::string *err);

// Launchers (one per kernel family); each returns CT_OK or CT_EDEVICE (message in err).
ct_status launch_direct(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w,
                        const void *bias, void *y, const Act &act, hipStream_t st, std::string *err);
bool grouped_supports(const Geom &g, ct_dtype dt, bool cl, const void *x);
// Depthwise specialisation inside the grouped family (one channel in and out per group,
// float16, channels-first, equal strides 1, 2 or 4, tap runs of step 1).
bool depthwise_supports(const Geom &g, ct_dtype dt, bool cl, const void *x);
ct_status launch_depthwise(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w,
                           const void *bias, void *y, const Act &act, hipStream_t st, std::string *err);
ct_status launch_grouped(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w,
                         const void *bias, void *y, const Act &act, hipStream_t st, std::string *err);
// Channels-last depthwise specialisation inside the grouped family (float16, one channel
// in and out per group, C a multiple of 8, spatial rank 1 or 2, strides up to 2).
bool dwcl_supports(const Geom &g, ct_dtype dt, bool cl, const void *x);
ct_status launch_dwcl(const Geom &g, const void *x, const void *w, const void *bias, void *y, const Act &act,
                      hipStream_t st, std::string *err);
bool igemm_supports(const Geom &g, ct_dtype dt, bool cl, const void *x, std::string *why);
size_t igemm_workspace_bytes(const Geom &g, ct_dtype dt);
// Tile configurations of the float16 implicit-GEMM kernel: how many there are, and a
// process-wide override (-1: automatic choice).
int igemm_tile_count();
void igemm_force_tile(int tile);
int igemm_forced_tile();
// float32 implicit GEMM on MFMA (the CT_KERNEL_IGEMM family for float32 inputs)
bool igemm32_supports(const Geom &g, bool cl, std::string *why);
ct_status launch_igemm32(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                         const Act &act, hipStream_t st, std::string *err);
// The all-phase kernel (ct_mphase.hip): strided calls with at least 4 residue classes,
// C/group a multiple of 32; preferred when M/group <= 64.  Its packed weights are the
// fragment-major packing of 64-channel tiles.
bool mphase_supports(const Geom &g, bool cl, std::string *why);
size_t mphase_workspace_bytes(const Geom &g, bool cl);
ct_status launch_mphase(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                        const Act &act, void *wsp, size_t ws_bytes, hipStream_t st, std::string *err, bool w_conv);
// The tap-split kernel (ct_tapsplit.hip): stride 1 on every axis, C/group a multiple of
// 32, at most 32 taps, the input window of a 64-position box in LDS; preferred for 3-D
// calls with M/group <= 64.  Its packed weights are the fragment-major packing.
bool tapsplit_supports(const Geom &g, bool cl, std::string *why);
size_t tapsplit_workspace_bytes(const Geom &g, bool cl);
ct_status launch_tapsplit(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                          const Act &act, void *wsp, size_t ws_bytes, hipStream_t st, std::string *err, bool w_conv);
// W (or a forward convolution's W, taps reversed) into the fragment-major packing with
// Cgp input and Mgp output channels per group (zero padded).
ct_status launch_pack_w_frag(const Geom &g, const void *w, void *wp, int Cgp, int Mgp, bool w_conv, hipStream_t st,
                             std::string *err);
// workspace: caller scratch of ws_bytes (>= igemm_workspace_bytes), or NULL to take
// stream-ordered scratch from the library pool (scratch_malloc / hipFreeAsync on st).  w_conv (float16
// only): w is a forward convolution's weight (M, C/group, k) and g the stride-1
// transposed convolution that equals that convolution; it is read with reversed taps.
ct_status launch_igemm(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w,
                       const void *bias, void *y, const Act &act, void *workspace, size_t ws_bytes,
                       hipStream_t st, std::string *err, bool w_conv = false);

}  // namespace ct
