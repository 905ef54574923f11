// ct_grouped.hip -- bandwidth kernel for grouped / depthwise transposed convolution.
//
// Grouped variant of the operator (webgpu-kernels "ai.onnx.ConvTranspose" README,
// Attributes: group; Implementation variants: a grouped stride-phase route where every
// gathered input sample feeds a block of the group's output channels and the group's
// weights are staged once per workgroup).  With few channels per group the work per
// output is a handful of taps, so the kernel is bound by HBM traffic, not arithmetic,
// and uses no MFMA.
//
// One block covers (image n, group g, output plane, band of output rows).  It stages
// the input rows that band reads, for the group's C/group channels and for every input
// plane the output plane's taps along the first axis read (rank 3), in LDS (zero columns
// added on both sides so no column test is needed), and the group's weights in LDS.
// Each thread then produces 8 consecutive outputs of one output row and one output
// channel: per axis the taps of a residue form an arithmetic progression
// (k = k0 + u*s/gcd(s,d), input i = j + beta0 - u*d/gcd(s,d)), fetched from small
// per-residue tables.  Accumulation is float32; the 8 results are rounded once and stored
// as one 16-byte vector where the row allows it.  Layout: NCHW-style (channels-first)
// only; spatial rank 1, 2 or 3.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "ct_internal.hpp"

namespace ct {
namespace {

constexpr int kGMaxRes = 16;      // largest stride per axis
constexpr int kGMaxTaps = 16;     // largest kernel size per axis
constexpr int kGLdsBytes = 48 * 1024;
constexpr int kGThreads = 256;
constexpr int kGBatch = 8;        // staged elements per thread in flight together

struct GArgs {
    int N, C, M, G, Cg, Mg;
    int L0, O0, K0, s0;
    int L1, L2, O1, O2, K1, K2;
    int s1, s2, b1, b2, d1, d2;
    int band;        // output rows per block
    int nbands;
    int pad2;        // zero columns staged left of input column 0
    int row_w;       // staged row width in elements
    int rows_max;    // staged input rows per channel and plane (capacity)
    int planes_max;  // staged input planes (the most taps of any residue on the first axis)
    // per residue: first tap, its input offset, tap count (progression steps below)
    short k0_1[kGMaxRes], be_1[kGMaxRes], nt_1[kGMaxRes];
    short k0_2[kGMaxRes], be_2[kGMaxRes], nt_2[kGMaxRes];
    short k0_0[kGMaxRes], be_0[kGMaxRes], nt_0[kGMaxRes];
    short ks0, ks1, ks2, bs0, bs1, bs2;
    Act act;  // output activation
};

__device__ __forceinline__ int fdiv(int a, int q) { return a >= 0 ? a / q : -((-a + q - 1) / q); }

template <typename T>
__global__ __launch_bounds__(kGThreads) void grouped_kernel(const T *__restrict__ x, const T *__restrict__ w,
                                                            const T *__restrict__ bias, T *__restrict__ y,
                                                            GArgs p)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[kGLdsBytes];
    T *const sx = reinterpret_cast<T *>(lds);

    int blk = blockIdx.x;
    const int band = blk % p.nbands;
    blk /= p.nbands;
    const int o0 = blk % p.O0;
    blk /= p.O0;
    const int g = blk % p.G;
    const int n = blk / p.G;
    const int oh0 = band * p.band;
    const int oh1 = min(oh0 + p.band, p.O1);
    // first axis: the output plane's residue, its taps and their input planes (planes
    // outside the input are staged as zeros)
    const int r0 = o0 % p.s0, j0 = o0 / p.s0;
    const int nt0 = p.nt_0[r0], k00 = p.k0_0[r0], be0 = p.be_0[r0];

    // input rows this band reads: i = (o + b - k d) / s over o in [oh0, oh1), k in [0, K)
    const int ilo = max(0, fdiv(oh0 + p.b1 - (p.K1 - 1) * p.d1 + p.s1 - 1, p.s1));
    const int ihi = min(p.L1 - 1, fdiv(oh1 - 1 + p.b1, p.s1));
    const int nrows = max(0, ihi - ilo + 1);
    const int rw = p.row_w;

    // stage rows [ilo, ihi] of the group's channels for each tap plane, zero-padded on
    // both sides: slot (u0, c) holds channel c of input plane j0 + be0 - u0 * bs0
    const size_t plane = size_t(p.L1) * p.L2;
    const size_t vol = size_t(p.L0) * plane;
    const int per_ch = p.rows_max * rw;
    float *const sw = reinterpret_cast<float *>(lds + size_t(p.planes_max) * p.Cg * per_ch * sizeof(T));
    const int ntaps = p.K0 * p.K1 * p.K2;
    const int ntaps12 = p.K1 * p.K2;
    for (int u = threadIdx.x; u < p.Cg * p.Mg * ntaps; u += kGThreads)
        sw[u] = float(w[size_t(g) * p.Cg * p.Mg * ntaps + u]);
    const int per_slot = nrows * rw;
    // rounds of kGBatch elements per thread: unconditional loads (element 0 of x when the
    // slot is padding), all in flight before any is written
    const int nstage = nt0 * p.Cg * per_slot;
    const UDiv dslot(per_slot), dcg(p.Cg), drw(rw);  // index splits by multiply-high
    const T *const xg = x + (size_t(n) * p.C + size_t(g) * p.Cg) * vol;
    for (int base = 0; base < nstage; base += kGThreads * kGBatch) {
        T v[kGBatch];
        unsigned okm = 0;
#pragma unroll
        for (int k = 0; k < kGBatch; ++k) {
            const int u = base + threadIdx.x + k * kGThreads;
            const int sl = dslot.div(u);  // slot = u0 * Cg + c
            const int rem = u - sl * per_slot;
            const int u0 = dcg.div(sl), c = sl - u0 * p.Cg;
            const int r = drw.div(rem), col = rem - r * rw;
            const int i2 = col - p.pad2;
            const int i0 = j0 + be0 - u0 * p.bs0;
            const bool ok = u < nstage && i2 >= 0 && i2 < p.L2 && i0 >= 0 && i0 < p.L0;
            v[k] = *(ok ? xg + (size_t(c) * vol + size_t(i0) * plane + size_t(ilo + r) * p.L2 + i2) : x);
            okm |= unsigned(ok) << k;
        }
#pragma unroll
        for (int k = 0; k < kGBatch; ++k) {
            const int u = base + threadIdx.x + k * kGThreads;
            if (u < nstage) {
                const int sl = dslot.div(u);
                const int rem = u - sl * per_slot;
                const int r = drw.div(rem), col = rem - r * rw;
                sx[sl * per_ch + r * rw + col] = ((okm >> k) & 1u) ? v[k] : T(0.0f);
            }
        }
    }
    __syncthreads();

    // work items: (output channel in group, output row, 8-column segment)
    const int segs = (p.O2 + 7) / 8;
    const int items = p.Mg * (oh1 - oh0) * segs;
    for (int it = threadIdx.x; it < items; it += kGThreads) {
        const int seg = it % segs;
        const int rest = it / segs;
        const int oh = oh0 + rest % (oh1 - oh0);
        const int mm = rest / (oh1 - oh0);
        const int ow0 = seg * 8;
        float acc[8];
        const float bv = bias ? float(bias[g * p.Mg + mm]) : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = bv;
        // taps along rows for this output row
        const int r1 = oh % p.s1;
        const int j1 = oh / p.s1;
        const int nt1 = p.nt_1[r1];
        const int k01 = p.k0_1[r1];
        const int be1 = p.be_1[r1];
        // per output column: its residue's tap count, first input column and first tap
        // (looked up once per item, outside the channel and tap loops)
        int nt2e[8], i2e[8], k2e[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ow = ow0 + e;
            const int r2 = ow % p.s2;
            nt2e[e] = p.nt_2[r2];
            i2e[e] = ow / p.s2 + p.be_2[r2];
            k2e[e] = p.k0_2[r2];
        }
        for (int c = 0; c < p.Cg; ++c)
        for (int u0 = 0; u0 < nt0; ++u0) {
            const T *xc = sx + (u0 * p.Cg + c) * per_ch;
            const float *wc = sw + (c * p.Mg + mm) * ntaps + (k00 + u0 * p.ks0) * ntaps12;
            for (int u1 = 0; u1 < nt1; ++u1) {
                const int i1 = j1 + be1 - u1 * p.bs1;
                if (i1 < ilo || i1 > ihi) continue;
                const T *xr = xc + (i1 - ilo) * rw + p.pad2;
                const float *wr = wc + (k01 + u1 * p.ks1) * p.K2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    for (int u2 = 0; u2 < nt2e[e]; ++u2) {
                        // columns out of [0, L2) read the staged zero padding
                        acc[e] += float(xr[i2e[e] - u2 * p.bs2]) * wr[k2e[e] + u2 * p.ks2];
                    }
                }
            }
        }
        if (!p.act.identity()) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = p.act(acc[e]);
        }
        T *yr = y + (((size_t(n) * p.M + size_t(g) * p.Mg + mm) * p.O0 + o0) * p.O1 + oh) * p.O2 + ow0;
        const bool full = ow0 + 8 <= p.O2;
        if (sizeof(T) == 2 && full && (reinterpret_cast<uintptr_t>(yr) % 16 == 0)) {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const unsigned lo = __builtin_bit_cast(unsigned short, _Float16(acc[2 * k]));
                const unsigned hi = __builtin_bit_cast(unsigned short, _Float16(acc[2 * k + 1]));
                o[k] = lo | (hi << 16);
            }
            *reinterpret_cast<u32x4 *>(yr) = o;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (ow0 + e < p.O2) yr[e] = T(acc[e]);
        }
    }
}

struct GPlan {
    GArgs a;
    int blocks;
};

bool make_gplan(const Geom &g, size_t esz, GPlan *pl, std::string *why)
{
    auto no = [&](const char *m) {
        *why = m;
        return false;
    };
    if (g.s[0] > kGMaxRes || g.s[1] > kGMaxRes || g.s[2] > kGMaxRes) return no("stride too large");
    if (g.K[0] > kGMaxTaps || g.K[1] > kGMaxTaps || g.K[2] > kGMaxTaps) return no("kernel too large");
    GArgs &a = pl->a;
    std::memset(&a, 0, sizeof(a));
    a.N = int(g.N);
    a.C = int(g.C);
    a.M = int(g.M);
    a.G = int(g.G);
    a.Cg = int(g.Cg);
    a.Mg = int(g.Mg);
    a.L0 = int(g.L[0]);
    a.O0 = int(g.O[0]);
    a.K0 = int(g.K[0]);
    a.s0 = int(g.s[0]);
    a.L1 = int(g.L[1]);
    a.L2 = int(g.L[2]);
    a.O1 = int(g.O[1]);
    a.O2 = int(g.O[2]);
    a.K1 = int(g.K[1]);
    a.K2 = int(g.K[2]);
    a.s1 = int(g.s[1]);
    a.s2 = int(g.s[2]);
    a.b1 = int(g.b[1]);
    a.b2 = int(g.b[2]);
    a.d1 = int(g.d[1]);
    a.d2 = int(g.d[2]);
    const int64_t gs0 = std::__gcd(g.s[0], g.d[0]);
    a.ks0 = short(g.s[0] / gs0);
    a.bs0 = short(g.d[0] / gs0);
    const int64_t gs1 = std::__gcd(g.s[1], g.d[1]), gs2 = std::__gcd(g.s[2], g.d[2]);
    a.ks1 = short(g.s[1] / gs1);
    a.bs1 = short(g.d[1] / gs1);
    a.ks2 = short(g.s[2] / gs2);
    a.bs2 = short(g.d[2] / gs2);
    int bemin2 = 0, bemax2 = 0;
    bool first = true;
    int planes = 1;
    for (int ax = 0; ax <= 2; ++ax)
        for (int r = 0; r < g.s[ax]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, ax, r, &ph)) return no("too many taps");
            short *k0 = ax == 0 ? a.k0_0 : ax == 1 ? a.k0_1 : a.k0_2;
            short *be = ax == 0 ? a.be_0 : ax == 1 ? a.be_1 : a.be_2;
            short *nt = ax == 0 ? a.nt_0 : ax == 1 ? a.nt_1 : a.nt_2;
            if (ax == 0) planes = std::max(planes, ph.ntaps);
            k0[r] = short(ph.ntaps ? ph.k[0] : 0);
            be[r] = short(ph.ntaps ? ph.beta[0] : 0);
            nt[r] = short(ph.ntaps);
            if (ax == 2 && ph.ntaps) {
                const int hi = ph.beta[0], lo = ph.beta[ph.ntaps - 1];
                bemin2 = first ? lo : std::min(bemin2, lo);
                bemax2 = first ? hi : std::max(bemax2, hi);
                first = false;
            }
        }
    // staged columns: i2 = j2 + beta ranges over [beta_min, (O2-1)/s2 + beta_max]
    const int jmax2 = int((g.O[2] - 1) / g.s[2]) + 7;  // +7: a segment may run past O2
    a.pad2 = std::max(0, -bemin2);
    const int right = std::max<int>(int(g.L[2]), jmax2 + bemax2 + 1);
    a.row_w = (a.pad2 + right + 7) / 8 * 8;
    // rows per band: the staged rows of Cg channels in every tap plane plus the group's
    // weights fit in LDS
    a.planes_max = planes;
    const int64_t wbytes = int64_t(g.Cg) * g.Mg * g.K[0] * g.K[1] * g.K[2] * 4;
    const int64_t per_row = int64_t(planes) * g.Cg * a.row_w * int64_t(esz);
    if (wbytes + per_row * 2 > kGLdsBytes) return no("group does not fit in LDS");
    const int rows_cap = int((kGLdsBytes - wbytes) / per_row);
    // a band of B output rows reads at most (B - 1 + (K1-1)*d1) / s1 + 2 input rows
    int bandrows = int(g.O[1]);
    while (bandrows > 1 && ((bandrows - 1 + (g.K[1] - 1) * g.d[1]) / g.s[1] + 2) > rows_cap) bandrows = (bandrows + 1) / 2;
    if (((bandrows - 1 + (g.K[1] - 1) * g.d[1]) / g.s[1] + 2) > rows_cap) return no("rows do not fit in LDS");
    a.band = bandrows;
    a.nbands = int((g.O[1] + bandrows - 1) / bandrows);
    a.rows_max = int(std::min<int64_t>(rows_cap, g.L[1] > 0 ? g.L[1] : 1));
    const int64_t blocks = g.N * g.G * g.O[0] * a.nbands;
    if (blocks <= 0 || blocks > (1ll << 31) - 1) return no("grid size");
    pl->blocks = int(blocks);
    return true;
}

}  // namespace

bool grouped_supports(const Geom &g, ct_dtype dt, bool cl, const void *x)
{
    if (g.G >= 2 && dwcl_supports(g, dt, cl, x)) return true;
    if (cl || g.G < 2 || g.Cg > 8 || g.Mg > 8 || g.x_elems() <= 0) return false;
    if (depthwise_supports(g, dt, cl, x)) return true;
    GPlan pl;
    std::string why;
    return make_gplan(g, dt == CT_FLOAT16 ? 2 : 4, &pl, &why);
}

ct_status launch_grouped(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w, const void *bias,
                         void *y, const Act &act, hipStream_t st, std::string *err)
{
    if (!grouped_supports(g, dt, cl, x)) {
        *err = "grouped kernel cannot serve this call";
        return CT_EUNSUPPORTED;
    }
    if (depthwise_supports(g, dt, cl, x)) return launch_depthwise(g, dt, cl, x, w, bias, y, act, st, err);
    if (dwcl_supports(g, dt, cl, x)) return launch_dwcl(g, x, w, bias, y, act, st, err);
    GPlan pl;
    if (!make_gplan(g, dt == CT_FLOAT16 ? 2 : 4, &pl, err)) return CT_EUNSUPPORTED;
    pl.a.act = act;
    mark_before(st);
    if (dt == CT_FLOAT16)
        hipLaunchKernelGGL(grouped_kernel<_Float16>, dim3(unsigned(pl.blocks)), dim3(kGThreads), 0, st,
                           static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w),
                           static_cast<const _Float16 *>(bias), static_cast<_Float16 *>(y), pl.a);
    else
        hipLaunchKernelGGL(grouped_kernel<float>, dim3(unsigned(pl.blocks)), dim3(kGThreads), 0, st,
                           static_cast<const float *>(x), static_cast<const float *>(w),
                           static_cast<const float *>(bias), static_cast<float *>(y), pl.a);
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("grouped kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
