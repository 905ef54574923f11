// ct_grouped.hip -- bandwidth kernel for grouped / depthwise transposed convolution.
//
// Grouped variant of the operator (webgpu-kernels "ai.onnx.ConvTranspose" README,
// Attributes: group; Implementation variants: a grouped stride-phase route where every
// gathered input sample feeds a block of the group's output channels and the group's
// weights are staged once per workgroup).  With few channels per group the work per
// output is a handful of taps, so the kernel is bound by HBM traffic, not arithmetic,
// and uses no MFMA.
//
// One block covers (image n, group g, band of output rows).  It stages the input rows
// that band reads, for the group's C/group channels, in LDS (zero columns added on both
// sides so no column test is needed), and the group's weights in LDS.  Each thread then
// produces 8 consecutive outputs of one output row and one output channel: per output
// column the taps form an arithmetic progression (k = k0 + u*s/gcd(s,d), input
// i = j + beta0 - u*d/gcd(s,d)), fetched from small per-residue tables.  Accumulation is
// float32; the 8 results are rounded once and stored as one 16-byte vector where the
// row allows it.  Layout: NCHW-style (channels-first) only; spatial rank 1 or 2.
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
constexpr int kDwChunks = 8;                            // 16-byte staging chunks per thread
constexpr int kDwLdsBytes = kDwChunks * kGThreads * 16;  // depthwise staged band

struct GArgs {
    int N, C, M, G, Cg, Mg;
    int L1, L2, O1, O2, K1, K2;
    int s1, s2, b1, b2, d1, d2;
    int band;        // output rows per block
    int nbands;
    int pad2;        // zero columns staged left of input column 0
    int row_w;       // staged row width in elements
    int rows_max;    // staged input rows per channel (capacity)
    // per residue: first tap, its input offset, tap count (progression steps below)
    short k0_1[kGMaxRes], be_1[kGMaxRes], nt_1[kGMaxRes];
    short k0_2[kGMaxRes], be_2[kGMaxRes], nt_2[kGMaxRes];
    short ks1, ks2, bs1, bs2;
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
    const int g = blk % p.G;
    const int n = blk / p.G;
    const int oh0 = band * p.band;
    const int oh1 = min(oh0 + p.band, p.O1);

    // input rows this band reads: i = (o + b - k d) / s over o in [oh0, oh1), k in [0, K)
    const int ilo = max(0, fdiv(oh0 + p.b1 - (p.K1 - 1) * p.d1 + p.s1 - 1, p.s1));
    const int ihi = min(p.L1 - 1, fdiv(oh1 - 1 + p.b1, p.s1));
    const int nrows = max(0, ihi - ilo + 1);
    const int rw = p.row_w;

    // stage rows [ilo, ihi] of the group's channels, zero-padded on both sides
    const size_t plane = size_t(p.L1) * p.L2;
    const int per_ch = p.rows_max * rw;
    float *const sw = reinterpret_cast<float *>(lds + size_t(p.Cg) * per_ch * sizeof(T));
    const int ntaps = p.K1 * p.K2;
    for (int u = threadIdx.x; u < p.Cg * p.Mg * ntaps; u += kGThreads)
        sw[u] = float(w[size_t(g) * p.Cg * p.Mg * ntaps + u]);
    for (int u = threadIdx.x; u < p.Cg * nrows * rw; u += kGThreads) {
        const int c = u / (nrows * rw);
        const int rem = u - c * nrows * rw;
        const int r = rem / rw, col = rem - r * rw;
        const int i2 = col - p.pad2;
        T v = T(0.0f);
        if (i2 >= 0 && i2 < p.L2)
            v = x[(size_t(n) * p.C + size_t(g) * p.Cg + c) * plane + size_t(ilo + r) * p.L2 + i2];
        sx[c * per_ch + r * rw + col] = v;
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
        for (int c = 0; c < p.Cg; ++c) {
            const T *xc = sx + c * per_ch;
            const float *wc = sw + (c * p.Mg + mm) * ntaps;
            for (int u1 = 0; u1 < nt1; ++u1) {
                const int i1 = j1 + be1 - u1 * p.bs1;
                if (i1 < ilo || i1 > ihi) continue;
                const T *xr = xc + (i1 - ilo) * rw + p.pad2;
                const float *wr = wc + (k01 + u1 * p.ks1) * p.K2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ow = ow0 + e;
                    const int r2 = ow % p.s2;
                    const int j2 = ow / p.s2;
                    const int nt2 = p.nt_2[r2];
                    const int k02 = p.k0_2[r2];
                    const int be2 = p.be_2[r2];
                    for (int u2 = 0; u2 < nt2; ++u2) {
                        // columns out of [0, L2) read the staged zero padding
                        const int i2 = j2 + be2 - u2 * p.bs2;
                        acc[e] += float(xr[i2]) * wr[k02 + u2 * p.ks2];
                    }
                }
            }
        }
        T *yr = y + ((size_t(n) * p.M + size_t(g) * p.Mg + mm) * p.O1 + oh) * p.O2 + ow0;
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

// Depthwise fast path (one input and one output channel per group, equal stride S on
// both axes).  Output pixel (S*j1 + rh, S*j2 + rw) reads inputs (j1 + wlo1 + a,
// j2 + wlo2 + c) for a < RW, c < CW through an effective kernel E[rh][rw][a][c] that
// holds W's tap for that offset or 0 -- a small dense correlation per phase pair, so
// every loop bound and register index below is a compile-time constant.  A thread makes
// S output rows x 8 output columns from one register window of inputs.
template <int S, int RW, int CW, bool VEC>
__global__ __launch_bounds__(kGThreads) void depthwise_kernel(const _Float16 *__restrict__ x,
                                                              const _Float16 *__restrict__ w,
                                                              const _Float16 *__restrict__ bias,
                                                              _Float16 *__restrict__ y, GArgs p, int wlo1, int wlo2)
{
    constexpr int OC = 8;                  // output columns per thread
    constexpr int JC = OC / S;             // input-grid columns they span
    constexpr int XW = JC + CW - 1;        // register window width
    extern __shared__ __attribute__((aligned(16))) unsigned char dw_lds[];  // staged rows, sized at launch
    _Float16 *const sx = reinterpret_cast<_Float16 *>(dw_lds);
    __shared__ float seff[S][S][RW][CW];

    int blk = blockIdx.x;
    const int band = blk % p.nbands;
    const int c = blk / p.nbands;  // plane index n * C + channel
    const int ch = c % p.C;
    const int oh0 = band * p.band;
    const int oh1 = min(oh0 + p.band, p.O1);
    const int j1lo = oh0 / S, j1hi = (oh1 - 1) / S;  // input-grid rows of the band
    // staged input rows: [j1lo + wlo1, j1hi + wlo1 + RW - 1]
    const int ilo = j1lo + wlo1;
    const int nrows = (j1hi - j1lo) + RW;
    const int rw_ = p.row_w;

    // one effective-kernel entry per thread (S*S*RW*CW <= 256): tap k with
    // rh + b - k d == (wlo + a) S on each axis, else 0
    static_assert(S * S * RW * CW <= kGThreads, "effective kernel larger than the block");
    float ev = 0.0f;
    {
        const int u = threadIdx.x;
        const int cc = u % CW, a = (u / CW) % RW, rwp = (u / (CW * RW)) % S, rhp = u / (CW * RW * S);
        const int t1 = rhp + p.b1 - (wlo1 + a) * S, t2 = rwp + p.b2 - (wlo2 + cc) * S;
        const bool ok = u < S * S * RW * CW && t1 >= 0 && t1 % p.d1 == 0 && t1 / p.d1 < p.K1 && t2 >= 0 &&
                        t2 % p.d2 == 0 && t2 / p.d2 < p.K2;
        const float t = float(w[size_t(ch) * p.K1 * p.K2 + (ok ? (t1 / p.d1) * p.K2 + t2 / p.d2 : 0)]);
        ev = ok ? t : 0.0f;
    }
    const size_t plane = size_t(p.L1) * p.L2;
    const _Float16 *xp = x + size_t(c) * plane;
    const _Float16 braw = *(bias ? bias + ch : xp);  // unconditional; used only with a bias
    if (VEC) {
        // 16-byte chunks: with L2 and pad2 multiples of 8 a chunk is wholly inside the
        // row or wholly padding.  Every load is issued before the first LDS write.
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const int cpr = rw_ / 8, nch = nrows * cpr;
        u32x4 v[kDwChunks];
#pragma unroll
        for (int q = 0; q < kDwChunks; ++q) {
            const int u = threadIdx.x + q * kGThreads;
            const int r = u / cpr, i2 = (u - r * cpr) * 8 - p.pad2, i1 = ilo + r;
            // unconditional load from a clamped address, masked afterwards: no branch
            // splits the batch, so all loads stay in flight together
            const bool ok = u < nch && i1 >= 0 && i1 < p.L1 && i2 >= 0 && i2 < p.L2;
            const u32x4 t = *reinterpret_cast<const u32x4 *>(xp + (ok ? size_t(i1) * p.L2 + i2 : 0));
            const unsigned m = ok ? ~0u : 0u;
            v[q] = u32x4{t[0] & m, t[1] & m, t[2] & m, t[3] & m};
        }
#pragma unroll
        for (int q = 0; q < kDwChunks; ++q) {
            const int u = threadIdx.x + q * kGThreads;
            if (u < nch) reinterpret_cast<u32x4 *>(sx)[u] = v[q];
        }
    } else {
        const int n_el = nrows * rw_;
        for (int u0 = 0; u0 < n_el; u0 += 8 * kGThreads) {
            _Float16 v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int u = u0 + threadIdx.x + q * kGThreads;
                const int r = u / rw_, i1 = ilo + r, i2 = u - r * rw_ - p.pad2;
                const bool ok = u < n_el && i1 >= 0 && i1 < p.L1 && i2 >= 0 && i2 < p.L2;
                const _Float16 t = xp[ok ? size_t(i1) * p.L2 + i2 : 0];
                v[q] = ok ? t : _Float16(0.0f);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int u = u0 + threadIdx.x + q * kGThreads;
                if (u < n_el) sx[u] = v[q];
            }
        }
    }
    if (threadIdx.x < S * S * RW * CW) (&seff[0][0][0][0])[threadIdx.x] = ev;
    __syncthreads();
    const float bv = bias ? float(braw) : 0.0f;

    float eff[S][S][RW][CW];
#pragma unroll
    for (int i = 0; i < S * S * RW * CW; ++i) (&eff[0][0][0][0])[i] = (&seff[0][0][0][0])[i];
    const int segs = (p.O2 + OC - 1) / OC;
    const int jrows = j1hi - j1lo + 1;
    for (int it = threadIdx.x; it < jrows * segs; it += kGThreads) {
        const int seg = it % segs, jr = it / segs;
        const int j1 = j1lo + jr;
        const int j2 = seg * JC;
        // input window: rows jr .. jr+RW-1 of the stage, columns j2 + wlo2 .. + XW - 1
        float xin[RW][XW];
        const _Float16 *base = sx + jr * rw_ + (j2 + wlo2 + p.pad2);
#pragma unroll
        for (int a = 0; a < RW; ++a)
#pragma unroll
            for (int q = 0; q < XW; ++q) xin[a][q] = float(base[a * rw_ + q]);
#pragma unroll
        for (int rh = 0; rh < S; ++rh) {
            const int oh = S * j1 + rh;
            float out[OC];
#pragma unroll
            for (int e = 0; e < OC; ++e) {
                const int rwp = e % S, je = e / S;
                float acc = bv;
#pragma unroll
                for (int a = 0; a < RW; ++a)
#pragma unroll
                    for (int cc = 0; cc < CW; ++cc) acc += xin[a][je + cc] * eff[rh][rwp][a][cc];
                out[e] = acc;
            }
            if (oh < oh0 || oh >= oh1) continue;
            _Float16 *yr = y + (size_t(c) * p.O1 + oh) * p.O2 + seg * OC;
            if (seg * OC + OC <= p.O2 && (reinterpret_cast<uintptr_t>(yr) % 16 == 0)) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                u32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const unsigned lo = __builtin_bit_cast(unsigned short, _Float16(out[2 * k]));
                    const unsigned hi = __builtin_bit_cast(unsigned short, _Float16(out[2 * k + 1]));
                    o[k] = lo | (hi << 16);
                }
                *reinterpret_cast<u32x4 *>(yr) = o;
            } else {
#pragma unroll
                for (int e = 0; e < OC; ++e)
                    if (seg * OC + e < p.O2) yr[e] = _Float16(out[e]);
            }
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
    if (g.nsp > 2 || g.L[0] != 1 || g.K[0] != 1 || g.O[0] != 1) return no("spatial rank 1 or 2 only");
    if (g.s[1] > kGMaxRes || g.s[2] > kGMaxRes) return no("stride too large");
    if (g.K[1] > kGMaxTaps || g.K[2] > kGMaxTaps) return no("kernel too large");
    GArgs &a = pl->a;
    std::memset(&a, 0, sizeof(a));
    a.N = int(g.N);
    a.C = int(g.C);
    a.M = int(g.M);
    a.G = int(g.G);
    a.Cg = int(g.Cg);
    a.Mg = int(g.Mg);
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
    const int64_t gs1 = std::__gcd(g.s[1], g.d[1]), gs2 = std::__gcd(g.s[2], g.d[2]);
    a.ks1 = short(g.s[1] / gs1);
    a.bs1 = short(g.d[1] / gs1);
    a.ks2 = short(g.s[2] / gs2);
    a.bs2 = short(g.d[2] / gs2);
    int bemin2 = 0, bemax2 = 0;
    bool first = true;
    for (int ax = 1; ax <= 2; ++ax)
        for (int r = 0; r < g.s[ax]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, ax, r, &ph)) return no("too many taps");
            short *k0 = ax == 1 ? a.k0_1 : a.k0_2, *be = ax == 1 ? a.be_1 : a.be_2, *nt = ax == 1 ? a.nt_1 : a.nt_2;
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
    // rows per band: the staged rows of Cg channels plus the group's weights fit in LDS
    const int64_t wbytes = int64_t(g.Cg) * g.Mg * g.K[1] * g.K[2] * 4;
    const int64_t per_row = int64_t(g.Cg) * a.row_w * int64_t(esz);
    if (wbytes + per_row * 2 > kGLdsBytes) return no("group does not fit in LDS");
    const int rows_cap = int((kGLdsBytes - wbytes) / per_row);
    // a band of B output rows reads at most (B - 1 + (K1-1)*d1) / s1 + 2 input rows
    int bandrows = int(g.O[1]);
    while (bandrows > 1 && ((bandrows - 1 + (g.K[1] - 1) * g.d[1]) / g.s[1] + 2) > rows_cap) bandrows = (bandrows + 1) / 2;
    if (((bandrows - 1 + (g.K[1] - 1) * g.d[1]) / g.s[1] + 2) > rows_cap) return no("rows do not fit in LDS");
    a.band = bandrows;
    a.nbands = int((g.O[1] + bandrows - 1) / bandrows);
    a.rows_max = int(std::min<int64_t>(rows_cap, g.L[1] > 0 ? g.L[1] : 1));
    const int64_t blocks = g.N * g.G * a.nbands;
    if (blocks <= 0 || blocks > (1ll << 31) - 1) return no("grid size");
    pl->blocks = int(blocks);
    return true;
}

// Depthwise fast path plan: window offsets wlo, extents RW x CW, staged row width and
// output-row band.  Returns false when the shape is outside the compiled variants.
struct DwPlan {
    GArgs a;
    int blocks, S, RW, CW, wlo1, wlo2;
    bool vec;          // 16-byte staging
    size_t lds_bytes;  // staged rows of one band
};

bool make_dwplan(const Geom &g, ct_dtype dt, const void *x, DwPlan *pl)
{
    if (dt != CT_FLOAT16 || g.Cg != 1 || g.Mg != 1 || g.nsp > 2 || g.L[0] != 1 || g.O[0] != 1) return false;
    const int S = int(g.s[2]);
    if (g.s[1] != S || (S != 1 && S != 2)) return false;
    int wlo[3] = {0, 0, 0}, whi[3] = {0, 0, 0};
    for (int ax = 1; ax <= 2; ++ax) {
        bool any = false;
        for (int r = 0; r < S; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, ax, r, &ph)) return false;
            if (!ph.ntaps) continue;
            const int hi = ph.beta[0], lo = ph.beta[ph.ntaps - 1];
            wlo[ax] = any ? std::min(wlo[ax], lo) : lo;
            whi[ax] = any ? std::max(whi[ax], hi) : hi;
            any = true;
        }
        if (!any) return false;
    }
    const int RW = whi[1] - wlo[1] + 1, CW = whi[2] - wlo[2] + 1;
    const bool compiled = (S == 2 && ((RW == 3 && CW == 3) || (RW == 2 && CW == 2))) ||
                          (S == 1 && ((RW == 3 && CW == 3) || (RW == 5 && CW == 5)));
    if (!compiled) return false;
    GArgs &a = pl->a;
    std::memset(&a, 0, sizeof(a));
    a.N = int(g.N);
    a.C = int(g.C);
    a.M = int(g.M);
    a.G = int(g.G);
    a.Cg = 1;
    a.Mg = 1;
    a.L1 = int(g.L[1]);
    a.L2 = int(g.L[2]);
    a.O1 = int(g.O[1]);
    a.O2 = int(g.O[2]);
    a.K1 = int(g.K[1]);
    a.K2 = int(g.K[2]);
    a.s1 = a.s2 = S;
    a.b1 = int(g.b[1]);
    a.b2 = int(g.b[2]);
    a.d1 = int(g.d[1]);
    a.d2 = int(g.d[2]);
    const int JC = 8 / S;
    const int segs = int((g.O[2] + 7) / 8);
    pl->vec = g.L[2] % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 && -wlo[2] <= 8;
    a.pad2 = pl->vec ? 8 : std::max(0, -wlo[2]);
    const int need = a.pad2 + segs * JC + wlo[2] + CW - 1;  // last staged column read + 1
    a.row_w = (std::max<int>(need, a.pad2 + int(g.L[2])) + 7) / 8 * 8;
    // band of output rows (a multiple of S) whose staged input rows fit the LDS budget
    int band = int((g.O[1] + S - 1) / S) * S;
    auto rows_for = [&](int b) { return (b + S - 1) / S + RW; };
    while (band > S && int64_t(rows_for(band)) * a.row_w * 2 > kDwLdsBytes) band = (band / 2 + S - 1) / S * S;
    if (int64_t(rows_for(band)) * a.row_w * 2 > kDwLdsBytes) return false;
    // few planes: split into more bands so the grid still fills the chip
    while (band >= 8 * S && g.N * g.C * ((g.O[1] + band - 1) / band) < 2048) band = (band / 2 + S - 1) / S * S;
    a.band = band;
    a.nbands = int((g.O[1] + band - 1) / band);
    const int64_t blocks = g.N * g.C * a.nbands;
    if (blocks <= 0 || blocks > (1ll << 31) - 1) return false;
    pl->blocks = int(blocks);
    pl->lds_bytes = size_t(rows_for(band)) * a.row_w * 2;
    pl->S = S;
    pl->RW = RW;
    pl->CW = CW;
    pl->wlo1 = wlo[1];
    pl->wlo2 = wlo[2];
    return true;
}

template <int S, int RW, int CW>
void launch_dw(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    const _Float16 *xh = static_cast<const _Float16 *>(x), *wh = static_cast<const _Float16 *>(w),
                   *bh = static_cast<const _Float16 *>(bias);
    _Float16 *yh = static_cast<_Float16 *>(y);
    if (pl.vec)
        hipLaunchKernelGGL((depthwise_kernel<S, RW, CW, true>), dim3(unsigned(pl.blocks)), dim3(kGThreads),
                           pl.lds_bytes, st, xh, wh, bh, yh, pl.a, pl.wlo1, pl.wlo2);
    else
        hipLaunchKernelGGL((depthwise_kernel<S, RW, CW, false>), dim3(unsigned(pl.blocks)), dim3(kGThreads),
                           pl.lds_bytes, st, xh, wh, bh, yh, pl.a, pl.wlo1, pl.wlo2);
}

}  // namespace

bool grouped_supports(const Geom &g, ct_dtype dt, bool cl)
{
    (void)dt;
    if (cl || g.G < 2 || g.Cg > 8 || g.Mg > 8 || g.L[1] * g.L[2] == 0) return false;
    GPlan pl;
    std::string why;
    return make_gplan(g, dt == CT_FLOAT16 ? 2 : 4, &pl, &why);
}

ct_status launch_grouped(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w, const void *bias,
                         void *y, hipStream_t st, std::string *err)
{
    if (!grouped_supports(g, dt, cl)) {
        *err = "grouped kernel cannot serve this call";
        return CT_EUNSUPPORTED;
    }
    DwPlan dw;
    if (make_dwplan(g, dt, x, &dw)) {
        mark_before(st);
        if (dw.S == 2 && dw.RW == 3) launch_dw<2, 3, 3>(dw, x, w, bias, y, st);
        else if (dw.S == 2) launch_dw<2, 2, 2>(dw, x, w, bias, y, st);
        else if (dw.RW == 3) launch_dw<1, 3, 3>(dw, x, w, bias, y, st);
        else launch_dw<1, 5, 5>(dw, x, w, bias, y, st);
        mark_after(st);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) {
            *err = std::string("depthwise kernel launch failed: ") + hipGetErrorString(e);
            return CT_EDEVICE;
        }
        return CT_OK;
    }
    GPlan pl;
    make_gplan(g, dt == CT_FLOAT16 ? 2 : 4, &pl, err);
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
