// ct_dwcl.hip -- depthwise transposed convolution (one input and one output channel per
// group, group == C) for channels-last float16 tensors, spatial rank 1 or 2.
//
// The grouped form of the operator (webgpu-kernels "ai.onnx.ConvTranspose" README,
// Attributes: group) with C/group == M/group == 1, on the channels-last layout of the
// ClikaRT "conv_transpose" page: output channel c is the scatter of input channel c
// through its own kernel.  Read from the output side with the stride-phase split (output
// o = s*j + r on each axis), output (j, r) receives the taps of residue r from the inputs
// j + beta.  Every output needs a handful of multiply-adds, so the kernel is bound by HBM
// traffic (X read once, Y written once) and uses the vector ALUs, not MFMA.
//
//   * A workgroup owns a tile of phase-grid positions (8 x 16) and up to 64 channels
//     (8 octets of 8 channels, 16 bytes): the input window of the tile is staged in LDS
//     once ([row][column][channel octet], zeros outside the input), the tile's weights in
//     LDS as [tap][channel].
//   * A thread owns one channel octet: it keeps the weights of all residue classes and
//     taps of its 8 channels in registers, then for each of its positions and each class
//     sums the class's taps (float16 products, float32 accumulation), adds the bias and
//     writes the 8 channels of the output with one 16-byte store.  Consecutive threads
//     hold consecutive octets, so a wave writes whole 128-byte runs of channels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <type_traits>

#include "ct_internal.hpp"

namespace ct {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTJ1 = 8, kTJ2 = 16;  // phase-grid positions per tile

// acc + x * w for the low (high) float16 halves of x and w, in float32 with one rounding
// (v_fma_mix_f32: the float16 operands are widened exactly), so weights stay packed
// float16 in registers
__device__ __forceinline__ float fma_mix_lo(float acc, unsigned x, unsigned w)
{
    asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(x), "v"(w));
    return acc;
}
__device__ __forceinline__ float fma_mix_hi(float acc, unsigned x, unsigned w)
{
    asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,1,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(x), "v"(w));
    return acc;
}
constexpr int kMaxOct = 8;         // channel octets per tile (64 channels: more, lighter blocks)
constexpr int kMaxS = 2, kMaxT = 4;
constexpr int kWinBatch = 6;      // window loads per thread in flight together
constexpr int kWBatch = 4;        // weight loads per thread in flight together

struct DwClArgs {
    int N, C, L1, L2, O1, O2, K1, K2;
    int s1, s2, J1, J2;
    int bmin1, bmin2, HR, HC;      // tile window: origin offset and extents
    int co, otiles, tiles1, tiles2, nblocks;
    // per residue r of each axis and tap u < T: window offset beta - bmin and kernel index
    // (-1: no tap, weight 0)
    int off1[kMaxS][kMaxT], off2[kMaxS][kMaxT];
    int k1[kMaxS][kMaxT], k2[kMaxS][kMaxT];
    Act act;
};

template <int S1, int S2, int T1, int T2>
__global__ __launch_bounds__(kThreads) void dwcl_kernel(const _Float16 *__restrict__ x, const _Float16 *__restrict__ w,
                                                        const _Float16 *__restrict__ bias, _Float16 *__restrict__ y,
                                                        DwClArgs p)
{
    constexpr int NE = S1 * S2 * T1 * T2;  // weight entries per channel held by a thread
    extern __shared__ __attribute__((aligned(16))) unsigned char dwcl_lds[];
    const int tid = threadIdx.x;

    int rest = blockIdx.x;
    const int ot = rest % p.otiles;
    rest /= p.otiles;
    const int t2 = rest % p.tiles2;
    rest /= p.tiles2;
    const int t1 = rest % p.tiles1;
    const int n = rest / p.tiles1;
    const int co = p.co;                        // octets of this tile
    const int c_lo = ot * co * 8;               // first channel of the tile
    const int j1lo = t1 * kTJ1, j2lo = t2 * kTJ2;
    const int i1o = j1lo + p.bmin1, i2o = j2lo + p.bmin2;
    const int KK = p.K1 * p.K2;
    const int rowb = co * 16;                   // LDS bytes per window position
    unsigned char *const sx = dwcl_lds;         // [HR][HC][co octets]
    _Float16 *const sw = reinterpret_cast<_Float16 *>(dwcl_lds + p.HR * p.HC * rowb);  // [tap][co * 8]

    // ---- the tile's input window and weights into LDS ----
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int items = p.HR * p.HC * co;
        const UDiv dco(co), dhc(p.HC), dkk(KK);  // index splits by multiply-high
        // rounds of kWinBatch loads per thread, all in flight before any is written
        for (int base = 0; base < items; base += kThreads * kWinBatch) {
            u32x4 v[kWinBatch];
            unsigned okm = 0;
#pragma unroll
            for (int k = 0; k < kWinBatch; ++k) {
                const int u = base + tid + k * kThreads;
                const int q = dco.div(u), oc = u - q * co;
                const int hr = dhc.div(q), hc = q - hr * p.HC;
                const int i1 = i1o + hr, i2 = i2o + hc;
                const bool ok = u < items && i1 >= 0 && i1 < p.L1 && i2 >= 0 && i2 < p.L2 && c_lo + oc * 8 < p.C;
                const size_t off = ok ? ((size_t(n) * p.L1 + i1) * p.L2 + i2) * p.C + c_lo + oc * 8 : 0;
                v[k] = *reinterpret_cast<const u32x4 *>(x + off);  // x[0] when masked
                okm |= unsigned(ok) << k;
            }
#pragma unroll
            for (int k = 0; k < kWinBatch; ++k) {
                const int u = base + tid + k * kThreads;
                if (u < items) {
                    const int q = dco.div(u), oc = u - q * co;
                    *reinterpret_cast<u32x4 *>(sx + q * rowb + oc * 16) = ((okm >> k) & 1u) ? v[k] : zero;
                }
            }
        }
        const int wn = co * 8 * KK;
        for (int base = 0; base < wn; base += kThreads * kWBatch) {
            _Float16 v[kWBatch];
            unsigned okm = 0;
#pragma unroll
            for (int k = 0; k < kWBatch; ++k) {
                const int u = base + tid + k * kThreads;
                const int c = dkk.div(u), t = u - c * KK;
                const bool ok = u < wn && c_lo + c < p.C;
                v[k] = w[ok ? size_t(c_lo + c) * KK + t : 0];
                okm |= unsigned(ok) << k;
            }
#pragma unroll
            for (int k = 0; k < kWBatch; ++k) {
                const int u = base + tid + k * kThreads;
                if (u < wn) {
                    const int c = dkk.div(u), t = u - c * KK;
                    sw[t * (co * 8) + c] = ((okm >> k) & 1u) ? v[k] : _Float16(0.0f);
                }
            }
        }
    }
    __syncthreads();

    const int oc = tid % co, slot = tid / co, nslots = kThreads / co;
    if (slot >= nslots) return;  // threads past the last whole slot (co does not divide 256)
    // the thread's weights: entry e = ((r1 * S2 + r2) * T1 + a) * T2 + cc
    u32x4 wv[NE];
#pragma unroll
    for (int r1 = 0; r1 < S1; ++r1)
#pragma unroll
        for (int r2 = 0; r2 < S2; ++r2)
#pragma unroll
            for (int a = 0; a < T1; ++a)
#pragma unroll
                for (int cc = 0; cc < T2; ++cc) {
                    const int e = ((r1 * S2 + r2) * T1 + a) * T2 + cc;
                    const int k1 = p.k1[r1][a], k2 = p.k2[r2][cc];
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(&sw[(k1 >= 0 && k2 >= 0 ? k1 * p.K2 + k2 : 0) * (co * 8) + oc * 8]);
                    wv[e] = (k1 >= 0 && k2 >= 0) ? v : u32x4{0u, 0u, 0u, 0u};
                }
    float bv[8];
    {
        const int c = c_lo + oc * 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) bv[k] = (bias && c + k < p.C) ? float(bias[c + k]) : 0.0f;
    }
    const bool vec = c_lo + oc * 8 + 8 <= p.C && reinterpret_cast<uintptr_t>(y) % 16 == 0;
    const bool full_lines = co % 8 == 0 && p.C % 64 == 0 && reinterpret_cast<uintptr_t>(y) % 128 == 0;

    // streaming stores when adjacent lanes cover whole 128-byte lines of Y (the tile's
    // channel run of a pixel); two copies of the loop, since a store under a run-time
    // choice would be merged with the plain one and lose its cache hint
    auto body = [&](auto fin, auto streaming) {
        for (int pos = slot; pos < kTJ1 * kTJ2; pos += nslots) {
            const int pj1 = pos / kTJ2, pj2 = pos - pj1 * kTJ2;
            const int j1 = j1lo + pj1, j2 = j2lo + pj2;
#pragma unroll
            for (int r1 = 0; r1 < S1; ++r1)
#pragma unroll
                for (int r2 = 0; r2 < S2; ++r2) {
                    const int o1 = p.s1 * j1 + r1, o2 = p.s2 * j2 + r2;
                    if (o1 >= p.O1 || o2 >= p.O2) continue;
                    float acc[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) acc[k] = bv[k];
#pragma unroll
                    for (int a = 0; a < T1; ++a)
#pragma unroll
                        for (int cc = 0; cc < T2; ++cc) {
                            const int e = ((r1 * S2 + r2) * T1 + a) * T2 + cc;
                            const int wr = pj1 + p.off1[r1][a], wc = pj2 + p.off2[r2][cc];
                            const u32x4 xv = *reinterpret_cast<const u32x4 *>(sx + (wr * p.HC + wc) * rowb + oc * 16);
#pragma unroll
                            for (int k = 0; k < 4; ++k) {  // channels 2k (low halves), 2k + 1 (high)
                                acc[2 * k] = fma_mix_lo(acc[2 * k], xv[k], wv[e][k]);
                                acc[2 * k + 1] = fma_mix_hi(acc[2 * k + 1], xv[k], wv[e][k]);
                            }
                        }
                    _Float16 *dst = y + ((size_t(n) * p.O1 + o1) * p.O2 + o2) * p.C + c_lo + oc * 8;
                    if (vec) {
                        f16x8 o;
#pragma unroll
                        for (int k = 0; k < 8; ++k) o[k] = _Float16(fin(acc[k]));
                        // Y is written once and read by no block; partial lines go through
                        // the cache, which merges them
                        if constexpr (decltype(streaming)::value)
                            __builtin_nontemporal_store(o, reinterpret_cast<f16x8 *>(dst));
                        else
                            *reinterpret_cast<f16x8 *>(dst) = o;
                    } else {
                        for (int k = 0; k < 8 && c_lo + oc * 8 + k < p.C; ++k) dst[k] = _Float16(fin(acc[k]));
                    }
                }
        }
    };
    if (full_lines)
        with_activation(p.act, [&](auto fin) { body(fin, std::true_type{}); });
    else
        with_activation(p.act, [&](auto fin) { body(fin, std::false_type{}); });
}

struct DwClPlan {
    DwClArgs a;
    int S1, S2, T1, T2;
    size_t lds;
};

bool make_dwcl_plan(const Geom &g, DwClPlan *pl)
{
    if (g.nsp > 2 || g.L[0] != 1 || g.K[0] != 1 || g.O[0] != 1) return false;
    DwClArgs &a = pl->a;
    std::memset(&a, 0, sizeof(a));
    a.N = int(g.N);
    a.C = int(g.C);
    a.L1 = int(g.L[1]);
    a.L2 = int(g.L[2]);
    a.O1 = int(g.O[1]);
    a.O2 = int(g.O[2]);
    a.K1 = int(g.K[1]);
    a.K2 = int(g.K[2]);
    a.s1 = int(g.s[1]);
    a.s2 = int(g.s[2]);
    if (a.s1 > kMaxS || a.s2 > kMaxS) return false;
    int T[3] = {0, 0, 0};
    int bmin[3] = {0, 0, 0}, bmax[3] = {0, 0, 0};
    for (int ax = 1; ax <= 2; ++ax) {
        bool first = true;
        for (int r = 0; r < g.s[ax]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, ax, r, &ph) || ph.ntaps > kMaxT) return false;
            T[ax] = std::max(T[ax], ph.ntaps);
            for (int u = 0; u < ph.ntaps; ++u) {
                bmin[ax] = first ? ph.beta[u] : std::min(bmin[ax], ph.beta[u]);
                bmax[ax] = first ? ph.beta[u] : std::max(bmax[ax], ph.beta[u]);
                first = false;
            }
        }
        T[ax] = std::max(T[ax], 1);
    }
    for (int ax = 1; ax <= 2; ++ax)
        for (int r = 0; r < kMaxS; ++r)
            for (int u = 0; u < kMaxT; ++u) {
                int off = 0, k = -1;
                if (r < g.s[ax]) {
                    AxisPhase ph;
                    axis_phase(g, ax, r, &ph);
                    if (u < ph.ntaps) {
                        off = ph.beta[u] - bmin[ax];
                        k = ph.k[u];
                    }
                }
                (ax == 1 ? a.off1 : a.off2)[r][u] = off;
                (ax == 1 ? a.k1 : a.k2)[r][u] = k;
            }
    // the compiled instances: rank 2 with equal strides, rank 1 (unit axis 1)
    pl->S1 = a.s1;
    pl->S2 = a.s2;
    pl->T1 = T[1];
    pl->T2 = T[2];
    const bool rank1 = g.L[1] == 1 && g.K[1] == 1 && g.O[1] == 1 && a.s1 == 1;
    if (rank1) {
        pl->T1 = 1;
        if (pl->T2 > 4) return false;
        if (pl->T2 == 3 && a.s2 == 2) pl->T2 = 4;  // instances: s 2 with T 1, 2, 4
    } else {
        if (a.s1 != a.s2) return false;
        const int t = std::max(pl->T1, pl->T2);
        if (a.s1 == 2 && t > 2) return false;  // instances: s 2 with T 1 or 2; s 1 with T 1..3
        if (a.s1 == 1 && t > 3) return false;
        pl->T1 = pl->T2 = t;
    }
    a.bmin1 = bmin[1];
    a.bmin2 = bmin[2];
    a.HR = kTJ1 + bmax[1] - bmin[1];
    a.HC = kTJ2 + bmax[2] - bmin[2];
    a.J1 = int((g.O[1] + g.s[1] - 1) / g.s[1]);
    a.J2 = int((g.O[2] + g.s[2] - 1) / g.s[2]);
    a.tiles1 = (a.J1 + kTJ1 - 1) / kTJ1;
    a.tiles2 = (a.J2 + kTJ2 - 1) / kTJ2;
    const int oct = int((g.C + 7) / 8);
    a.co = std::min(oct, kMaxOct);
    a.otiles = (oct + a.co - 1) / a.co;
    const long long blocks = (long long)g.N * a.tiles1 * a.tiles2 * a.otiles;
    if (blocks < 1 || blocks > INT32_MAX) return false;
    a.nblocks = int(blocks);
    pl->lds = size_t(a.HR) * a.HC * a.co * 16 + size_t(a.co) * 8 * a.K1 * a.K2 * 2;
    if (pl->lds > 64 * 1024) return false;
    return true;
}

template <int S1, int S2, int T1, int T2>
bool launch_if(const DwClPlan &pl, const void *x, const void *w, const void *b, void *y, hipStream_t st)
{
    if (pl.S1 != S1 || pl.S2 != S2 || pl.T1 != T1 || pl.T2 != T2) return false;
    hipLaunchKernelGGL((dwcl_kernel<S1, S2, T1, T2>), dim3(unsigned(pl.a.nblocks)), dim3(kThreads), pl.lds, st,
                       static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w),
                       static_cast<const _Float16 *>(b), static_cast<_Float16 *>(y), pl.a);
    return true;
}

bool has_instance(const DwClPlan &pl)
{
    static const int inst[][4] = {{2, 2, 1, 1}, {2, 2, 2, 2}, {1, 1, 1, 1}, {1, 1, 2, 2}, {1, 1, 3, 3},
                                  {1, 2, 1, 1}, {1, 2, 1, 2}, {1, 2, 1, 4}, {1, 1, 1, 2}, {1, 1, 1, 3}, {1, 1, 1, 4}};
    for (const auto &i : inst)
        if (pl.S1 == i[0] && pl.S2 == i[1] && pl.T1 == i[2] && pl.T2 == i[3]) return true;
    return false;
}

}  // namespace

bool dwcl_supports(const Geom &g, ct_dtype dt, bool cl, const void *x)
{
    if (!cl || dt != CT_FLOAT16 || g.Cg != 1 || g.Mg != 1 || g.C % 8 != 0 || g.x_elems() <= 0) return false;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return false;
    DwClPlan pl;
    return make_dwcl_plan(g, &pl) && has_instance(pl);
}

ct_status launch_dwcl(const Geom &g, const void *x, const void *w, const void *bias, void *y, const Act &act,
                      hipStream_t st, std::string *err)
{
    DwClPlan pl;
    if (!make_dwcl_plan(g, &pl) || !has_instance(pl)) {
        *err = "channels-last depthwise kernel cannot serve this call";
        return CT_EUNSUPPORTED;
    }
    pl.a.act = act;
    mark_before(st);
    const bool launched =
        launch_if<2, 2, 1, 1>(pl, x, w, bias, y, st) || launch_if<2, 2, 2, 2>(pl, x, w, bias, y, st) ||
        launch_if<1, 1, 1, 1>(pl, x, w, bias, y, st) || launch_if<1, 1, 2, 2>(pl, x, w, bias, y, st) ||
        launch_if<1, 1, 3, 3>(pl, x, w, bias, y, st) || launch_if<1, 2, 1, 1>(pl, x, w, bias, y, st) ||
        launch_if<1, 2, 1, 2>(pl, x, w, bias, y, st) || launch_if<1, 2, 1, 4>(pl, x, w, bias, y, st) ||
        launch_if<1, 1, 1, 2>(pl, x, w, bias, y, st) || launch_if<1, 1, 1, 3>(pl, x, w, bias, y, st) ||
        launch_if<1, 1, 1, 4>(pl, x, w, bias, y, st);
    mark_after(st);
    const hipError_t e = launched ? hipGetLastError() : hipErrorInvalidConfiguration;
    if (e != hipSuccess) {
        *err = std::string("channels-last depthwise kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
