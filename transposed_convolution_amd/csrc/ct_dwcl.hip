// ct_dwcl.hip -- depthwise transposed convolution (one input and one output channel per
// group, group == C) for channels-last float16 tensors, spatial rank 1 to 3.
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
//   * Rank 3: a workgroup also owns one output plane o0 = s0*j0 + r0; it stages the tile's
//     window of every input plane j0 + beta that residue r0's first-axis taps read, one
//     after another, with the taps' weights, and sums over them too.
//   * Groups of CG = C/group = M/group channels, CG in {2, 4, 8} (ranks 1 and 2): an
//     octet of output channels holds whole groups, whose input channels are the same
//     octet of X, so the window is staged as for CG = 1; output channel k of the octet
//     sums input channels (k / CG) * CG + j, j < CG, with weights read from LDS per tap.
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
// phase-grid positions per tile: 14 x 8 divides a 56 x 56 phase grid exactly and gives
// each of the 32 position slots 3-4 positions; 8 x 16 left a quarter of the tiles an
// eighth empty, 8 x 8 gave too little work per thread, 28 x 8 too few blocks
constexpr int kTJ1 = 14, kTJ2 = 8;

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
// the same with the half of x and of w chosen separately (xh, wh: high halves; constants
// after unrolling, so one instruction remains)
__device__ __forceinline__ float fma_mix_sel(float acc, unsigned x, bool xh, unsigned w, bool wh)
{
    if (xh && wh) return fma_mix_hi(acc, x, w);
    if (!xh && !wh) return fma_mix_lo(acc, x, w);
    if (xh)
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(x), "v"(w));
    else
        asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[1,1,0]" : "+v"(acc) : "v"(x), "v"(w));
    return acc;
}
constexpr int kMaxOct = 8;         // channel octets per tile (64 channels: more, lighter blocks)
constexpr int kMaxS = 2, kMaxT = 4;
constexpr int kMaxS0 = 4;         // largest stride on the first axis (rank 3)
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
    // first axis (rank 3; one plane otherwise): output plane o0 = s0 * j0 + r0 reads input
    // planes j0 + be00(r0) - u * bs0 with kernel index k00(r0) + u * ks0, u < nt0(r0); the
    // per-residue values are 16-bit fields r0 of these words
    int L0, O0, K0, s0, ks0, bs0;
    unsigned long long nt0w, k00w, be00w;
    Act act;
};

// T0: the most first-axis taps of an output plane (rank 3), 0 for ranks 1 and 2
// CG: channels per group (1: depthwise)
template <int S1, int S2, int T1, int T2, int T0, int CG>
__global__ __launch_bounds__(kThreads) void dwcl_kernel(const _Float16 *__restrict__ x, const _Float16 *__restrict__ w,
                                                        const _Float16 *__restrict__ bias, _Float16 *__restrict__ y,
                                                        DwClArgs p)
{
    constexpr int NE = S1 * S2 * T1 * T2;  // weight entries per channel and plane held by a thread
    constexpr int NT0 = T0 > 0 ? T0 : 1;   // staged input planes
    extern __shared__ __attribute__((aligned(16))) unsigned char dwcl_lds[];
    const int tid = threadIdx.x;

    // each XCD takes a contiguous run of tiles, so the column halo a tile shares with its
    // neighbours is read from HBM once (with the hardware's round-robin order it was read
    // by several XCDs: X came in 1.31 times)
    int rest = xcd_remap(blockIdx.x, p.nblocks);
    const int ot = rest % p.otiles;
    rest /= p.otiles;
    const int t2 = rest % p.tiles2;
    rest /= p.tiles2;
    const int t1 = rest % p.tiles1;
    rest /= p.tiles1;
    // the output plane and the input planes of its first-axis taps (bit u of live: tap u
    // reads a plane inside the input)
    int n = rest, o0 = 0, k0 = 0, i0 = 0, live = 1;
    if constexpr (T0 > 0) {
        o0 = rest % p.O0;
        n = rest / p.O0;
        const int j0 = o0 / p.s0, r0 = o0 - j0 * p.s0;
        auto field = [&](unsigned long long wd) { return int(short((wd >> (16 * r0)) & 0xffffu)); };
        k0 = field(p.k00w);
        i0 = j0 + field(p.be00w);
        const int nt0 = field(p.nt0w);
        live = 0;
#pragma unroll
        for (int v = 0; v < T0; ++v)
            if (v < nt0 && i0 - v * p.bs0 >= 0 && i0 - v * p.bs0 < p.L0) live |= 1 << v;
    }
    const int co = p.co;                        // octets of this tile
    const int c_lo = ot * co * 8;               // first channel of the tile
    const int j1lo = t1 * kTJ1, j2lo = t2 * kTJ2;
    const int i1o = j1lo + p.bmin1, i2o = j2lo + p.bmin2;
    const int KK = p.K1 * p.K2;
    const int rowb = co * 16;                   // LDS bytes per window position
    const int wsz = p.HR * p.HC * rowb;         // LDS bytes per staged plane
    unsigned char *const sx = dwcl_lds;         // [plane][HR][HC][co octets]
    _Float16 *const sw = reinterpret_cast<_Float16 *>(dwcl_lds + NT0 * wsz);  // [plane][tap][co * 8]

    // ---- the tile's input window and weights into LDS ----
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int per = p.HR * p.HC * co;  // items per plane
        const int items = NT0 * per;
        const UDiv dco(co), dhc(p.HC), dkk(KK), dper(per), dwp(co * 8 * KK);  // index splits by multiply-high
        // rounds of kWinBatch loads per thread, all in flight before any is written
        for (int base = 0; base < items; base += kThreads * kWinBatch) {
            u32x4 v[kWinBatch];
            unsigned okm = 0;
#pragma unroll
            for (int k = 0; k < kWinBatch; ++k) {
                const int u = base + tid + k * kThreads;
                const int sl = T0 > 0 ? dper.div(u) : 0, uu = u - sl * per;
                const int q = dco.div(uu), oc = uu - q * co;
                const int hr = dhc.div(q), hc = q - hr * p.HC;
                const int i1 = i1o + hr, i2 = i2o + hc, ip = i0 - sl * p.bs0;
                const bool ok = u < items && ((live >> sl) & 1) && i1 >= 0 && i1 < p.L1 && i2 >= 0 && i2 < p.L2 &&
                                c_lo + oc * 8 < p.C;
                const size_t off = ok ? (((size_t(n) * p.L0 + ip) * p.L1 + i1) * p.L2 + i2) * p.C + c_lo + oc * 8 : 0;
                v[k] = *reinterpret_cast<const u32x4 *>(x + off);  // x[0] when masked
                okm |= unsigned(ok) << k;
            }
#pragma unroll
            for (int k = 0; k < kWinBatch; ++k) {
                const int u = base + tid + k * kThreads;
                if (u < items) {
                    const int sl = T0 > 0 ? dper.div(u) : 0, uu = u - sl * per;
                    const int q = dco.div(uu), oc = uu - q * co;
                    *reinterpret_cast<u32x4 *>(sx + sl * wsz + q * rowb + oc * 16) = ((okm >> k) & 1u) ? v[k] : zero;
                }
            }
        }
        // weights of each staged plane's tap: w[c][k0 + u * ks0][t] into [plane][tap][channel]
        // (CG = 1), or w[c_in][m % CG][k0 + u * ks0][t] into [plane][tap][j][m] for output
        // channel m of the tile and input j of its group (CG > 1)
        const int wpl = co * 8 * KK * CG;  // per plane
        const int wn = NT0 * wpl;
        const UDiv dgk(CG * KK);
        for (int base = 0; base < wn; base += kThreads * kWBatch) {
            _Float16 v[kWBatch];
            unsigned okm = 0;
#pragma unroll
            for (int k = 0; k < kWBatch; ++k) {
                const int u = base + tid + k * kThreads;
                const int sl = T0 > 0 ? dwp.div(u) : 0, uu = u - sl * wpl;
                if constexpr (CG == 1) {
                    const int c = dkk.div(uu), t = uu - c * KK;
                    const bool ok = u < wn && ((live >> sl) & 1) && c_lo + c < p.C;
                    v[k] = w[ok ? (size_t(c_lo + c) * p.K0 + k0 + sl * p.ks0) * KK + t : 0];
                    okm |= unsigned(ok) << k;
                } else {
                    const int m = dgk.div(uu), rem = uu - m * (CG * KK);
                    const int j = dkk.div(rem), t = rem - j * KK;
                    const int cin = c_lo + (m / CG) * CG + j;
                    const bool ok = u < wn && ((live >> sl) & 1) && c_lo + m < p.C;
                    v[k] = w[ok ? ((size_t(cin) * CG + m % CG) * p.K0 + k0 + sl * p.ks0) * KK + t : 0];
                    okm |= unsigned(ok) << k;
                }
            }
#pragma unroll
            for (int k = 0; k < kWBatch; ++k) {
                const int u = base + tid + k * kThreads;
                if (u < wn) {
                    const int sl = T0 > 0 ? dwp.div(u) : 0, uu = u - sl * wpl;
                    if constexpr (CG == 1) {
                        const int c = dkk.div(uu), t = uu - c * KK;
                        sw[sl * wpl + t * (co * 8) + c] = ((okm >> k) & 1u) ? v[k] : _Float16(0.0f);
                    } else {
                        const int m = dgk.div(uu), rem = uu - m * (CG * KK);
                        const int j = dkk.div(rem), t = rem - j * KK;
                        sw[sl * wpl + (t * CG + j) * (co * 8) + m] = ((okm >> k) & 1u) ? v[k] : _Float16(0.0f);
                    }
                }
            }
        }
    }
    __syncthreads();

    const int oc = tid % co, slot = tid / co, nslots = kThreads / co;
    if (slot >= nslots) return;  // threads past the last whole slot (co does not divide 256)
    // the thread's weights: entry e = ((r1 * S2 + r2) * T1 + a) * T2 + cc of each plane
    // (CG = 1; groups read theirs from LDS per tap)
    u32x4 wv[CG == 1 ? NT0 : 1][CG == 1 ? NE : 1];
#pragma unroll
    for (int v0 = 0; v0 < (CG == 1 ? NT0 : 0); ++v0)
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
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(
                            &sw[v0 * co * 8 * KK + (k1 >= 0 && k2 >= 0 ? k1 * p.K2 + k2 : 0) * (co * 8) + oc * 8]);
                        wv[v0][e] = (k1 >= 0 && k2 >= 0) ? v : u32x4{0u, 0u, 0u, 0u};
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
                    for (int v0 = 0; v0 < NT0; ++v0) {
                        if (T0 > 0 && !((live >> v0) & 1)) continue;  // uniform over the block
#pragma unroll
                        for (int a = 0; a < T1; ++a)
#pragma unroll
                            for (int cc = 0; cc < T2; ++cc) {
                                const int e = ((r1 * S2 + r2) * T1 + a) * T2 + cc;
                                const int wr = pj1 + p.off1[r1][a], wc = pj2 + p.off2[r2][cc];
                                if constexpr (CG == 1) {
                                    const u32x4 xv =
                                        *reinterpret_cast<const u32x4 *>(sx + v0 * wsz + (wr * p.HC + wc) * rowb + oc * 16);
#pragma unroll
                                    for (int k = 0; k < 4; ++k) {  // channels 2k (low halves), 2k + 1 (high)
                                        acc[2 * k] = fma_mix_lo(acc[2 * k], xv[k], wv[v0][e][k]);
                                        acc[2 * k + 1] = fma_mix_hi(acc[2 * k + 1], xv[k], wv[v0][e][k]);
                                    }
                                } else {
                                    const int k1 = p.k1[r1][a], k2 = p.k2[r2][cc];
                                    if (k1 < 0 || k2 < 0) continue;  // no tap (uniform)
                                    const u32x4 xv =
                                        *reinterpret_cast<const u32x4 *>(sx + v0 * wsz + (wr * p.HC + wc) * rowb + oc * 16);
                                    const _Float16 *const wt = sw + (size_t(v0) * KK + k1 * p.K2 + k2) * CG * (co * 8) + oc * 8;
#pragma unroll
                                    for (int j = 0; j < CG; ++j) {
                                        // output k of the octet takes input (k / CG) * CG + j
                                        const u32x4 wj = *reinterpret_cast<const u32x4 *>(wt + j * (co * 8));
#pragma unroll
                                        for (int k = 0; k < 8; ++k) {
                                            const int xi = (k / CG) * CG + j;
                                            acc[k] = fma_mix_sel(acc[k], xv[xi >> 1], xi & 1, wj[k >> 1], k & 1);
                                        }
                                    }
                                }
                            }
                    }
                    _Float16 *dst = y + (((size_t(n) * p.O0 + o0) * p.O1 + o1) * p.O2 + o2) * p.C + c_lo + oc * 8;
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
    int T0;  // kernel's T0: the most first-axis taps of a residue (rank 3), else 0
    int CG;  // channels per group (C/group = M/group)
    size_t lds;
};

bool make_dwcl_plan(const Geom &g, DwClPlan *pl)
{
    DwClArgs &a = pl->a;
    std::memset(&a, 0, sizeof(a));
    // first axis (one plane below rank 3): per residue its taps as a progression
    if (g.s[0] > kMaxS0) return false;
    const int64_t gs0 = std::__gcd(g.s[0], g.d[0]);
    a.ks0 = int(g.s[0] / gs0);
    a.bs0 = int(g.d[0] / gs0);
    int T0 = 0;
    for (int r = 0; r < g.s[0]; ++r) {
        AxisPhase ph;
        if (!axis_phase(g, 0, r, &ph)) return false;
        for (int u = 1; u < ph.ntaps; ++u)
            if (ph.k[u] - ph.k[u - 1] != a.ks0 || ph.beta[u - 1] - ph.beta[u] != a.bs0) return false;
        const int k0 = ph.ntaps ? ph.k[0] : 0, be0 = ph.ntaps ? ph.beta[0] : 0;
        if (k0 > 32767 || be0 < -32768 || be0 > 32767) return false;
        a.nt0w |= (unsigned long long)(ph.ntaps & 0xffff) << (16 * r);
        a.k00w |= (unsigned long long)(k0 & 0xffff) << (16 * r);
        a.be00w |= (unsigned long long)(unsigned(be0) & 0xffffu) << (16 * r);
        T0 = std::max(T0, ph.ntaps);
    }
    if (T0 == 0 || T0 > 3) return false;  // no tap reaches an output plane, or too many planes
    pl->T0 = g.nsp == 3 ? T0 : 0;
    a.L0 = int(g.L[0]);
    a.O0 = int(g.O[0]);
    a.K0 = int(g.K[0]);
    a.s0 = int(g.s[0]);
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
    const long long blocks = (long long)g.N * g.O[0] * a.tiles1 * a.tiles2 * a.otiles;
    if (blocks < 1 || blocks > INT32_MAX) return false;
    a.nblocks = int(blocks);
    const int nt0 = std::max(pl->T0, 1);  // staged planes
    pl->CG = int(g.Cg);
    pl->lds = nt0 * (size_t(a.HR) * a.HC * a.co * 16 + size_t(a.co) * 8 * a.K1 * a.K2 * 2 * pl->CG);
    if (pl->lds > 64 * 1024) return false;
    return true;
}

template <int S1, int S2, int T1, int T2, int T0, int CG = 1>
bool launch_if(const DwClPlan &pl, const void *x, const void *w, const void *b, void *y, hipStream_t st)
{
    if (pl.S1 != S1 || pl.S2 != S2 || pl.T1 != T1 || pl.T2 != T2 || pl.T0 != T0 || pl.CG != CG) return false;
    hipLaunchKernelGGL((dwcl_kernel<S1, S2, T1, T2, T0, CG>), dim3(unsigned(pl.a.nblocks)), dim3(kThreads), pl.lds, st,
                       static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w),
                       static_cast<const _Float16 *>(b), static_cast<_Float16 *>(y), pl.a);
    return true;
}

// equal strides on the last two axes: ranks 2 and 3
template <int T0, int CG = 1>
bool launch_square(const DwClPlan &pl, const void *x, const void *w, const void *b, void *y, hipStream_t st)
{
    return launch_if<2, 2, 1, 1, T0, CG>(pl, x, w, b, y, st) || launch_if<2, 2, 2, 2, T0, CG>(pl, x, w, b, y, st) ||
           launch_if<1, 1, 1, 1, T0, CG>(pl, x, w, b, y, st) || launch_if<1, 1, 2, 2, T0, CG>(pl, x, w, b, y, st) ||
           launch_if<1, 1, 3, 3, T0, CG>(pl, x, w, b, y, st);
}

bool has_instance(const DwClPlan &pl)
{
    // (S1, S2, T1, T2): ranks 2 and 3, then rank 1 (T0 = 0 only)
    static const int square[][4] = {{2, 2, 1, 1}, {2, 2, 2, 2}, {1, 1, 1, 1}, {1, 1, 2, 2}, {1, 1, 3, 3}};
    static const int rank1[][4] = {{1, 2, 1, 1}, {1, 2, 1, 2}, {1, 2, 1, 4}, {1, 1, 1, 2}, {1, 1, 1, 3}, {1, 1, 1, 4}};
    if (pl.CG != 1) {  // groups: the rank-2 instances
        if (pl.CG != 2 && pl.CG != 4 && pl.CG != 8) return false;
        for (const auto &i : square)
            if (pl.S1 == i[0] && pl.S2 == i[1] && pl.T1 == i[2] && pl.T2 == i[3]) return pl.T0 == 0;
        return false;
    }
    for (const auto &i : square)
        if (pl.S1 == i[0] && pl.S2 == i[1] && pl.T1 == i[2] && pl.T2 == i[3]) return pl.T0 >= 0 && pl.T0 <= 3;
    if (pl.T0 != 0) return false;
    for (const auto &i : rank1)
        if (pl.S1 == i[0] && pl.S2 == i[1] && pl.T1 == i[2] && pl.T2 == i[3]) return true;
    return false;
}

}  // namespace

bool dwcl_supports(const Geom &g, ct_dtype dt, bool cl, const void *x)
{
    if (!cl || dt != CT_FLOAT16 || g.Cg != g.Mg || g.Cg > 8 || 8 % g.Cg != 0 || g.C % 8 != 0 || g.x_elems() <= 0)
        return false;
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
        launch_square<0>(pl, x, w, bias, y, st) || launch_if<1, 2, 1, 1, 0>(pl, x, w, bias, y, st) ||
        launch_if<1, 2, 1, 2, 0>(pl, x, w, bias, y, st) || launch_if<1, 2, 1, 4, 0>(pl, x, w, bias, y, st) ||
        launch_if<1, 1, 1, 2, 0>(pl, x, w, bias, y, st) || launch_if<1, 1, 1, 3, 0>(pl, x, w, bias, y, st) ||
        launch_if<1, 1, 1, 4, 0>(pl, x, w, bias, y, st) || launch_square<1>(pl, x, w, bias, y, st) ||
        launch_square<2>(pl, x, w, bias, y, st) || launch_square<3>(pl, x, w, bias, y, st) ||
        launch_square<0, 2>(pl, x, w, bias, y, st) || launch_square<0, 4>(pl, x, w, bias, y, st) ||
        launch_square<0, 8>(pl, x, w, bias, y, st);
    mark_after(st);
    const hipError_t e = launched ? hipGetLastError() : hipErrorInvalidConfiguration;
    if (e != hipSuccess) {
        *err = std::string("channels-last depthwise kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
