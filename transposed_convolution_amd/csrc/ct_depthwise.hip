// ct_depthwise.hip -- depthwise transposed convolution (one input and one output channel
// per group, group == C) in float16, channels-first, spatial rank 1 or 2.
//
// The grouped form of the operator (webgpu-kernels "ai.onnx.ConvTranspose" README,
// Attributes: group) with C/group == M/group == 1: each output plane is the scatter of one
// input plane through its own K1 x K2 kernel.  Read from the output side with the
// stride-phase split (output o = S*j + r), the taps of residue r on one axis read inputs
// i = j + beta for a run of consecutive beta (when d divides S the run has step 1), so
// each of the S*S output phases is a small dense correlation of the input with a T1 x T2
// sub-kernel of W.  The work per output is a handful of multiply-adds: the kernel is bound
// by HBM traffic (read X once, write Y once), so it uses the vector ALUs, not MFMA.
//
// Work unit = (plane n*C + channel, band of output rows).  A block stages the band's input
// rows in LDS (zero columns on both sides, so no column tests remain), then each thread
// makes S output rows x 8 output columns: for each output row phase it reads T1 input
// rows at that phase's row offset, and each column phase applies its T1 x T2 sub-kernel
// (held in registers) at its own column offset within that window.  Blocks are persistent
// and issue the global loads of their next unit before computing the current one.
// Products of float16 values are exact in float32; pairs of column taps are summed by a
// packed float16 dot product with float32 accumulation.  Each result is rounded once to
// float16 and a row of 8 is written as one 16-byte store.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "ct_internal.hpp"

namespace ct {
namespace {

constexpr int kDwThreads = 256;
constexpr int kDwMaxS = 4;                                 // largest stride served
constexpr int kDwMaxChunks = 8;                              // 16-byte input chunks per thread per unit
constexpr int kDwStageBytes = kDwMaxChunks * kDwThreads * 16;  // staged band (float16), upper bound
constexpr int kDwGuard = 8;                                    // zero elements ahead of staged row 0

struct DwArgs {
    int C, L1, L2, O1, O2, K1, K2, b1, b2, d1, d2;
    int band, nbands, units;
    int row_w;     // staged row stride R in elements (multiple of 8): L2 inputs, then zeros
    int nrows;     // staged rows per unit
    int lo1, lo2;  // smallest input offset beta over all phases, per axis
    int span1;     // staged rows beyond the band's input rows: hi1 - lo1 + 1
    int stage_elems;    // halves per stage buffer (multiple of 8)
    int a0_1[kDwMaxS];  // per row residue: its window's row offset from lo1
    Act act;            // output activation
};

template <int S, int T1, int T2, int OFF2, int NQ>
__global__ __launch_bounds__(kDwThreads) void depthwise_kernel(const _Float16 *__restrict__ x,
                                                               const _Float16 *__restrict__ w,
                                                               const _Float16 *__restrict__ bias,
                                                               _Float16 *__restrict__ y, DwArgs p)
{
    constexpr int OC = 8;               // output columns per thread
    constexpr int JC = OC / S;          // input-grid columns they span
    constexpr int NE = S * S * T1 * T2;  // sub-kernel entries over all phases
    // column offset of residue r's window (0 or 1), fixed at compile time so every
    // register index below is a constant; row offsets are LDS addresses and stay runtime
    constexpr int MAXO2 = (OFF2 != 0) ? 1 : 0;
    constexpr int XW = JC + T2 - 1 + MAXO2;  // window columns per row
    constexpr int NP = T2 / 2;               // column-tap pairs per sub-kernel row
    static_assert(NE <= kDwThreads, "sub-kernels larger than the block");
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    // Stage: kDwGuard zero elements, then nrows rows of R elements each: input columns
    // [0, L2) followed by zeros up to R.  Reads left of a row land in the previous row's
    // zeros (or the leading guard), reads right of it in its own.
    extern __shared__ __attribute__((aligned(16))) unsigned char dw_lds[];
    _Float16 *const sx = reinterpret_cast<_Float16 *>(dw_lds);
    __shared__ _Float16 seff[NE];

    const int R = p.row_w, cpl = p.L2 / 8;
    const int segs = (p.O2 + OC - 1) / OC;
    const int plane_in = p.L1 * p.L2;

    // ---- unit-invariant per-thread constants ----
    // sub-kernel entry e = ((rh * S + rw) * T1 + a) * T2 + cc holds the tap k on each axis
    // with r + b - k d == beta S, beta = lo + a0[r] + a; eidx = k1 * K2 + k2, or -1
    int eidx = -1;
    {
        const int e = threadIdx.x;
        const int cc = e % T2, a = (e / T2) % T1, rwp = (e / (T2 * T1)) % S, rhp = (e / (T2 * T1 * S)) % S;
        const int t1 = rhp + p.b1 - (p.lo1 + p.a0_1[rhp] + a) * S;
        const int t2 = rwp + p.b2 - (p.lo2 + ((OFF2 >> rwp) & 1) + cc) * S;
        if (e < NE && t1 >= 0 && t1 % p.d1 == 0 && t1 / p.d1 < p.K1 && t2 >= 0 && t2 % p.d2 == 0 &&
            t2 / p.d2 < p.K2)
            eidx = (t1 / p.d1) * p.K2 + t2 / p.d2;
    }
    // chunk q of this thread is the k-th 16-byte piece of the band's valid input rows:
    // row k / cpl of them, column 8 * (k % cpl)
    int chr[NQ], chc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int k = threadIdx.x + q * kDwThreads;
        chr[q] = k / cpl;
        chc[q] = (k - chr[q] * cpl) * 8;
    }
    const int seg0 = threadIdx.x % segs, jr0 = threadIdx.x / segs;
    const int dseg = kDwThreads % segs, djr = kDwThreads / segs;

    struct Unit {
        int c, ch, oh0, oh1, j1lo, j1hi, ilo, vr0, nvr;
    };
    auto unit_of = [&](int t) {
        Unit u;
        const int band = t % p.nbands;
        u.c = t / p.nbands;
        u.ch = u.c % p.C;
        u.oh0 = band * p.band;
        u.oh1 = min(u.oh0 + p.band, p.O1);
        u.j1lo = u.oh0 / S;
        u.j1hi = (u.oh1 - 1) / S;
        u.ilo = u.j1lo + p.lo1;  // input row of staged row 0
        // staged rows [vr0, vr0 + nvr) hold input rows; the others of the p.nrows are zero
        const int first = max(u.ilo, 0), last = min(u.ilo + p.nrows, p.L1);
        u.vr0 = first - u.ilo;
        u.nvr = max(last - first, 0);
        return u;
    };
    // Operands of one unit, loaded ahead.  Loads are unconditional from clamped addresses;
    // the validity mask is applied when the chunk is staged, so nothing waits for the
    // data before then.
    u32x4 v[NQ];
    unsigned vok = 0;
    _Float16 ew, braw;
    auto issue = [&](const Unit &u) {
        const _Float16 *xp = x + size_t(u.c) * plane_in;
        const _Float16 *xb = xp + (u.ilo + u.vr0) * p.L2;  // first valid row: contiguous from here
        ew = w[size_t(u.ch) * p.K1 * p.K2 + max(eidx, 0)];
        braw = *(bias ? bias + u.ch : xp);  // used only with a bias
        const int nch = u.nvr * cpl;
        vok = 0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int k = threadIdx.x + q * kDwThreads;
            const bool ok = k < nch;
            v[q] = *reinterpret_cast<const u32x4 *>(ok ? xb + 8 * k : xp);
            vok |= unsigned(ok) << q;
        }
    };

    // zero the whole stage once: guards and row tails are never written again
    for (int k = threadIdx.x; k < p.stage_elems / 8; k += kDwThreads)
        reinterpret_cast<u32x4 *>(sx)[k] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    int t = blockIdx.x;  // the grid never exceeds the unit count
    Unit cur = unit_of(t);
    issue(cur);
    for (;;) {
        // ---- stage the current unit ----
        // staged rows without input (above row 0 or below row L1-1): zeros
        {
            const int nz = (p.nrows - cur.nvr) * cpl;
            for (int k = threadIdx.x; k < nz; k += kDwThreads) {
                int r = k / cpl;
                r = r < cur.vr0 ? r : r + cur.nvr;
                reinterpret_cast<u32x4 *>(sx + kDwGuard + r * R)[k % cpl] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if ((vok >> q) & 1u)
                *reinterpret_cast<u32x4 *>(sx + kDwGuard + (cur.vr0 + chr[q]) * R + chc[q]) = v[q];
        if (threadIdx.x < NE) seff[threadIdx.x] = eidx >= 0 ? ew : _Float16(0.0f);
        const float bv = bias ? float(braw) : 0.0f;
        __syncthreads();
        // sub-kernels in registers: column-tap pairs for the packed dot products, and
        // the odd last column tap (T2 odd) as float
        h2 wp[S][S][T1][NP > 0 ? NP : 1];
        float wt[S][S][T1];
#pragma unroll
        for (int rh = 0; rh < S; ++rh)
#pragma unroll
            for (int rwp = 0; rwp < S; ++rwp)
#pragma unroll
                for (int a = 0; a < T1; ++a) {
                    const _Float16 *e = seff + ((rh * S + rwp) * T1 + a) * T2;
#pragma unroll
                    for (int m = 0; m < NP; ++m) wp[rh][rwp][a][m] = h2{e[2 * m], e[2 * m + 1]};
                    wt[rh][rwp][a] = (T2 & 1) ? float(e[T2 - 1]) : 0.0f;
                }

        // ---- load the next unit ahead, if there is one ----
        const int tn = t + int(gridDim.x);
        const Unit nxt = unit_of(min(tn, p.units - 1));
        if (tn < p.units) issue(nxt);

        // ---- compute and store the current unit ----
        const int jrows = cur.j1hi - cur.j1lo + 1;
        _Float16 *const yplane = y + size_t(cur.c) * p.O1 * p.O2;
        for (int seg = seg0, jr = jr0; jr < jrows;) {
            const int j1 = cur.j1lo + jr;
            const _Float16 *row0 = sx + kDwGuard + jr * R + (seg * JC + p.lo2);
#pragma unroll
            for (int rh = 0; rh < S; ++rh) {
                const int oh = S * j1 + rh;
                // this row phase's T1 input rows, XW columns from the segment's start
                const _Float16 *win = row0 + p.a0_1[rh] * R;
                _Float16 xs[T1][XW];
#pragma unroll
                for (int a = 0; a < T1; ++a)
#pragma unroll
                    for (int q = 0; q < XW; ++q) xs[a][q] = win[a * R + q];
                float out[OC];
#pragma unroll
                for (int rwp = 0; rwp < S; ++rwp) {
                    const int o2 = (OFF2 >> rwp) & 1;
#pragma unroll
                    for (int je = 0; je < JC; ++je) {
                        float acc = bv;
#pragma unroll
                        for (int a = 0; a < T1; ++a) {
#pragma unroll
                            for (int m = 0; m < NP; ++m)
                                acc = __builtin_amdgcn_fdot2(h2{xs[a][je + o2 + 2 * m], xs[a][je + o2 + 2 * m + 1]},
                                                             wp[rh][rwp][a][m], acc, false);
                            if (T2 & 1) acc += float(xs[a][je + o2 + T2 - 1]) * wt[rh][rwp][a];
                        }
                        out[je * S + rwp] = acc;
                    }
                }
                if (!p.act.identity()) {
#pragma unroll
                    for (int e = 0; e < OC; ++e) out[e] = p.act(out[e]);
                }
                if (oh < cur.oh1) {
                    _Float16 *yr = yplane + size_t(oh) * p.O2 + seg * OC;
                    if (seg * OC + OC <= p.O2 && (reinterpret_cast<uintptr_t>(yr) % 16 == 0)) {
                        u32x4 o;
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            o[k] = __builtin_bit_cast(unsigned, __builtin_convertvector(f2{out[2 * k], out[2 * k + 1]}, h2));
                        *reinterpret_cast<u32x4 *>(yr) = o;
                    } else {
#pragma unroll
                        for (int e = 0; e < OC; ++e)
                            if (seg * OC + e < p.O2) yr[e] = _Float16(out[e]);
                    }
                }
            }
            seg += dseg;
            jr += djr;
            if (seg >= segs) {
                seg -= segs;
                ++jr;
            }
        }
        __syncthreads();  // the stage and seff are rewritten next
        if (tn >= p.units) break;
        t = tn;
        cur = nxt;
    }
}

struct DwPlan {
    DwArgs a;
    int S, T1, T2, off2;  // off2: bit r = column window offset of residue r
    int nq;               // 16-byte input chunks per thread that stage one band
    size_t lds_bytes;     // staged band
};

// Per axis: the run of input offsets beta each residue reads, widened to a common
// length T; lo and the per-residue offsets a0 place every run inside one staged window.
bool axis_windows(const Geom &g, int ax, int S, int *T, int *lo, int *hi, int *a0)
{
    int bmin[kDwMaxS], nt[kDwMaxS];
    int t = 0;
    for (int r = 0; r < S; ++r) {
        AxisPhase ph;
        if (!axis_phase(g, ax, r, &ph)) return false;
        nt[r] = ph.ntaps;
        if (!ph.ntaps) continue;
        // taps by ascending k have descending beta; a run must have step 1
        if (ph.ntaps > 1 && ph.beta[0] - ph.beta[1] != 1) return false;
        bmin[r] = ph.beta[ph.ntaps - 1];
        t = std::max(t, ph.ntaps);
    }
    if (t == 0) return false;  // no tap reaches any output: the generic kernel handles it
    bool any = false;
    for (int r = 0; r < S; ++r)
        if (nt[r]) {
            *lo = any ? std::min(*lo, bmin[r]) : bmin[r];
            *hi = any ? std::max(*hi, bmin[r] + t - 1) : bmin[r] + t - 1;
            any = true;
        }
    for (int r = 0; r < S; ++r) a0[r] = nt[r] ? bmin[r] - *lo : 0;
    *T = t;
    return true;
}

// Compiled (S, T, column offset pattern) combinations.
bool dw_compiled(int S, int T1, int T2, int off2)
{
    if (T1 != T2) return false;
    if (S == 1) return off2 == 0 && (T1 == 3 || T1 == 5);
    if (S == 2) return T1 >= 1 && T1 <= 3;  // every off2 in [0, 4)
    if (S == 4) return T1 == 2 && (off2 == 0 || off2 == 12);
    return false;
}

bool make_dwplan(const Geom &g, ct_dtype dt, bool cl, const void *x, DwPlan *pl)
{
    if (dt != CT_FLOAT16 || cl || g.Cg != 1 || g.Mg != 1 || g.G < 2 || g.nsp > 2 || g.L[0] != 1 ||
        g.O[0] != 1 || g.L[1] * g.L[2] == 0 || g.L[1] * g.L[2] >= (1ll << 31))
        return false;
    const int S = int(g.s[2]);
    if (g.s[1] != S || (S != 1 && S != 2 && S != 4)) return false;
    DwArgs &a = pl->a;
    std::memset(&a, 0, sizeof(a));
    int T1, T2, hi1, hi2, a0_2[kDwMaxS];
    if (!axis_windows(g, 1, S, &T1, &a.lo1, &hi1, a.a0_1) || !axis_windows(g, 2, S, &T2, &a.lo2, &hi2, a0_2))
        return false;
    int off2 = 0;
    for (int r = 0; r < S; ++r) {
        if (a0_2[r] > 1) return false;
        off2 |= a0_2[r] << r;
    }
    if (!dw_compiled(S, T1, T2, off2)) return false;
    a.C = int(g.C);
    a.L1 = int(g.L[1]);
    a.L2 = int(g.L[2]);
    a.O1 = int(g.O[1]);
    a.O2 = int(g.O[2]);
    a.K1 = int(g.K[1]);
    a.K2 = int(g.K[2]);
    a.b1 = int(g.b[1]);
    a.b2 = int(g.b[2]);
    a.d1 = int(g.d[1]);
    a.d2 = int(g.d[2]);
    a.span1 = hi1 - a.lo1 + 1;
    const int JC = 8 / S;
    const int segs = int((g.O[2] + 7) / 8);
    // rows are staged as 16-byte chunks: rows of a multiple of 8 elements, aligned X; the
    // leading guard must cover the leftmost read
    if (g.L[2] % 8 != 0 || reinterpret_cast<uintptr_t>(x) % 16 != 0 || -a.lo2 > kDwGuard) return false;
    // row stride: the zeros after a row cover reads left of the next row (lo2) and reads
    // right of this one (last segment, widest phase window)
    a.row_w = (std::max<int>(int(g.L[2]) - a.lo2, segs * JC + hi2) + 7) / 8 * 8;
    const int64_t cpl = g.L[2] / 8;
    auto rows_for = [&](int b) { return (b + S - 1) / S - 1 + a.span1; };
    auto bytes_for = [&](int b) { return (int64_t(kDwGuard) + int64_t(rows_for(b)) * a.row_w) * 2; };
    auto fits = [&](int b) { return bytes_for(b) <= kDwStageBytes && rows_for(b) * cpl <= kDwMaxChunks * kDwThreads; };
    // band of output rows (a multiple of S) whose staged rows fit
    int band = int((g.O[1] + S - 1) / S) * S;
    while (band > S && !fits(band)) band = (band / 2 + S - 1) / S * S;
    if (!fits(band)) return false;
    // few planes: more bands so the grid still fills the chip
    while (band >= 8 * S && g.N * g.C * ((g.O[1] + band - 1) / band) < 2048) band = (band / 2 + S - 1) / S * S;
    a.band = band;
    a.nbands = int((g.O[1] + band - 1) / band);
    a.nrows = rows_for(band);
    const int64_t units = g.N * g.C * a.nbands;
    if (units <= 0 || units > (1ll << 31) - 1) return false;
    a.units = int(units);
    a.stage_elems = int(bytes_for(band) / 2);
    pl->lds_bytes = size_t(bytes_for(band));
    pl->nq = int((a.nrows * cpl + kDwThreads - 1) / kDwThreads);
    pl->S = S;
    pl->T1 = T1;
    pl->T2 = T2;
    pl->off2 = off2;
    return true;
}

// Resident blocks of one kernel instance on the current device (occupancy x CUs),
// remembered per (kernel, dynamic LDS bytes, device).
int resident_blocks(const void *fn, size_t lds)
{
    struct Entry {
        const void *fn;
        size_t lds;
        int dev, blocks;
    };
    static thread_local Entry cache[32];
    static thread_local int ncache = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    for (int i = 0; i < std::min(ncache, 32); ++i)
        if (cache[i].fn == fn && cache[i].lds == lds && cache[i].dev == dev) return cache[i].blocks;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kDwThreads, lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int blocks = std::max(1, per_cu) * std::max(1, cus);
    cache[ncache % 32] = Entry{fn, lds, dev, blocks};
    ++ncache;
    return blocks;
}

template <int S, int T1, int T2, int OFF2, int NQ>
void launch_t(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    auto fn = depthwise_kernel<S, T1, T2, OFF2, NQ>;
    const int res = resident_blocks(reinterpret_cast<const void *>(fn), pl.lds_bytes);
    const int grid = std::min(pl.a.units, res > 0 ? res : pl.a.units);
    hipLaunchKernelGGL(fn, dim3(unsigned(grid)), dim3(kDwThreads), pl.lds_bytes, st,
                       static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w),
                       static_cast<const _Float16 *>(bias), static_cast<_Float16 *>(y), pl.a);
}

template <int S, int T1, int T2, int OFF2>
void launch_o(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    if (pl.nq <= 2) launch_t<S, T1, T2, OFF2, 2>(pl, x, w, bias, y, st);
    else launch_t<S, T1, T2, OFF2, kDwMaxChunks>(pl, x, w, bias, y, st);
}

template <int S, int T>
void launch_s2(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    switch (pl.off2) {
    case 0: launch_o<S, T, T, 0>(pl, x, w, bias, y, st); break;
    case 1: launch_o<S, T, T, 1>(pl, x, w, bias, y, st); break;
    case 2: launch_o<S, T, T, 2>(pl, x, w, bias, y, st); break;
    default: launch_o<S, T, T, 3>(pl, x, w, bias, y, st); break;
    }
}

}  // namespace

bool depthwise_supports(const Geom &g, ct_dtype dt, bool cl, const void *x)
{
    DwPlan pl;
    return make_dwplan(g, dt, cl, x, &pl);
}

ct_status launch_depthwise(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w, const void *bias,
                           void *y, const Act &act, hipStream_t st, std::string *err)
{
    DwPlan pl;
    if (!make_dwplan(g, dt, cl, x, &pl)) {
        *err = "depthwise kernel cannot serve this call";
        return CT_EUNSUPPORTED;
    }
    pl.a.act = act;
    mark_before(st);
    if (pl.S == 1 && pl.T1 == 3) launch_o<1, 3, 3, 0>(pl, x, w, bias, y, st);
    else if (pl.S == 1) launch_o<1, 5, 5, 0>(pl, x, w, bias, y, st);
    else if (pl.S == 2 && pl.T1 == 1) launch_s2<2, 1>(pl, x, w, bias, y, st);
    else if (pl.S == 2 && pl.T1 == 2) launch_s2<2, 2>(pl, x, w, bias, y, st);
    else if (pl.S == 2) launch_s2<2, 3>(pl, x, w, bias, y, st);
    else if (pl.off2 == 0) launch_o<4, 2, 2, 0>(pl, x, w, bias, y, st);
    else launch_o<4, 2, 2, 12>(pl, x, w, bias, y, st);
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("depthwise kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
