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
// makes 8 columns of one output row at a time: it reads T1 input rows at the row phase's
// offset, and each column phase applies its T1 x T2 sub-kernel (held in registers) at its
// own column offset within that window.  Blocks are persistent and issue the global loads
// of their next unit before computing the current one.  Products of float16 values are
// exact in float32; pairs of column taps are summed by a packed float16 dot product with
// float32 accumulation.  Each result is rounded once to float16 and a row of 8 is written
// as one 16-byte store; consecutive threads write consecutive pieces of Y, so with rows
// of whole pieces the stores are streaming stores of whole lines.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <type_traits>

#include "ct_internal.hpp"

namespace ct {
namespace {

constexpr int kDwThreads = 256;
constexpr int kDwMaxS = 4;                                 // largest stride served
constexpr int kDwMaxChunks = 8;                              // 16-byte input chunks per thread per unit
constexpr int kDwStageBytes = kDwMaxChunks * kDwThreads * 16;  // staged band (float16), upper bound
constexpr int kDwGuard = 8;                                    // zero elements ahead of staged row 0
constexpr int kDwMaxS0 = 4;                                    // largest stride on the first axis (rank 3)
constexpr int kDwMaxPlanes = 3;                                // staged input planes per unit (rank 3)

struct DwArgs {
    int C, L1, L2, O1, O2, K1, K2, b1, b2, d1, d2;
    int band, nbands, units;
    int row_w;     // staged row stride R in elements (multiple of 8): L2 inputs, then zeros
    int nrows;     // staged rows per unit
    int lo1, lo2;  // smallest input offset beta over all phases, per axis
    int span1;     // staged rows beyond the band's input rows: hi1 - lo1 + 1
    int stage_elems;    // halves per stage buffer (multiple of 8)
    int sh;             // column shift of the staged rows (0..3): window reads start 8-byte aligned
    int a0_1[kDwMaxS];  // per row residue: its window's row offset from lo1
    // first axis (rank 3; a single plane otherwise): output plane o0 = s0 * j0 + r0 reads
    // input planes i0 = j0 + be00(r0) - u * bs0 with kernel index k00(r0) + u * ks0 for
    // u < nt0(r0); the per-residue values are 16-bit fields r0 of these words (a table
    // indexed at run time would be read from memory inside the unit loop).  A unit takes
    // every residue of one j0: it stages the npl input planes j0 + bmin0 ... (the union
    // of its residues' taps) and writes the s0 output planes s0 * j0 + r0.
    int L0, O0, K0, s0, ks0, bs0;
    unsigned long long nt0w, k00w, be00w;
    int J0, bmin0, npl;
    int slot_elems;  // halves per staged plane (the planes are staged one after another)
    Act act;         // output activation
};

// T0: the most first-axis taps of an output plane (rank 3); 0 for ranks 1 and 2, whose
// units read one plane and skip the first-axis bookkeeping.  CG: channels per group
// (C/group = M/group; ranks 1 and 2): a unit stages the CG input planes of one group and
// writes its CG output planes, each the sum over the group's input channels (CG = 1:
// depthwise).
template <int S, int T1, int T2, int OFF2, int NQ, int T0, int CG = 1>
__global__ __launch_bounds__(kDwThreads) void depthwise_kernel(const _Float16 *__restrict__ x,
                                                               const _Float16 *__restrict__ w,
                                                               const _Float16 *__restrict__ bias,
                                                               _Float16 *__restrict__ y, DwArgs p)
{
    constexpr int OC = 8;               // output columns per thread
    constexpr int JC = OC / S;          // input-grid columns they span
    constexpr int NE = S * S * T1 * T2;  // sub-kernel entries over all phases
    static_assert(T0 == 0 || CG == 1, "groups of channels for ranks 1 and 2 only");
    constexpr bool GRP = CG > 1;
    constexpr bool MULTI = T0 > 0 || GRP;  // several staged planes and output planes per unit
    // per unit: input planes read per output plane, staged planes, output planes (at most)
    constexpr int NT0 = T0 > 0 ? T0 : CG;
    constexpr int NPL = T0 > 0 ? kDwMaxPlanes : CG;
    constexpr int NRS = T0 > 0 ? kDwMaxS0 : CG;
    // column offset of residue r's window (0 or 1), fixed at compile time so every
    // register index below is a constant; row offsets are LDS addresses and stay runtime
    constexpr int MAXO2 = (OFF2 != 0) ? 1 : 0;
    constexpr int XW = JC + T2 - 1 + MAXO2;  // window columns per row
    constexpr int NP = T2 / 2;               // column-tap pairs per sub-kernel row
    static_assert(NE <= kDwThreads, "sub-kernels larger than the block");
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    // Stage: kDwGuard + sh zero elements, then nrows rows of R elements each: input
    // columns [0, L2) followed by zeros up to R.  Reads left of a row land in the previous
    // row's zeros (or the leading guard), reads right of it in its own.  The shift sh
    // makes kDwGuard + sh + lo2 a multiple of 4, so with S <= 2 every window read starts
    // on an 8-byte boundary (LDS reads that are not naturally aligned stall).
    extern __shared__ __attribute__((aligned(16))) unsigned char dw_lds[];
    _Float16 *const sx = reinterpret_cast<_Float16 *>(dw_lds);
    __shared__ _Float16 seff[NRS * NT0 * NE];  // sub-kernels of the unit's first-axis residues and taps
    __shared__ float sbias[NRS];                // several output planes: their bias

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
    // item (output row of the band, segment of 8 columns), segments fastest: the lanes of
    // a wave cover consecutive stretches of Y
    const int seg0 = threadIdx.x % segs, or0 = threadIdx.x / segs;
    const int dseg = kDwThreads % segs, dor = kDwThreads / segs;
    // whole rows of 16-byte pieces: consecutive items are consecutive in Y, so a wave's
    // stores cover whole lines and go out as streaming stores (Y is read by no block)
    const bool stream = p.O2 % OC == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;

    // 16-bit field r of a per-residue word
    auto field = [](unsigned long long wd, int r) { return int(short((wd >> (16 * r)) & 0xffffu)); };
    struct Unit {
        int c, pc, ch, oh0, oh1, j1lo, j1hi, ilo, vr0, nvr;
        int j0, i0, live;  // rank 3: phase-grid plane, input plane of slot 0; bit v: slot v is inside X
    };
    auto unit_of = [&](int t) {
        Unit u;
        const int band = t % p.nbands;
        u.c = t / p.nbands;  // ranks 1-2: the plane; rank 3: (image, channel, j0)
        if constexpr (!MULTI) {
            u.pc = u.c;
            u.j0 = u.i0 = 0;
            u.live = 1;
        } else if constexpr (GRP) {  // u.c: (image, group); its planes are u.c * CG + j
            u.pc = u.c;
            u.j0 = u.i0 = 0;
            u.live = (1 << CG) - 1;
        } else {
            u.pc = u.c / p.J0;  // image and channel
            u.j0 = u.c - u.pc * p.J0;
            u.i0 = u.j0 + p.bmin0;
            u.live = 0;
#pragma unroll
            for (int v = 0; v < NPL; ++v)
                if (v < p.npl && u.i0 + v >= 0 && u.i0 + v < p.L0) u.live |= 1 << v;
        }
        u.ch = GRP ? u.pc % (p.C / CG) : u.pc % p.C;  // grouped: the group
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
    // Chunk k of a unit is the (k % nch)-th 16-byte piece of the valid rows of staged plane
    // k / nch (nch pieces per plane); dsto[q] is where chunk q of the thread goes in LDS.
    u32x4 v[NQ];
    int dsto[NQ];     // rank 3
    unsigned vok = 0;  // one plane: bit q, chunk q holds input
    // one plane: chunk k = threadIdx.x + q * kDwThreads is the k-th 16-byte piece of the
    // band's valid input rows, row chr[q] of them at column chc[q], whatever the unit
    int chr[NQ], chc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int k = threadIdx.x + q * kDwThreads;
        chr[q] = k / cpl;
        chc[q] = (k - chr[q] * cpl) * 8;
    }
    _Float16 ew[NRS][NT0], braw;  // several output planes: thread r < NRS loads plane r's bias
    auto issue = [&](const Unit &u) {
        const _Float16 *xp = x + size_t(u.pc) * p.L0 * plane_in;  // the image and channel
        const int nch = u.nvr * cpl;
        if constexpr (!MULTI) {
            const _Float16 *xb = xp + (u.ilo + u.vr0) * p.L2;  // first valid row: contiguous from here
            ew[0][0] = w[size_t(u.ch) * p.K1 * p.K2 + max(eidx, 0)];
            braw = *(bias ? bias + u.ch : xp);  // used only with a bias
            vok = 0;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int k = threadIdx.x + q * kDwThreads;
                const bool ok = k < nch;
                v[q] = *reinterpret_cast<const u32x4 *>(ok ? xb + 8 * k : xp);
                vok |= unsigned(ok) << q;
            }
            return;
        }
        // the sub-kernel entries of every residue's taps (threads below NE); grouped: of
        // output channel r of the group and its input channel v0, w[g CG + v0][r]
        const size_t plane_w = size_t(p.K1) * p.K2;
        if (threadIdx.x < NE) {
#pragma unroll
            for (int r = 0; r < NRS; ++r)
#pragma unroll
                for (int v0 = 0; v0 < NT0; ++v0) {
                    if constexpr (GRP) {
                        ew[r][v0] = w[(size_t(u.ch * CG + v0) * CG + r) * plane_w + max(eidx, 0)];
                    } else {
                        const bool okw = r < p.s0 && v0 < field(p.nt0w, r);
                        ew[r][v0] = w[(size_t(u.ch) * p.K0 + (okw ? field(p.k00w, r) + v0 * p.ks0 : 0)) * plane_w + max(eidx, 0)];
                    }
                }
        }
        braw = *(bias ? bias + (GRP ? u.ch * CG + min(int(threadIdx.x), NRS - 1) : u.ch) : xp);  // only with a bias
        const UDiv dn(nch > 0 ? nch : 1), dc(cpl);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int k = threadIdx.x + q * kDwThreads;
            const int sl = dn.div(k), kk = k - sl * nch;
            const bool ok = nch > 0 && sl < p.npl && ((u.live >> sl) & 1);
            const int r = dc.div(kk), c8 = (kk - r * cpl) * 8;
            // rows ilo + vr0 + r of input plane i0 + sl, contiguous from the first valid row
            const _Float16 *src = xp + (size_t(u.i0 + sl) * plane_in + size_t(u.ilo + u.vr0 + r) * p.L2 + c8);
            v[q] = *reinterpret_cast<const u32x4 *>(ok ? src : xp);
            dsto[q] = ok ? sl * p.slot_elems + kDwGuard + p.sh + (u.vr0 + r) * R + c8 : -1;
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
        // (in every plane that is read; planes of no tap are neither staged nor read)
        {
            const int nz = (p.nrows - cur.nvr) * cpl;
#pragma unroll
            for (int v0 = 0; v0 < NPL; ++v0) {
                if (MULTI && !((cur.live >> v0) & 1)) continue;
                _Float16 *const sp = sx + v0 * p.slot_elems + kDwGuard;
                for (int k = threadIdx.x; k < nz; k += kDwThreads) {
                    int r = k / cpl;
                    r = r < cur.vr0 ? r : r + cur.nvr;
                    reinterpret_cast<u32x4 *>(sp + r * R)[k % cpl] = u32x4{0u, 0u, 0u, 0u};
                    // the shifted row's last sh elements spill into the next chunk
                    if (p.sh > 0 && k % cpl == cpl - 1)
                        reinterpret_cast<u32x4 *>(sp + r * R)[cpl] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (!MULTI ? ((vok >> q) & 1u) != 0 : dsto[q] >= 0) {
                _Float16 *dst = !MULTI ? sx + kDwGuard + p.sh + (cur.vr0 + chr[q]) * R + chc[q] : sx + dsto[q];
                const u32x4 vq = v[q];
                if (p.sh == 0) {  // 16-byte aligned
                    *reinterpret_cast<u32x4 *>(dst) = vq;
                } else if (p.sh == 2) {  // 4-byte aligned
#pragma unroll
                    for (int k = 0; k < 4; ++k) reinterpret_cast<unsigned *>(dst)[k] = vq[k];
                } else {  // 2-byte aligned: a half, three aligned pairs, a half
                    *reinterpret_cast<unsigned short *>(dst) = (unsigned short)(vq[0] & 0xffffu);
#pragma unroll
                    for (int k = 0; k < 3; ++k)
                        reinterpret_cast<unsigned *>(dst + 1)[k] = (vq[k] >> 16) | (vq[k + 1] << 16);
                    *reinterpret_cast<unsigned short *>(dst + 7) = (unsigned short)(vq[3] >> 16);
                }
            }
        if (MULTI && threadIdx.x < NRS) sbias[threadIdx.x] = bias ? float(braw) : 0.0f;
        if (threadIdx.x < NE) {
#pragma unroll
            for (int r = 0; r < NRS; ++r)
#pragma unroll
                for (int v0 = 0; v0 < NT0; ++v0)
                    if (T0 == 0 || r < p.s0)
                        seff[(r * NT0 + v0) * NE + threadIdx.x] =
                            eidx >= 0 && (T0 == 0 || v0 < field(p.nt0w, r)) ? ew[r][v0] : _Float16(0.0f);
        }
        __syncthreads();
        // ---- load the next unit ahead, if there is one ----
        const int tn = t + int(gridDim.x);
        const Unit nxt = unit_of(min(tn, p.units - 1));
        if (tn < p.units) issue(nxt);

        // ---- compute and store the current unit ----
        // Each item is one output row oh = S * j1 + rh: its row phase rh selects the
        // window's row offset and the sub-kernels (selects over the S phases in registers)
        const int orows = cur.oh1 - cur.oh0;  // oh0 is a multiple of S: oh0 = S * j1lo
        int a0r[S];
#pragma unroll
        for (int r = 0; r < S; ++r) a0r[r] = p.a0_1[r] * R;
        // rank 3: output plane s0 * j0 + r0 of each first-axis residue r0 in turn; its taps
        // v0 < ntr read staged plane sbase - v0 * bs0
        // grouped: output channel r0 of the group, its taps v0 < CG the group's input planes
        const int nres = T0 > 0 ? p.s0 : CG;
        for (int r0 = 0; r0 < nres; ++r0) {
        const float bv = !MULTI ? (bias ? float(braw) : 0.0f) : sbias[GRP ? r0 : 0];
        _Float16 *yplane = y + (size_t(cur.c) * CG + (GRP ? r0 : 0)) * p.O1 * p.O2;
        int ntr = NT0, sbase = 0;
        if constexpr (T0 > 0) {
            const int o0 = p.s0 * cur.j0 + r0;
            if (o0 >= p.O0) break;
            ntr = field(p.nt0w, r0);
            sbase = field(p.be00w, r0) - p.bmin0;
            yplane = y + (size_t(cur.pc) * p.O0 + o0) * p.O1 * p.O2;
        }
        // sub-kernels in registers: column-tap pairs for the packed dot products, and
        // the odd last column tap (T2 odd) as float (one set per first-axis tap)
        h2 wp[NT0][S][S][T1][NP > 0 ? NP : 1];
        float wt[NT0][S][S][T1];
#pragma unroll
        for (int v0 = 0; v0 < NT0; ++v0)
#pragma unroll
            for (int rh = 0; rh < S; ++rh)
#pragma unroll
                for (int rwp = 0; rwp < S; ++rwp)
#pragma unroll
                    for (int a = 0; a < T1; ++a) {
                        const _Float16 *e = seff + (r0 * NT0 + v0) * NE + ((rh * S + rwp) * T1 + a) * T2;
#pragma unroll
                        for (int m = 0; m < NP; ++m) wp[v0][rh][rwp][a][m] = h2{e[2 * m], e[2 * m + 1]};
                        wt[v0][rh][rwp][a] = (T2 & 1) ? float(e[T2 - 1]) : 0.0f;
                    }
        // copies of the item loop, with and without streaming stores (a store under a
        // run-time choice would be merged with the plain one and lose its cache hint) and
        // with and without an activation (a run-time test in the loop made the compiler
        // shuffle the eight results between registers on every item)
        auto items = [&](auto streaming, auto identity) __attribute__((always_inline)) {
        for (int seg = seg0, orr = or0; orr < orows;) {
            const int jr = orr / S, rh = orr - jr * S;
            // value of row phase rh among S candidates of 32 bits, by byte permutes on its
            // bits: a select would be folded into an indexed load from a private array
            const unsigned sel1 = (rh & 1) ? 0x03020100u : 0x07060504u;  // perm(a, b, .) = b : a
            const unsigned sel2 = (rh & 2) ? 0x03020100u : 0x07060504u;
            auto pick = [&](const auto (&c)[S]) __attribute__((always_inline)) {
                using T = typename std::remove_cv<typename std::remove_reference<decltype(c[0])>::type>::type;
                static_assert(sizeof(T) == 4, "32-bit candidates");
                auto u = [](T v) { return __builtin_bit_cast(unsigned, v); };
                if constexpr (S == 1) {
                    return c[0];
                } else if constexpr (S == 2) {
                    return __builtin_bit_cast(T, __builtin_amdgcn_perm(u(c[0]), u(c[1]), sel1));
                } else {
                    static_assert(S == 4, "strides 1, 2 and 4");
                    const unsigned lo = __builtin_amdgcn_perm(u(c[0]), u(c[1]), sel1);
                    const unsigned hi = __builtin_amdgcn_perm(u(c[2]), u(c[3]), sel1);
                    return __builtin_bit_cast(T, __builtin_amdgcn_perm(lo, hi, sel2));
                }
            };
            const int a0 = pick(a0r);
            // this row phase's T1 input rows, XW columns from the segment's start
            const _Float16 *win = sx + kDwGuard + p.sh + jr * R + a0 + (seg * JC + p.lo2);
            float out[OC];
#pragma unroll
            for (int e = 0; e < OC; ++e) out[e] = bv;
#pragma unroll
            for (int v0 = 0; v0 < NT0; ++v0) {
                const int slot = GRP ? v0 : sbase - v0 * p.bs0;
                if (T0 > 0 && !(v0 < ntr && ((cur.live >> slot) & 1))) continue;  // uniform over the block
                h2 ws[S][T1][NP > 0 ? NP : 1];
                float wts[S][T1];
#pragma unroll
                for (int rwp = 0; rwp < S; ++rwp)
#pragma unroll
                    for (int a = 0; a < T1; ++a) {
#pragma unroll
                        for (int m = 0; m < NP; ++m) {
                            h2 c[S];
#pragma unroll
                            for (int r = 0; r < S; ++r) c[r] = wp[v0][r][rwp][a][m];
                            ws[rwp][a][m] = pick(c);
                        }
                        float c[S];
#pragma unroll
                        for (int r = 0; r < S; ++r) c[r] = wt[v0][r][rwp][a];
                        wts[rwp][a] = pick(c);
                    }
                const _Float16 *const wn = win + slot * p.slot_elems;
                _Float16 xs[T1][XW];
                if constexpr (S <= 2) {
                    // 8-byte aligned: whole 4-element pieces
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                    constexpr int NV = (XW + 3) / 4;
#pragma unroll
                    for (int a = 0; a < T1; ++a) {
                        const u32x2 *wv = reinterpret_cast<const u32x2 *>(wn + a * R);
#pragma unroll
                        for (int v = 0; v < NV; ++v) {
                            const u32x2 pv = wv[v];
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (4 * v + e < XW)
                                    xs[a][4 * v + e] = __builtin_bit_cast(_Float16, (unsigned short)((pv[e >> 1] >> (16 * (e & 1))) & 0xffffu));
                        }
                    }
                } else {
#pragma unroll
                    for (int a = 0; a < T1; ++a)
#pragma unroll
                        for (int q = 0; q < XW; ++q) xs[a][q] = wn[a * R + q];
                }
#pragma unroll
                for (int rwp = 0; rwp < S; ++rwp) {
                    const int o2 = (OFF2 >> rwp) & 1;
#pragma unroll
                    for (int je = 0; je < JC; ++je) {
                        float acc = out[je * S + rwp];
#pragma unroll
                        for (int a = 0; a < T1; ++a) {
#pragma unroll
                            for (int m = 0; m < NP; ++m)
                                acc = __builtin_amdgcn_fdot2(h2{xs[a][je + o2 + 2 * m], xs[a][je + o2 + 2 * m + 1]},
                                                             ws[rwp][a][m], acc, false);
                            if (T2 & 1) acc += float(xs[a][je + o2 + T2 - 1]) * wts[rwp][a];
                        }
                        out[je * S + rwp] = acc;
                    }
                }
            }
            if constexpr (!decltype(identity)::value) {
#pragma unroll
                for (int e = 0; e < OC; ++e) out[e] = p.act(out[e]);
            }
            _Float16 *yr = yplane + size_t(cur.oh0 + orr) * p.O2 + seg * OC;
            if (seg * OC + OC <= p.O2 && (reinterpret_cast<uintptr_t>(yr) % 16 == 0)) {
                u32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    o[k] = __builtin_bit_cast(unsigned, __builtin_convertvector(f2{out[2 * k], out[2 * k + 1]}, h2));
                if constexpr (decltype(streaming)::value)
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(yr));
                else
                    *reinterpret_cast<u32x4 *>(yr) = o;
            } else {
#pragma unroll
                for (int e = 0; e < OC; ++e)
                    if (seg * OC + e < p.O2) yr[e] = _Float16(out[e]);
            }
            seg += dseg;
            orr += dor;
            if (seg >= segs) {
                seg -= segs;
                ++orr;
            }
        }
        };
        const bool idn = p.act.identity();
        if (stream && idn)
            items(std::true_type{}, std::true_type{});
        else if (stream)
            items(std::true_type{}, std::false_type{});
        else if (idn)
            items(std::false_type{}, std::true_type{});
        else
            items(std::false_type{}, std::false_type{});
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
    int T0;               // kernel's T0: most first-axis taps of a residue (rank 3), else 0
    int CG;               // channels per group (1: depthwise)
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
bool dw_compiled(int S, int T1, int T2, int off2, int T0, int CG)
{
    if (T1 != T2) return false;
    // groups of 2, 4 or 8 channels (ranks 1 and 2): stride 2 with up to 2 taps per phase
    // and row, and with 3 or stride 1 with 3 for groups up to 4 (registers)
    if (CG > 1)
        return T0 == 0 && (CG == 2 || CG == 4 || CG == 8) &&
               ((S == 2 && T1 <= 2) || (CG <= 4 && ((S == 2 && T1 == 3) || (S == 1 && T1 == 3 && off2 == 0))));
    // rank 3 (1 to 3 first-axis taps per output plane): stride 2 with up to 3 taps per
    // row and column phase, stride 1 with 3 taps
    if (T0 >= 1 && T0 <= 3) return (S == 2 && T1 >= 1 && T1 <= 3) || (S == 1 && T1 == 3 && off2 == 0);
    if (T0 != 0) return false;
    if (S == 1) return off2 == 0 && (T1 == 3 || T1 == 5);
    if (S == 2) return T1 >= 1 && T1 <= 3;  // every off2 in [0, 4)
    if (S == 4) return T1 == 2 && (off2 == 0 || off2 == 12);
    return false;
}

bool make_dwplan(const Geom &g, ct_dtype dt, bool cl, const void *x, DwPlan *pl)
{
    if (dt != CT_FLOAT16 || cl || g.Cg != g.Mg || g.Cg > 8 || (g.Cg > 1 && g.nsp == 3) || g.G < 2 ||
        g.L[0] * g.L[1] * g.L[2] == 0 ||
        g.O[0] == 0 || g.L[0] * g.L[1] * g.L[2] >= (1ll << 31) || g.O[0] >= (1ll << 31))
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
    // first axis (a single plane below rank 3): per residue its taps as a progression
    if (g.s[0] > kDwMaxS0) return false;
    const int64_t gs0 = std::__gcd(g.s[0], g.d[0]);
    a.ks0 = int(g.s[0] / gs0);
    a.bs0 = int(g.d[0] / gs0);
    int T0 = 0, bmin0 = 0, bmax0 = 0;
    bool any0 = false;
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
        if (ph.ntaps) {  // input planes j0 + beta of this residue: beta in [beta[last], beta[0]]
            bmin0 = any0 ? std::min(bmin0, ph.beta[ph.ntaps - 1]) : ph.beta[ph.ntaps - 1];
            bmax0 = any0 ? std::max(bmax0, ph.beta[0]) : ph.beta[0];
            any0 = true;
        }
    }
    if (T0 == 0) return false;  // no tap reaches any output plane: the generic kernel handles it
    a.L0 = int(g.L[0]);
    a.O0 = int(g.O[0]);
    a.K0 = int(g.K[0]);
    a.s0 = int(g.s[0]);
    a.J0 = int((g.O[0] + g.s[0] - 1) / g.s[0]);
    a.bmin0 = bmin0;
    a.npl = bmax0 - bmin0 + 1;  // staged planes per unit: the union of the residues' taps
    pl->T0 = g.nsp == 3 ? T0 : 0;
    pl->CG = int(g.Cg);
    if (!dw_compiled(S, T1, T2, off2, pl->T0, pl->CG)) return false;
    if (pl->T0 > 0 && a.npl > kDwMaxPlanes) return false;
    if (pl->CG > 1) {  // a group's CG input planes, image by image: plane (n G + g) CG + j
        a.L0 = pl->CG;
        a.npl = pl->CG;
    }
    const int npl = pl->T0 > 0 || pl->CG > 1 ? a.npl : 1;  // staged planes
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
    // shift of the staged rows: kDwGuard + sh + lo2 a multiple of 4 (S <= 2; S = 4 reads
    // 2-element runs and keeps sh = 0)
    a.sh = S <= 2 ? ((-(kDwGuard + a.lo2)) % 4 + 4) % 4 : 0;
    // the shifted row (and its zeroing, one chunk longer) stays inside the row stride
    a.row_w = (std::max<int>({int(g.L[2]) - a.lo2, segs * JC + hi2, a.sh > 0 ? int(g.L[2]) + 8 : 0}) + 7) / 8 * 8;
    const int64_t cpl = g.L[2] / 8;
    auto rows_for = [&](int b) { return (b + S - 1) / S - 1 + a.span1; };
    // + 8: the last row shifted by sh, and the 4-element window reads past a row's end
    auto bytes_for = [&](int b) { return (int64_t(kDwGuard) + int64_t(rows_for(b)) * a.row_w + 8) * 2; };
    // (npl planes of them)
    auto fits = [&](int b) {
        return npl * bytes_for(b) <= kDwStageBytes && npl * rows_for(b) * cpl <= kDwMaxChunks * kDwThreads;
    };
    // band of output rows (a multiple of S) whose staged rows fit
    int band = int((g.O[1] + S - 1) / S) * S;
    while (band > S && !fits(band)) band = (band / 2 + S - 1) / S * S;
    if (!fits(band)) return false;
    // few planes: more bands so the grid still fills the chip
    const int64_t planes = g.N * (g.C / pl->CG) * (pl->T0 > 0 ? a.J0 : 1);  // units per band
    while (band >= 8 * S && planes * ((g.O[1] + band - 1) / band) < 2048) band = (band / 2 + S - 1) / S * S;
    a.band = band;
    a.nbands = int((g.O[1] + band - 1) / band);
    a.nrows = rows_for(band);
    const int64_t units = planes * a.nbands;
    if (units <= 0 || units > (1ll << 31) - 1) return false;
    a.units = int(units);
    a.slot_elems = int(bytes_for(band) / 2);
    a.stage_elems = npl * a.slot_elems;
    pl->lds_bytes = size_t(npl) * size_t(bytes_for(band));
    pl->nq = int((npl * a.nrows * cpl + kDwThreads - 1) / kDwThreads);
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

template <int S, int T1, int T2, int OFF2, int NQ, int T0, int CG>
void launch_t(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    auto fn = depthwise_kernel<S, T1, T2, OFF2, NQ, T0, CG>;
    const int res = resident_blocks(reinterpret_cast<const void *>(fn), pl.lds_bytes);
    const int grid = std::min(pl.a.units, res > 0 ? res : pl.a.units);
    hipLaunchKernelGGL(fn, dim3(unsigned(grid)), dim3(kDwThreads), pl.lds_bytes, st,
                       static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(w),
                       static_cast<const _Float16 *>(bias), static_cast<_Float16 *>(y), pl.a);
}

template <int S, int T1, int T2, int OFF2, int T0, int CG>
void launch_o(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    if constexpr (CG == 1) {  // groups: the large-chunk instance only
        if (pl.nq <= 2) {
            launch_t<S, T1, T2, OFF2, 2, T0, 1>(pl, x, w, bias, y, st);
            return;
        }
    }
    launch_t<S, T1, T2, OFF2, kDwMaxChunks, T0, CG>(pl, x, w, bias, y, st);
}

template <int S, int T, int T0, int CG>
void launch_s2(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    switch (pl.off2) {
    case 0: launch_o<S, T, T, 0, T0, CG>(pl, x, w, bias, y, st); break;
    case 1: launch_o<S, T, T, 1, T0, CG>(pl, x, w, bias, y, st); break;
    case 2: launch_o<S, T, T, 2, T0, CG>(pl, x, w, bias, y, st); break;
    default: launch_o<S, T, T, 3, T0, CG>(pl, x, w, bias, y, st); break;
    }
}

// the compiled instances for T0 first-axis taps and CG channels per group (dw_compiled
// lists them)
template <int T0, int CG = 1>
void launch_all(const DwPlan &pl, const void *x, const void *w, const void *bias, void *y, hipStream_t st)
{
    if (pl.S == 2 && pl.T1 == 1) launch_s2<2, 1, T0, CG>(pl, x, w, bias, y, st);
    else if (pl.S == 2 && pl.T1 == 2) launch_s2<2, 2, T0, CG>(pl, x, w, bias, y, st);
    else if constexpr (CG <= 4) {
        if (pl.S == 1 && pl.T1 == 3) launch_o<1, 3, 3, 0, T0, CG>(pl, x, w, bias, y, st);
        else if (pl.S == 2) launch_s2<2, 3, T0, CG>(pl, x, w, bias, y, st);
        else if constexpr (T0 == 0 && CG == 1) {
            if (pl.S == 1) launch_o<1, 5, 5, 0, 0, 1>(pl, x, w, bias, y, st);
            else if (pl.off2 == 0) launch_o<4, 2, 2, 0, 0, 1>(pl, x, w, bias, y, st);
            else launch_o<4, 2, 2, 12, 0, 1>(pl, x, w, bias, y, st);
        }
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
    if (pl.CG == 2) launch_all<0, 2>(pl, x, w, bias, y, st);
    else if (pl.CG == 4) launch_all<0, 4>(pl, x, w, bias, y, st);
    else if (pl.CG == 8) launch_all<0, 8>(pl, x, w, bias, y, st);
    else if (pl.T0 == 0) launch_all<0>(pl, x, w, bias, y, st);
    else if (pl.T0 == 1) launch_all<1>(pl, x, w, bias, y, st);
    else if (pl.T0 == 2) launch_all<2>(pl, x, w, bias, y, st);
    else launch_all<3>(pl, x, w, bias, y, st);
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("depthwise kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
