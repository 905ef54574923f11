// ct_mphase.hip -- all-phase implicit GEMM for strided float16 transposed convolutions
// with few output channels per group (gfx950 MFMA).
//
// Method (webgpu-kernels "ai.onnx.ConvTranspose" README, Implementation variants: the
// stride-phase route and the implicit-gather GEMM that stores output elements directly).
// The outputs split by residue r modulo the stride on every axis; residue class r of
// outputs o = r + s*j receives the taps k with (r + b - k*d) divisible by s, from the
// inputs i = j + beta_k.  Here one workgroup computes, for a box of phase-grid positions
// j (one plane, 2 or 4 rows, 32 columns) and 64 output channels, EVERY residue class at once:
// its outputs are the whole box o in [s*j_lo, s*(j_lo + extent)) of Y, and every class
// reads the same input window, so the window is loaded once for all classes.
//
//   * The input window of all C/group channels (the union of every class's taps) is
//     loaded once into LDS ([plane][row][column][channel], a 16-byte pad per position),
//     then each wave runs without barriers.
//   * Each of the 4 waves owns up to two residue classes (the host pairs heavy and light
//     classes so the waves' tap counts are close) over the box's 64 or 128 positions and
//     64 output channels: 2 x 2 x (2 or 4) MFMA 32x32 tiles, float32 accumulators.
//   * A step is one tap x 32 input channels: the wave reads its weight fragments straight
//     from the fragment-major packing into registers (a ring of RING steps in flight)
//     and the input fragments of the tap's shifted window from LDS:
//     v_mfma_f32_32x32x16_f16, 16 per step.
//   * Epilogue: the accumulators plus bias, one rounding, go into LDS as the output box,
//     which is then stored as whole contiguous rows with 16-byte vectors (no phase-strided
//     2-byte stores).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <numeric>

#include "ct_internal.hpp"

namespace ct {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTC = 32;             // phase-grid columns per box
constexpr int kSlots = 2;           // residue classes per wave
constexpr int kMaxClass = 8;        // 4 waves x 2 slots
constexpr int kRing = 4;            // steps of weight fragments in flight per wave
constexpr int kBiasBytes = 64 * 4;  // the block's 64 bias values (float32) at the end of LDS
// Boxes of TR phase-grid rows (one 32-position tile per row): 2 rows in 78 KB of LDS, two
// blocks per CU, so one block's window loads and stores overlap the other's MFMAs; or 4
// rows in 158 KB, one block per CU, for windows that need the room.
constexpr int lds_bytes(int tr) { return tr == 2 ? 80 * 1024 - 2048 : 160 * 1024 - 2048; }
constexpr int stage_bytes(int tr) { return lds_bytes(tr) - kBiasBytes; }
constexpr int kHaloVec = 32;        // 16-byte halo loads per thread and round

struct MpArgs {
    int N, C, M, Cg, Mg, G, T, Mgp, Cgp;
    int L[3], O[3], s[3], K[3];
    int J[3];                        // phase-grid extent (residue 0's, the largest)
    int rtiles, ctiles, mtiles, nblocks;
    int bmin[3], HP, HR, HC, pitch;  // input window: origin offset, extents, LDS bytes per position
    int E[3], lgE[3];                // output box extents s0 x s1*4 x s2*32 (powers of two) and their log2
    int cpitch;                      // channels-first staging: halves per channel (box + 8)
    int kstep[3], bstep[3];
    int ntap[3][8], tk0[3][8], tb0[3][8];
    int wave_cls[4][kSlots];         // residue class r0 | r1 << 8 | r2 << 16, or -1
    int tr;                          // phase-grid rows per box (2 or 4)
    Act act;
};

__device__ __forceinline__ int floor_div8(int v) { return v >= 0 ? v / 8 : -((-v + 7) / 8); }

template <bool CL, int TR>
__global__ __launch_bounds__(kThreads, TR == 2 ? 2 : 1) void mphase_kernel(const _Float16 *x, const _Float16 *__restrict__ wf,
                                                                           const _Float16 *__restrict__ bias,
                                                                           _Float16 *__restrict__ y, MpArgs p)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[lds_bytes(TR)];
    float *const sbias = reinterpret_cast<float *>(lds + stage_bytes(TR));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---------------- the box this block computes ----------------
    int rest = blockIdx.x;
    const int ct = rest % p.ctiles;
    rest /= p.ctiles;
    const int rt = rest % p.rtiles;
    rest /= p.rtiles;
    const int j0 = rest % p.J[0];
    rest /= p.J[0];
    const int mt = rest % p.mtiles;
    rest /= p.mtiles;
    const int g = rest % p.G;
    const int n = rest / p.G;
    const int row_lo = rt * TR, col_lo = ct * kTC;
    const int i0o = j0 + p.bmin[0], i1o = row_lo + p.bmin[1], i2o = col_lo + p.bmin[2];
    const int L0 = p.L[0], L1 = p.L[1], L2 = p.L[2];

    // bias of the block's 64 channels, loaded now and staged after the main loop
    const bool bias_ok = bias && tid < 64 && mt * 64 + tid < p.Mg;
    const _Float16 bias_h =
        bias_ok ? bias[g * p.Mg + mt * 64 + tid] : *reinterpret_cast<const _Float16 *>(bias ? bias : x);

    // ---------------- input window of every channel of the group into LDS ----------------
    // zeros where the window lies outside the input
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int pos = p.HP * p.HR * p.HC;
        if constexpr (CL) {
            // 16-byte vectors of 8 channels, channels innermost in both places
            const int cv = p.Cg / 8;
            const int items = pos * cv;
            const UDiv dcv(cv), dhc(p.HC), dhr(p.HR);  // item -> (position, octet) -> (plane, row, column)
            const _Float16 *xg = x + size_t(g) * p.Cg;
            for (int base = 0; base < items; base += kThreads * kHaloVec) {
                u32x4 v[kHaloVec];
#pragma unroll
                for (int k = 0; k < kHaloVec; ++k) {
                    const int u = base + tid + k * kThreads;
                    const int q = dcv.div(u), c8 = u - q * cv;
                    const int qr = dhc.div(q), hc = q - qr * p.HC;
                    const int hp = dhr.div(qr), hr = qr - hp * p.HR;
                    const int i0 = i0o + hp, i1 = i1o + hr, i2 = i2o + hc;
                    const bool ok = u < items && i0 >= 0 && i0 < L0 && i1 >= 0 && i1 < L1 && i2 >= 0 && i2 < L2;
                    const size_t off = ok ? (((size_t(n) * L0 + i0) * L1 + i1) * L2 + i2) * p.C + c8 * 8 : 0;
                    const u32x4 t = *reinterpret_cast<const u32x4 *>((ok ? xg : x) + off);
                    v[k] = ok ? t : zero;
                }
#pragma unroll
                for (int k = 0; k < kHaloVec; ++k) {
                    const int u = base + tid + k * kThreads;
                    if (u < items) {
                        const int q = dcv.div(u), c8 = u - q * cv;
                        *reinterpret_cast<u32x4 *>(lds + q * p.pitch + c8 * 16) = v[k];
                    }
                }
            }
        } else {
            // items (aligned 8-column vector, row, plane, channel octet), vector fastest, so
            // the lanes of one load read consecutive 16-byte pieces of one channel's rows: 8
            // loads of 16 bytes (8 columns of one channel each), transposed into 8 LDS
            // positions x 8 channels
            const int va = floor_div8(i2o);
            const int nvc = floor_div8(i2o + p.HC + 7) - va;
            const int oct = p.Cg / 8;
            const int items = p.HP * p.HR * nvc * oct;
            const UDiv dnv(nvc), dhr(p.HR), dhp(p.HP);  // item -> (vector, row, plane, octet)
            auto split = [&](int u, int &vc, int &hr, int &hp, int &o8) {
                const int t1 = dnv.div(u);
                vc = u - t1 * nvc;
                const int t2 = dhr.div(t1);
                hr = t1 - t2 * p.HR;
                o8 = dhp.div(t2);
                hp = t2 - o8 * p.HP;
            };
            const size_t plane_in = size_t(L0) * L1 * L2;
            const _Float16 *xg = x + (size_t(n) * p.C + size_t(g) * p.Cg) * plane_in;
            constexpr int IT = kHaloVec / 8;
            for (int base = 0; base < items; base += kThreads * IT) {
                u32x4 v[IT][8];
                bool okv[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int u = base + tid + it * kThreads;
                    int vc, hr, hp, o8;
                    split(u, vc, hr, hp, o8);
                    const int i0 = i0o + hp, i1 = i1o + hr, i2 = (va + vc) * 8;
                    const bool ok = u < items && i0 >= 0 && i0 < L0 && i1 >= 0 && i1 < L1 && i2 >= 0 && i2 < L2;
                    const _Float16 *src = ok ? xg + size_t(o8 * 8) * plane_in + (size_t(i0) * L1 + i1) * L2 + i2 : x;
                    const size_t step = ok ? plane_in : 0;
#pragma unroll
                    for (int k = 0; k < 8; ++k) v[it][k] = *reinterpret_cast<const u32x4 *>(src + k * step);
                    okv[it] = ok;
                }
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int u = base + tid + it * kThreads;
                    if (u >= items) continue;
                    int vc, hr, hp, o8;
                    split(u, vc, hr, hp, o8);
#pragma unroll
                    for (int pp = 0; pp < 8; ++pp) {
                        const int hc = (va + vc) * 8 + pp - i2o;
                        if (hc < 0 || hc >= p.HC) continue;
                        u32x4 o;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const unsigned lo = v[it][2 * jj][pp >> 1], hi = v[it][2 * jj + 1][pp >> 1];
                            o[jj] = (pp & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                        }
                        *reinterpret_cast<u32x4 *>(lds + ((hp * p.HR + hr) * p.HC + hc) * p.pitch + o8 * 16) =
                            okv[it] ? o : zero;
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---------------- the wave's residue classes ----------------
    f32x16 acc[kSlots][2][TR];
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jt = 0; jt < TR; ++jt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[sl][i][jt][r] = 0.0f;

    // lane's position in the window for tile jt (row jt) before the tap shift
    int hoff[TR];
#pragma unroll
    for (int jt = 0; jt < TR; ++jt) hoff[jt] = (jt * p.HC + (lane & 31)) * p.pitch + (lane >> 5) * 16;
    const int KB = p.Cgp / 16, MB = p.Mgp / 32, CB = p.Cg / 32;
    const f16x8 *const wfrag = reinterpret_cast<const f16x8 *>(wf);

    // a step: (tap t0, t1, t2 of the class, channel block cb of 32)
    struct Step {
        int t0, t1, t2, cb;
    };
#pragma unroll
    for (int sl = 0; sl < kSlots; ++sl) {
        const int cls = p.wave_cls[wave][sl];
        if (cls < 0) continue;  // wave-uniform
        const int r0 = cls & 0xff, r1 = (cls >> 8) & 0xff, r2 = cls >> 16;
        const int nt0 = p.ntap[0][r0], nt1 = p.ntap[1][r1], nt2 = p.ntap[2][r2];
        const int nsteps = nt0 * nt1 * nt2 * CB;
        if (nsteps == 0) continue;
        const int k00 = p.tk0[0][r0], k01 = p.tk0[1][r1], k02 = p.tk0[2][r2];
        const int b00 = p.tb0[0][r0] - p.bmin[0], b01 = p.tb0[1][r1] - p.bmin[1], b02 = p.tb0[2][r2] - p.bmin[2];
        auto advance = [&](Step &q) {
            if (++q.cb == CB) {
                q.cb = 0;
                if (++q.t2 == nt2) {
                    q.t2 = 0;
                    if (++q.t1 == nt1) {
                        q.t1 = 0;
                        ++q.t0;
                    }
                }
            }
        };
        auto load_a = [&](const Step &q, f16x8 (&dst)[2][2]) {
            const int tflat = ((k00 + q.t0 * p.kstep[0]) * p.K[1] + (k01 + q.t1 * p.kstep[1])) * p.K[2] +
                              (k02 + q.t2 * p.kstep[2]);
            const f16x8 *src = wfrag + (((size_t(g) * p.T + tflat) * MB + size_t(mt) * 2) * KB + size_t(q.cb) * 2) * 64 + lane;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) dst[i][h] = src[(size_t(i) * KB + h) * 64];
        };
        // the step's input fragments: tile jt's 32 positions, shifted by the step's tap
        auto load_b = [&](const Step &q, f16x8 (&b)[TR][2]) {
            const int sh = ((b00 - q.t0 * p.bstep[0]) * p.HR + (b01 - q.t1 * p.bstep[1])) * p.HC + (b02 - q.t2 * p.bstep[2]);
            const unsigned char *hb = lds + sh * p.pitch + q.cb * 64;
#pragma unroll
            for (int jt = 0; jt < TR; ++jt)
#pragma unroll
                for (int h = 0; h < 2; ++h) b[jt][h] = *reinterpret_cast<const f16x8 *>(hb + hoff[jt] + h * 32);
        };
        // channels-last: tile (channels x positions), so a lane holds 4 consecutive
        // channels of one position; channels-first: the transposed tile (positions x
        // channels), so a lane holds 4 consecutive positions of one channel (the operand
        // fragments have the same register layout in either role)
        auto mma = [&](const f16x8 (&a)[2][2], const f16x8 (&b)[TR][2]) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int jt = 0; jt < TR; ++jt)
                        acc[sl][i][jt] = CL ? __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][h], b[jt][h], acc[sl][i][jt], 0, 0, 0)
                                            : __builtin_amdgcn_mfma_f32_32x32x16_f16(b[jt][h], a[i][h], acc[sl][i][jt], 0, 0, 0);
        };
        f16x8 ring[kRing][2][2];
        f16x8 bf[2][TR][2];  // input fragments of the step (two buffers alternating)
        Step cur = {0, 0, 0, 0};
        Step pf = cur;
#pragma unroll
        for (int d = 0; d < kRing; ++d) {
            load_a(d < nsteps ? pf : cur, ring[d]);  // past the end: a valid, unused step
            advance(pf);
        }
        static_assert(kRing % 2 == 0, "fragment buffers alternate with the ring slots");
        for (int s0 = 0; s0 < nsteps; s0 += kRing) {
#pragma unroll
            for (int u = 0; u < kRing; ++u) {
                if (s0 + u < nsteps) {
                    load_b(cur, bf[u & 1]);
                    mma(ring[u], bf[u & 1]);
                    load_a(s0 + u + kRing < nsteps ? pf : cur, ring[u]);
                    advance(pf);
                    advance(cur);
                }
            }
        }
    }

    // ---------------- epilogue: the output box through LDS, whole rows out ----------------
    // Every residue class of the box is owned by some wave (classes without taps keep the
    // bias), so every staged value of the box is written.  Box extents are powers of two:
    // E0 = s0, E1 = 4 s1, E2 = 32 s2 (lgE: their log2).
    __syncthreads();  // every wave is done with the input window
    if (tid < 64) sbias[tid] = bias_ok ? float(bias_h) : 0.0f;
    const int E1 = p.E[1], E2 = p.E[2];
    const int lgE1 = p.lgE[1], lgE2 = p.lgE[2];
    _Float16 *const stile = reinterpret_cast<_Float16 *>(lds);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    auto pack4 = [](float v0, float v1, float v2, float v3) {  // one rounding per value
        const f16x2 lo = __builtin_convertvector(f32x2{v0, v1}, f16x2);
        const f16x2 hi = __builtin_convertvector(f32x2{v2, v3}, f16x2);
        return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    };
    __syncthreads();
    auto stage = [&](auto fin) {
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            const int cls = p.wave_cls[wave][sl];
            if (cls < 0) continue;
            const int r0 = cls & 0xff, r1 = (cls >> 8) & 0xff, r2 = cls >> 16;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jt = 0; jt < TR; ++jt) {
                    const int e1 = p.s[1] * jt + r1;
                    if constexpr (CL) {
                        // [position][channel], pitch 72: lane = position, 4 channels per write
                        const int e = ((r0 << lgE1) + e1) * E2 + p.s[2] * (lane & 31) + r2;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int m = i * 32 + q * 8 + (lane >> 5) * 4;
                            const f32x4 bq = *reinterpret_cast<const f32x4 *>(&sbias[m]);
                            *reinterpret_cast<u32x2 *>(&stile[e * 72 + m]) =
                                pack4(fin(acc[sl][i][jt][q * 4] + bq[0]), fin(acc[sl][i][jt][q * 4 + 1] + bq[1]),
                                      fin(acc[sl][i][jt][q * 4 + 2] + bq[2]), fin(acc[sl][i][jt][q * 4 + 3] + bq[3]));
                        }
                    } else {
                        // [channel][e0][e1][r2][column] (the classes of a row side by side,
                        // de-interleaved), channel pitch box + 8: lane = channel, 4
                        // consecutive columns per write
                        const int m = i * 32 + (lane & 31);
                        const float bm = sbias[m];
                        _Float16 *const row = stile + m * p.cpitch + ((((r0 << lgE1) + e1) * p.s[2] + r2) << 5);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<u32x2 *>(row + q * 8 + (lane >> 5) * 4) =
                                pack4(fin(acc[sl][i][jt][q * 4] + bm), fin(acc[sl][i][jt][q * 4 + 1] + bm),
                                      fin(acc[sl][i][jt][q * 4 + 2] + bm), fin(acc[sl][i][jt][q * 4 + 3] + bm));
                    }
                }
        }
    };
    with_activation(p.act, stage);
    __syncthreads();
    const int mvalid = min(64, p.Mg - mt * 64);
    const int o0b = p.s[0] * j0, o1b = p.s[1] * row_lo, o2b = p.s[2] * col_lo;
    const int O0 = p.O[0], O1 = p.O[1], O2 = p.O[2];
    // (the 16-byte output stores are streaming stores: Y is written once and read by no block)
    if constexpr (CL) {
        // one 16-byte vector of 8 channels per (position, channel octet), octet fastest
        const bool vec = (p.M % 8 == 0) && ((g * p.Mg + mt * 64) % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
        const int items = (p.E[0] << (lgE1 + lgE2)) * 8;
        _Float16 *const yb = y + size_t(n) * O0 * O1 * O2 * p.M + g * p.Mg + mt * 64;
        for (int u = tid; u < items; u += kThreads) {
            const int c8 = u & 7, e = u >> 3;
            const int e2 = e & (E2 - 1), e1 = (e >> lgE2) & (E1 - 1), e0 = e >> (lgE1 + lgE2);
            const int o0 = o0b + e0, o1 = o1b + e1, o2 = o2b + e2;
            if (o0 >= O0 || o1 >= O1 || o2 >= O2 || c8 * 8 >= mvalid) continue;
            _Float16 *dst = yb + ((size_t(o0) * O1 + o1) * O2 + o2) * p.M + c8 * 8;
            const _Float16 *src = &stile[e * 72 + c8 * 8];
            if (vec && c8 * 8 + 8 <= mvalid) {
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(src), reinterpret_cast<u32x4 *>(dst));
            } else {
                for (int k = 0; k < 8 && c8 * 8 + k < mvalid; ++k) dst[k] = src[k];
            }
        }
    } else {
        // per (channel, plane, row): E2 contiguous outputs from the de-interleaved classes
        // of the row; with s2 = 1 or 2, one 16-byte vector of 8 outputs per item
        const int s2 = p.s[2];
        const bool vec = (s2 <= 2) && (O2 % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
        const int lgPer = lgE2 - 3;  // vectors per row: E2 / 8
        const int items = (mvalid * p.E[0]) << (lgE1 + lgPer);
        const size_t plane_out = size_t(O0) * O1 * O2;
        _Float16 *const yb = y + (size_t(n) * p.M + g * p.Mg + mt * 64) * plane_out;
        for (int u = tid; u < items; u += kThreads) {
            const int c = u & ((1 << lgPer) - 1);
            const int rr = u >> lgPer;
            const int e1 = rr & (E1 - 1), e0m = rr >> lgE1;  // e0m = m * E0 + e0
            const int e0 = e0m & (p.E[0] - 1), m = e0m >> p.lgE[0];
            const int o0 = o0b + e0, o1 = o1b + e1;
            if (o0 >= O0 || o1 >= O1 || o2b + c * 8 >= O2) continue;
            _Float16 *dst = yb + m * plane_out + (size_t(o0) * O1 + o1) * O2 + o2b + c * 8;
            const _Float16 *row = stile + m * p.cpitch + ((((e0 << lgE1) + e1) * s2) << 5);
            if (vec && s2 == 2) {  // outputs 8c .. 8c+7: columns 4c .. 4c+3 of classes 0 and 1
                const u32x2 c0 = *reinterpret_cast<const u32x2 *>(row + 4 * c);
                const u32x2 c1 = *reinterpret_cast<const u32x2 *>(row + 32 + 4 * c);
                u32x4 o;
                o[0] = (c0.x & 0xffffu) | (c1.x << 16);
                o[1] = (c0.x >> 16) | (c1.x & 0xffff0000u);
                o[2] = (c0.y & 0xffffu) | (c1.y << 16);
                o[3] = (c0.y >> 16) | (c1.y & 0xffff0000u);
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(dst));
            } else if (vec) {  // s2 = 1: the row is stored as it is
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(row + 8 * c), reinterpret_cast<u32x4 *>(dst));
            } else {
                for (int k = 0; k < 8 && o2b + c * 8 + k < O2; ++k) {
                    const int e2 = c * 8 + k;
                    dst[k] = row[(e2 % s2) * 32 + e2 / s2];
                }
            }
        }
    }
}

// ---------------- host-side planning ----------------
bool make_mp_plan(const Geom &g, bool cl, MpArgs *a, std::string *why)
{
    auto no = [&](const char *m) {
        *why = m;
        return false;
    };
    std::memset(a, 0, sizeof(*a));
    if (g.Cg % 32 != 0) return no("all-phase kernel: C/group must be a multiple of 32");
    if (!cl && g.L[2] % 8 != 0) return no("all-phase kernel: innermost input size must be a multiple of 8");
    if (cl && g.C % 8 != 0) return no("all-phase kernel: C must be a multiple of 8");
    int nclass = 0, span1 = 0;
    int cls_r[kMaxClass][3], cls_taps[kMaxClass];
    for (int t = 0; t < kAxes; ++t) {
        if (g.s[t] > 8) return no("all-phase kernel: stride above 8");
        a->L[t] = int(g.L[t]);
        a->O[t] = int(g.O[t]);
        a->s[t] = int(g.s[t]);
        a->K[t] = int(g.K[t]);
        a->J[t] = int((g.O[t] + g.s[t] - 1) / g.s[t]);
        const int64_t gsd = std::gcd(g.s[t], g.d[t]);
        a->kstep[t] = int(g.s[t] / gsd);
        a->bstep[t] = int(g.d[t] / gsd);
        int bmin = INT32_MAX, bmax = INT32_MIN;
        for (int r = 0; r < g.s[t]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, t, r, &ph) || ph.ntaps > 8) return no("all-phase kernel: more than 8 taps per class");
            a->ntap[t][r] = ph.ntaps;
            a->tk0[t][r] = ph.ntaps ? ph.k[0] : 0;
            a->tb0[t][r] = ph.ntaps ? ph.beta[0] : 0;
            for (int k = 0; k < ph.ntaps; ++k) {
                if (ph.k[k] != ph.k[0] + k * a->kstep[t] || ph.beta[k] != ph.beta[0] - k * a->bstep[t])
                    return no("internal: taps are not an arithmetic progression");
                bmin = std::min(bmin, ph.beta[k]);
                bmax = std::max(bmax, ph.beta[k]);
            }
        }
        if (bmin > bmax) bmin = bmax = 0;  // no tap reaches this axis' outputs
        a->bmin[t] = bmin;
        const int span = bmax - bmin;
        if (t == 0) a->HP = 1 + span;
        if (t == 1) span1 = span;
        if (t == 2) a->HC = kTC + span;
    }
    // residue classes that have outputs
    for (int r0 = 0; r0 < g.s[0]; ++r0)
        for (int r1 = 0; r1 < g.s[1]; ++r1)
            for (int r2 = 0; r2 < g.s[2]; ++r2) {
                if (r0 >= g.O[0] || r1 >= g.O[1] || r2 >= g.O[2]) continue;
                if (nclass == kMaxClass) return no("all-phase kernel: more than 8 residue classes");
                cls_r[nclass][0] = r0;
                cls_r[nclass][1] = r1;
                cls_r[nclass][2] = r2;
                cls_taps[nclass] = a->ntap[0][r0] * a->ntap[1][r1] * a->ntap[2][r2];
                ++nclass;
            }
    if (nclass < 4) return no("all-phase kernel: fewer than 4 residue classes");
    // heaviest class first onto the least loaded wave with a free slot
    int order[kMaxClass];
    for (int i = 0; i < nclass; ++i) order[i] = i;
    std::stable_sort(order, order + nclass, [&](int u, int v) { return cls_taps[u] > cls_taps[v]; });
    int load[4] = {0, 0, 0, 0}, used[4] = {0, 0, 0, 0};
    for (int w = 0; w < 4; ++w)
        for (int sl = 0; sl < kSlots; ++sl) a->wave_cls[w][sl] = -1;
    for (int i = 0; i < nclass; ++i) {
        const int c = order[i];
        int best = -1;
        for (int w = 0; w < 4; ++w)
            if (used[w] < kSlots && (best < 0 || load[w] < load[best])) best = w;
        a->wave_cls[best][used[best]++] = cls_r[c][0] | (cls_r[c][1] << 8) | (cls_r[c][2] << 16);
        load[best] += cls_taps[c];
    }
    a->N = int(g.N);
    a->C = int(g.C);
    a->M = int(g.M);
    a->Cg = int(g.Cg);
    a->Mg = int(g.Mg);
    a->G = int(g.G);
    a->T = int(g.taps());
    a->Cgp = a->Cg;
    a->mtiles = int((g.Mg + 63) / 64);
    a->Mgp = a->mtiles * 64;
    a->pitch = a->Cg * 2 + 16;
    a->ctiles = (a->J[2] + kTC - 1) / kTC;
    for (int t = 0; t < kAxes; ++t)
        if (g.s[t] & (g.s[t] - 1)) return no("all-phase kernel: strides must be powers of two");
    a->E[0] = a->s[0];
    a->E[2] = a->s[2] * kTC;
    // the smaller box when its window and output box fit, else the larger one
    for (const int tr : {2, 4}) {
        a->tr = tr;
        a->HR = tr + span1;
        a->rtiles = (a->J[1] + tr - 1) / tr;
        a->E[1] = a->s[1] * tr;
        for (int t = 0; t < kAxes; ++t) a->lgE[t] = __builtin_ctz(unsigned(a->E[t]));
        a->cpitch = a->E[0] * a->E[1] * a->E[2] + 8;
        const long long box = (long long)a->E[0] * a->E[1] * a->E[2];
        if ((long long)a->HP * a->HR * a->HC * a->pitch > stage_bytes(tr) ||
            (cl ? box * 72 : (long long)a->cpitch * 64) * 2 > stage_bytes(tr))
            continue;
        const long long blocks = (long long)g.N * g.G * a->mtiles * a->J[0] * a->rtiles * a->ctiles;
        if (blocks > INT32_MAX || blocks < 1) return no("all-phase kernel: too many blocks");
        a->nblocks = int(blocks);
        return true;
    }
    return no("all-phase kernel: input window or output box exceeds LDS");
}

}  // namespace

bool mphase_supports(const Geom &g, bool cl, std::string *why)
{
    if (g.x_elems() <= 0) {
        *why = "empty input";
        return false;
    }
    MpArgs a;
    return make_mp_plan(g, cl, &a, why);
}

size_t mphase_workspace_bytes(const Geom &g, bool cl)
{
    MpArgs a;
    std::string why;
    if (!make_mp_plan(g, cl, &a, &why)) return 0;
    return size_t(a.G) * a.T * a.Mgp * a.Cgp * sizeof(_Float16);
}

ct_status launch_mphase(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                        const Act &act, void *wsp, size_t ws_bytes, hipStream_t st, std::string *err, bool w_conv)
{
    MpArgs a;
    if (!make_mp_plan(g, cl, &a, err)) return CT_EUNSUPPORTED;
    a.act = act;
    const size_t need = size_t(a.G) * a.T * a.Mgp * a.Cgp * sizeof(_Float16);
    if (ws_bytes < need) {
        *err = "workspace is smaller than the all-phase kernel needs";
        return CT_EINVAL;
    }
    ct_status s = launch_pack_w_frag(g, w, wsp, a.Cgp, a.Mgp, w_conv, st, err);
    if (s != CT_OK) return s;
    mark_before(st);
    auto run = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(unsigned(a.nblocks)), dim3(kThreads), 0, st, static_cast<const _Float16 *>(x),
                           static_cast<const _Float16 *>(wsp), static_cast<const _Float16 *>(bias),
                           static_cast<_Float16 *>(y), a);
    };
    if (cl) {
        if (a.tr == 2) run(mphase_kernel<true, 2>);
        else run(mphase_kernel<true, 4>);
    } else {
        if (a.tr == 2) run(mphase_kernel<false, 2>);
        else run(mphase_kernel<false, 4>);
    }
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("all-phase kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
