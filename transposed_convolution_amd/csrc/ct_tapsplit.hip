// ct_tapsplit.hip -- stride-1 implicit GEMM with the taps split across the waves, for
// float16 transposed convolutions with few output channels per group (gfx950 MFMA).
//
// Method (webgpu-kernels "ai.onnx.ConvTranspose" README, Implementation variants: the
// implicit-gather GEMM that reduces over input channels x taps and stores outputs
// directly).  With stride 1 on every axis every output o receives every tap k, from the
// input i = o + b - k*d, so an output box of consecutive positions reads one input
// window: the box grown by (K-1)*d on each axis.  One workgroup computes a box of 64 or 96
// consecutive output positions of one output plane (flattened over rows when a row is
// shorter than the box, else a run inside one row) x 64 output channels; 96 when that
// puts the call's blocks in fewer rounds of the chip's block slots:
//
//   * Two workgroups share a compute unit (78 KB of LDS each), so one's window loads
//     overlap the other's MFMAs.  The input window ([plane][row][column][channel], a
//     16-byte pad per position) holds 64 channels (32 when C/group is not a multiple of
//     64): the channels go through it in passes, each loaded by the whole block between
//     two barriers.
//   * Each of the 4 waves takes every fourth tap and computes the WHOLE box over its taps
//     (2 x 2 or 2 x 3 MFMA 32x32 tiles, float32 accumulators), so the waves read disjoint weights
//     and need no barrier in the main loop; a lane's input fragment address is its own
//     position's window offset plus the tap's shift, so rows of any width pack the box.
//   * A step is one tap x 32 input channels: weight fragments straight from the
//     fragment-major packing into registers (a ring of kRing steps in flight), input
//     fragments from LDS, v_mfma_f32_32x32x16_f16, 8 or 12 per step.
//   * Epilogue: the four waves' partial sums meet in LDS (float32, one tile row at a
//     time), a wave adds up one tile, adds the bias, rounds once and stages it in the
//     output box in LDS; the box then goes out as
//     contiguous runs (channels-first: the box's positions of a channel; channels-last:
//     64 channels of a position).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "ct_internal.hpp"

namespace ct {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
// A box holds NT 32-position MFMA tiles (NT = 2 or 3, chosen per call: 3 when it lets the
// blocks of the call fit fewer rounds of the chip's two-per-CU slots)
constexpr int box_of(int nt) { return nt * 32; }                 // output positions per box
constexpr int part_bytes(int nt) { return 4 * nt * 16 * 64 * 4; }  // one tile row of the waves' partial sums
constexpr int kRing = 4;             // steps of weight fragments in flight per wave
constexpr int kMaxTaps = 32;
constexpr int kLds = 78 * 1024;      // two workgroups per compute unit
constexpr int kBiasBytes = 64 * 4;   // the block's 64 bias values (float32) at the end of LDS
constexpr int kStage = kLds - kBiasBytes;
constexpr int kHaloVec = 8;          // 16-byte window loads per thread and round

struct TsArgs {
    int N, C, M, Cg, Mg, G, T, Mgp, Cgp;
    int L[3], O[3];
    int org[3];                 // window origin relative to the box: b - (K-1)*d per axis
    int HP, HR, HC, pitch;      // window extents (planes, rows, columns), LDS bytes per position
    int cw, passes;             // input channels per window pass (32 or 64), passes = C/group / cw
    int seg;                    // 1: a box is a run inside one output row; 0: flattened rows
    int tpr, ptiles, mtiles, nblocks;
    int ntap_w[4];              // taps of each wave (taps w, w + 4, ...)
    int nt;                     // 32-position tiles per box (the kernel's NT)
    int toff[kMaxTaps];         // window shift of tap t in positions
    Act act;
};

__device__ __forceinline__ int floor_div8(int v) { return v >= 0 ? v / 8 : -((-v + 7) / 8); }

template <bool CL, int NT>
__global__ __launch_bounds__(kThreads, 2) void tapsplit_kernel(const _Float16 *x, const _Float16 *__restrict__ wf,
                                                               const _Float16 *__restrict__ bias,
                                                               _Float16 *__restrict__ y, TsArgs p)
{
    constexpr int kNT = NT;                         // 32-position MFMA tiles per box
    constexpr int kBox = box_of(NT);                // output positions per box
    constexpr int kPartBytes = part_bytes(NT);      // float32 partial sums of one tile row
    constexpr int kSPitch = kBox + 8;               // staging pitch (halves) of the output box
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
    float *const sbias = reinterpret_cast<float *>(lds + kStage);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---------------- the box this block computes ----------------
    // neighbouring boxes (which share input rows and planes) on one XCD
    int rest = xcd_remap(blockIdx.x, p.nblocks);
    const int pt = rest % p.ptiles;
    rest /= p.ptiles;
    const int o0 = rest % p.O[0];
    rest /= p.O[0];
    const int mt = rest % p.mtiles;
    rest /= p.mtiles;
    const int g = rest % p.G;
    const int n = rest / p.G;
    const int O1 = p.O[1], O2 = p.O[2];
    int row_lo, col_lo, q0, q1;
    if (p.seg) {
        row_lo = pt / p.tpr;
        col_lo = (pt - row_lo * p.tpr) * kBox;
        q0 = row_lo * O2 + col_lo;
        q1 = q0 + min(kBox, O2 - col_lo);
    } else {
        q0 = pt * kBox;
        q1 = min(q0 + kBox, O1 * O2);
        row_lo = q0 / O2;
        col_lo = 0;
    }
    const int i0o = o0 + p.org[0], i1o = row_lo + p.org[1], i2o = col_lo + p.org[2];
    const int L0 = p.L[0], L1 = p.L[1], L2 = p.L[2];

    // bias of the block's 64 channels, loaded now and staged after the main loop
    const bool bias_ok = bias && tid < 64 && mt * 64 + tid < p.Mg;
    const _Float16 bias_h =
        bias_ok ? bias[g * p.Mg + mt * 64 + tid] : *reinterpret_cast<const _Float16 *>(bias ? bias : x);

    // ---------------- input window of channels [c0, c0 + cw) of the group into LDS ----------------
    // zeros where the window lies outside the input
    auto load_window = [&](int c0) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int pos = p.HP * p.HR * p.HC;
        if constexpr (CL) {
            // 16-byte vectors of 8 channels, channels innermost in both places
            const int cv = p.cw / 8;
            const int items = pos * cv;
            const UDiv dcv(cv), dhc(p.HC), dhr(p.HR);  // item -> (position, octet) -> (plane, row, column)
            const _Float16 *xg = x + size_t(g) * p.Cg + c0;
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
            // items (channel octet, aligned 8-column vector, row, plane), octet fastest: 8
            // loads of 16 bytes (8 columns of one channel each), transposed into 8 LDS
            // positions x 8 channels; the 16-byte LDS writes of consecutive octets of one
            // position fall in distinct banks
            const int va = floor_div8(i2o);
            const int nvc = floor_div8(i2o + p.HC + 7) - va;
            const int oct = p.cw / 8;
            const int items = p.HP * p.HR * nvc * oct;
            const UDiv doc(oct), dnv(nvc), dhr(p.HR);
            auto split = [&](int u, int &o8, int &vc, int &hr, int &hp) {
                const int t1 = doc.div(u);
                o8 = u - t1 * oct;
                const int t2 = dnv.div(t1);
                vc = t1 - t2 * nvc;
                hp = dhr.div(t2);
                hr = t2 - hp * p.HR;
            };
            const size_t plane_in = size_t(L0) * L1 * L2;
            const _Float16 *xg = x + (size_t(n) * p.C + size_t(g) * p.Cg + c0) * plane_in;
            constexpr int IT = kHaloVec / 8;
            for (int base = 0; base < items; base += kThreads * IT) {
                u32x4 v[IT][8];
                bool okv[IT];
#pragma unroll
                for (int it = 0; it < IT; ++it) {
                    const int u = base + tid + it * kThreads;
                    int o8, vc, hr, hp;
                    split(u, o8, vc, hr, hp);
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
                    int o8, vc, hr, hp;
                    split(u, o8, vc, hr, hp);
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
    };

    // ---------------- the wave's taps ----------------
    const int KB = p.Cgp / 16, MB = p.Mgp / 32;
    const int CBP = p.cw / 32;                 // channel blocks of 32 per window pass
    const int nsp = p.ntap_w[wave] * CBP;      // the wave's steps per pass
    const f16x8 *const wfrag = reinterpret_cast<const f16x8 *>(wf);
    struct Step {
        int u, cb;  // the wave's u-th tap (tap wave + 4u), channel block of 32 within the pass
    };
    auto advance = [&](Step &q) {
        if (++q.cb == CBP) {
            q.cb = 0;
            ++q.u;
        }
    };
    auto load_a = [&](int pass, const Step &q, f16x8 (&dst)[2][2]) {
        const int t = wave + 4 * q.u;
        const f16x8 *src =
            wfrag + (((size_t(g) * p.T + t) * MB + size_t(mt) * 2) * KB + size_t(pass * CBP + q.cb) * 2) * 64 + lane;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) dst[i][h] = src[(size_t(i) * KB + h) * 64];
    };

    f32x16 acc[2][kNT];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jt = 0; jt < kNT; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jt][r] = 0.0f;

    // lane's window position for tile jt before the tap shift (positions past the box
    // repeat its last one: computed, never stored)
    int hoff[kNT];
#pragma unroll
    for (int jt = 0; jt < kNT; ++jt) {
        int q = q0 + jt * 32 + (lane & 31);
        if (q >= q1) q = q1 - 1;
        const int row = p.seg ? row_lo : q / O2;
        const int col = q - row * O2;
        hoff[jt] = ((row - row_lo) * p.HC + (col - col_lo)) * p.pitch + (lane >> 5) * 16;
    }
    auto load_b = [&](const Step &q, f16x8 (&b)[kNT][2]) {
        const unsigned char *hb = lds + p.toff[wave + 4 * q.u] * p.pitch + q.cb * 64;
#pragma unroll
        for (int jt = 0; jt < kNT; ++jt)
#pragma unroll
            for (int h = 0; h < 2; ++h) b[jt][h] = *reinterpret_cast<const f16x8 *>(hb + hoff[jt] + h * 32);
    };
    // channels-last: tile (channels x positions), a lane holds 4 consecutive channels of
    // one position; channels-first: the transposed tile, 4 consecutive positions of one
    // channel (the operand fragments have the same register layout in either role)
    auto mma = [&](const f16x8 (&a)[2][2], const f16x8 (&b)[kNT][2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jt = 0; jt < kNT; ++jt)
                    acc[i][jt] = CL ? __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][h], b[jt][h], acc[i][jt], 0, 0, 0)
                                    : __builtin_amdgcn_mfma_f32_32x32x16_f16(b[jt][h], a[i][h], acc[i][jt], 0, 0, 0);
    };

    // ---------------- main loop: channel passes; in each, the wave's taps over the whole box ----------------
    // The window of one pass is loaded by the whole block between two barriers; the
    // pass's first kRing steps of weight fragments are issued before it, so the window's
    // wait covers them.  Within a pass the waves run without barriers.
    f16x8 ring[kRing][2][2];
    f16x8 bf[kNT][2];
    for (int pass = 0; pass < p.passes; ++pass) {
        if (pass > 0) __syncthreads();  // every wave is done with the previous window
        Step cur = {0, 0};
        Step pf = cur;
        if (nsp > 0) {
#pragma unroll
            for (int d = 0; d < kRing; ++d) {
                load_a(pass, d < nsp ? pf : cur, ring[d]);  // past the end: a valid, unused step
                advance(pf);
            }
        }
        load_window(pass * p.cw);
        __syncthreads();
        for (int s0 = 0; s0 < nsp; s0 += kRing) {
#pragma unroll
            for (int u = 0; u < kRing; ++u) {
                if (s0 + u < nsp) {
                    load_b(cur, bf);
                    mma(ring[u], bf);
                    load_a(pass, s0 + u + kRing < nsp ? pf : cur, ring[u]);
                    advance(pf);
                    advance(cur);
                }
            }
        }
    }

    // ---------------- epilogue: partial sums meet in LDS, the box goes out ----------------
    // Two rounds (tile row i = 0, 1): every wave writes its NT tiles of row i, then NT
    // waves (2i and 2i + 1 for NT = 2, else 0 .. NT - 1) add up tile (i, j) of all four
    // waves, add the bias, round once and stage them in the output box.
    __syncthreads();  // every wave is done with the input window
    if (tid < 64) sbias[tid] = bias_ok ? float(bias_h) : 0.0f;
    float *const part = reinterpret_cast<float *>(lds);  // [wave][jt][r][lane]
    _Float16 *const stile = reinterpret_cast<_Float16 *>(lds + kPartBytes);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    auto pack4 = [](float v0, float v1, float v2, float v3) {  // one rounding per value
        const f16x2 lo = __builtin_convertvector(f32x2{v0, v1}, f16x2);
        const f16x2 hi = __builtin_convertvector(f32x2{v2, v3}, f16x2);
        return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    };
#pragma unroll
    for (int fi = 0; fi < 2; ++fi) {
        if (fi > 0) __syncthreads();  // the previous round's partial sums have been read
#pragma unroll
        for (int jt = 0; jt < kNT; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[((wave * kNT + jt) * 16 + r) * 64 + lane] = acc[fi][jt][r];
        __syncthreads();
        if (kNT == 2 ? wave / kNT == fi : wave < kNT) {  // wave-uniform
            const int fj = wave % kNT;
            f32x16 sum;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < 4; ++w) v += part[((w * kNT + fj) * 16 + r) * 64 + lane];
                sum[r] = v;
            }
            auto stage = [&](auto fin) {
                if constexpr (CL) {
                    // [position][channel], pitch 72: lane = position, 4 consecutive channels per write
                    const int e = fj * 32 + (lane & 31);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int m = fi * 32 + q * 8 + (lane >> 5) * 4;
                        const f32x4 bq = *reinterpret_cast<const f32x4 *>(&sbias[m]);
                        *reinterpret_cast<u32x2 *>(&stile[e * 72 + m]) =
                            pack4(fin(sum[q * 4] + bq[0]), fin(sum[q * 4 + 1] + bq[1]), fin(sum[q * 4 + 2] + bq[2]),
                                  fin(sum[q * 4 + 3] + bq[3]));
                    }
                } else {
                    // [channel][position], pitch kBox + 8: lane = channel, 4 consecutive positions per write
                    const int m = fi * 32 + (lane & 31);
                    const float bm = sbias[m];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<u32x2 *>(&stile[m * kSPitch + fj * 32 + q * 8 + (lane >> 5) * 4]) =
                            pack4(fin(sum[q * 4] + bm), fin(sum[q * 4 + 1] + bm), fin(sum[q * 4 + 2] + bm),
                                  fin(sum[q * 4 + 3] + bm));
                }
            };
            with_activation(p.act, stage);
        }
    }
    __syncthreads();
    const int mvalid = min(64, p.Mg - mt * 64);
    const int nq = q1 - q0;
    const size_t plane_out = size_t(p.O[0]) * O1 * O2;
    if constexpr (CL) {
        // one 16-byte vector of 8 channels per (position, channel octet), octet fastest
        const bool vec = (p.M % 8 == 0) && ((g * p.Mg + mt * 64) % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
        _Float16 *const yb = y + (size_t(n) * plane_out + size_t(o0) * O1 * O2) * p.M + g * p.Mg + mt * 64;
        for (int u = tid; u < kBox * 8; u += kThreads) {
            const int c8 = u & 7, e = u >> 3;
            if (e >= nq || c8 * 8 >= mvalid) continue;
            const int q = q0 + e;
            _Float16 *dst = yb + size_t(q) * p.M + c8 * 8;
            const _Float16 *src = &stile[e * 72 + c8 * 8];
            if (vec && c8 * 8 + 8 <= mvalid) {
                *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
            } else {
                for (int k = 0; k < 8 && c8 * 8 + k < mvalid; ++k) dst[k] = src[k];
            }
        }
    } else {
        // per channel, the box's positions are one contiguous run of the output plane:
        // 4 positions (8 bytes) per item when the run is 8-byte aligned
        _Float16 *const yb = y + (size_t(n) * p.M + g * p.Mg + mt * 64) * plane_out + size_t(o0) * O1 * O2 + q0;
        const bool vec = (plane_out % 4 == 0) && ((size_t(O1) * O2) % 4 == 0) && (q0 % 4 == 0) &&
                         (reinterpret_cast<uintptr_t>(y) % 8 == 0);
        for (int u = tid; u < 64 * (kBox / 4); u += kThreads) {
            const int c4 = u % (kBox / 4), m = u / (kBox / 4);
            if (m >= mvalid || c4 * 4 >= nq) continue;
            _Float16 *dst = yb + size_t(m) * plane_out + c4 * 4;
            const _Float16 *src = &stile[m * kSPitch + c4 * 4];
            if (vec && c4 * 4 + 4 <= nq) {
                *reinterpret_cast<u32x2 *>(dst) = *reinterpret_cast<const u32x2 *>(src);
            } else {
                for (int k = 0; k < 4 && c4 * 4 + k < nq; ++k) dst[k] = src[k];
            }
        }
    }
}

// ---------------- host-side planning ----------------
// compute units of the current device (256 when there is none to ask)
int device_cus()
{
    static thread_local int dev_cached = -1, cus_cached = 0;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev == dev_cached) return cus_cached;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    dev_cached = dev;
    cus_cached = cus;
    return cus;
}

bool make_ts_plan(const Geom &g, bool cl, TsArgs *a, std::string *why)
{
    auto no = [&](const char *m) {
        *why = m;
        return false;
    };
    std::memset(a, 0, sizeof(*a));
    for (int t = 0; t < kAxes; ++t)
        if (g.s[t] != 1) return no("tap-split kernel: stride 1 only");
    if (g.Cg % 32 != 0) return no("tap-split kernel: C/group must be a multiple of 32");
    if (!cl && g.L[2] % 8 != 0) return no("tap-split kernel: innermost input size must be a multiple of 8");
    if (cl && g.C % 8 != 0) return no("tap-split kernel: C must be a multiple of 8");
    if (g.taps() > kMaxTaps) return no("tap-split kernel: more than 32 taps");
    if (g.O[1] * g.O[2] > INT32_MAX / 2) return no("tap-split kernel: output plane too large");
    int span[kAxes];
    for (int t = 0; t < kAxes; ++t) {
        a->L[t] = int(g.L[t]);
        a->O[t] = int(g.O[t]);
        span[t] = int((g.K[t] - 1) * g.d[t]);
        a->org[t] = int(g.b[t]) - span[t];
    }
    const int O2 = a->O[2];
    a->HP = 1 + span[0];
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
    for (int w = 0; w < 4; ++w) a->ntap_w[w] = (a->T - w + 3) / 4;
    static_assert(part_bytes(3) + 64 * (box_of(3) + 8) * 2 <= kStage && box_of(3) * 72 * 2 <= kStage - part_bytes(3),
                  "epilogue LDS");
    // the box-dependent part for NT tiles per box; false when the window does not fit
    auto fit = [&](TsArgs &b, int nt) {
        const int box = box_of(nt);
        b.nt = nt;
        b.seg = O2 >= box ? 1 : 0;
        b.tpr = b.seg ? (O2 + box - 1) / box : 1;
        b.ptiles = b.seg ? b.O[1] * b.tpr : int((int64_t(b.O[1]) * O2 + box - 1) / box);
        // rows a flattened box can touch: a run of box positions starting anywhere in a row
        b.HR = (b.seg ? 1 : (O2 - 1 + box - 1) / O2 + 1) + span[1];
        b.HC = (b.seg ? box : O2) + span[2];
        // 64 channels per window pass when they fit, else 32
        const long long positions = (long long)b.HP * b.HR * b.HC;
        b.cw = b.Cg % 64 == 0 && positions * (64 * 2 + 16) <= kStage ? 64 : 32;
        b.passes = b.Cg / b.cw;
        b.pitch = b.cw * 2 + 16;
        if (positions * b.pitch > kStage) return false;
        int t = 0;
        for (int k0 = 0; k0 < g.K[0]; ++k0)
            for (int k1 = 0; k1 < g.K[1]; ++k1)
                for (int k2 = 0; k2 < g.K[2]; ++k2, ++t)
                    b.toff[t] = int(((g.K[0] - 1 - k0) * g.d[0] * b.HR + (g.K[1] - 1 - k1) * g.d[1]) * b.HC +
                                    (g.K[2] - 1 - k2) * g.d[2]);
        const long long blocks = (long long)g.N * g.G * b.mtiles * b.O[0] * b.ptiles;
        if (blocks > INT32_MAX || blocks < 1) return false;
        b.nblocks = int(blocks);
        return true;
    };
    TsArgs a2 = *a, a3 = *a;
    const bool ok2 = fit(a2, 2), ok3 = fit(a3, 3);
    // rounds of the chip's two-per-CU block slots
    const long long slots = 2LL * device_cus();
    auto rounds = [&](const TsArgs &b) { return (b.nblocks + slots - 1) / slots; };
    if (ok3 && (!ok2 || rounds(a3) < rounds(a2))) *a = a3;
    else if (ok2) *a = a2;
    else return no("tap-split kernel: input window exceeds LDS");
    return true;
}

}  // namespace

bool tapsplit_supports(const Geom &g, bool cl, std::string *why)
{
    if (g.x_elems() <= 0) {
        *why = "empty input";
        return false;
    }
    TsArgs a;
    return make_ts_plan(g, cl, &a, why);
}

size_t tapsplit_workspace_bytes(const Geom &g, bool cl)
{
    TsArgs a;
    std::string why;
    if (g.x_elems() <= 0 || !make_ts_plan(g, cl, &a, &why)) return 0;
    return size_t(a.G) * a.T * a.Mgp * a.Cgp * sizeof(_Float16);
}

ct_status launch_tapsplit(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                          const Act &act, void *wsp, size_t ws_bytes, hipStream_t st, std::string *err, bool w_conv)
{
    TsArgs a;
    if (!make_ts_plan(g, cl, &a, err)) return CT_EUNSUPPORTED;
    a.act = act;
    const size_t need = size_t(a.G) * a.T * a.Mgp * a.Cgp * sizeof(_Float16);
    if (ws_bytes < need) {
        *err = "workspace is smaller than the tap-split kernel needs";
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
        if (a.nt == 3) run(tapsplit_kernel<true, 3>);
        else run(tapsplit_kernel<true, 2>);
    } else {
        if (a.nt == 3) run(tapsplit_kernel<false, 3>);
        else run(tapsplit_kernel<false, 2>);
    }
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("tap-split kernel launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
