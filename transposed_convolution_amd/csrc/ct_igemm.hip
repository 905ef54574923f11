// ct_igemm.hip -- stride-phase implicit GEMM for float16 on MFMA (gfx950).
//
// Method (webgpu-kernels "ai.onnx.ConvTranspose" README, Implementation variants: the
// stride-phase route, and the implicit-gather GEMM that reads input windows directly,
// stores output elements directly and reduces over input channels x taps, with no
// column matrix and no scatter pass).  Output positions are split by their residue r
// modulo the stride on every axis; one residue class ("phase") of outputs
// o = r + s*j receives exactly the taps k with (r + b - k*d) divisible by s, from the
// inputs i = j + beta_k.  Each phase is therefore a dense stride-1 correlation:
//     Y[n, m, r + s*j] = bias[m] + sum_{c in group} sum_{k in T(r)} X[n, c, j + beta_k] W[c, m', k]
// which is a GEMM with rows = output channels, columns = the phase's output pixels and
// depth = input channels x taps.  No zero-inserted input is ever formed.
//
// Kernel structure (one workgroup = 4 wave64s, one phase, a BM (output channels) x BN
// (phase pixels of one (n, j0) plane) tile; 256 x 256 with 64 channels per depth step
// when M/group > 64, else 64 x 512 with 32 channels per step):
//   * W is first re-laid out by pack_w_kernel into Wp[g][tap][m][c] (c contiguous,
//     zero padded to whole depth steps and whole channel tiles), so every weight tile is
//     a run of 16-byte loads.
//   * For each channel chunk and each valid tap along axis 0, the input "halo" that the
//     tile's taps along axes 1 and 2 touch is staged once in LDS as [row][col][channels];
//     every (t1, t2) tap then reads a shifted window of it.
//   * The MFMA v_mfma_f32_32x32x16_f16 runs with the weight tile as A (32 channels of m)
//     and the shifted halo window as B (32 pixels); float32 accumulators.
//   * Weight tiles are double-buffered in LDS and prefetched into registers one step
//     ahead, ahead of any halo loads (loads complete in issue order); the next group's
//     halo is prefetched into registers during the current group (with four taps per
//     group, a quarter per step, so every load count is static).  LDS rows carry 16
//     bytes of padding so 16-byte reads of consecutive rows fall in distinct banks.
//   * Epilogue: the output tile is staged through LDS, bias added, one
//     round-to-nearest-even conversion, 16-byte stores along the contiguous direction.
//   * Blocks are re-ordered so that the blocks an XCD receives (hardware round-robin)
//     are consecutive in work order: all phases of one pixel tile share that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <cstring>

#include "ct_internal.hpp"

namespace ct {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxRes = 8;               // largest stride handled per axis
constexpr int kMaxTap = 8;               // largest tap count per residue and axis
constexpr int kMaxPh = 64;               // largest number of phases
constexpr int kThreads = 256;            // 4 wave64s, one per SIMD
constexpr int kLdsBytes = 160 * 1024 - 2048;
// LDS bytes one block may use when OCC blocks share a compute unit (160 KB of LDS per CU)
constexpr int lds_budget(int occ) { return occ == 1 ? kLdsBytes : 160 * 1024 / occ - 1024; }
constexpr int kSinkBytes = 64 * 16;
constexpr int kBiasBytes = 256 * 4;      // the block's bias as float32 (at most 256 channels)
// quantized instances: per channel of the block the int32 compensation, the float32
// requantization multiplier and the shifted weight zero point
constexpr int kQTailBytes = 3 * 256 * 4;
constexpr int tail_bytes(bool q8) { return q8 ? kQTailBytes : kBiasBytes; }

struct IgArgs {
    int N, C, M, Cg, Mg, Cgp, Mgp, T, G;
    int L[3], O[3], s[3], K[3];
    int nchunk, mtiles;
    int nphase, interleave, nblocks;
    // Every table holds 32-bit words: the kernel reads them with scalar loads (sub-dword
    // fields would be read by vector loads, each waited for in turn at the kernel's start).
    int ph_start[kMaxPh + 1];
    int ph_r[kMaxPh];  // residues of a phase: r0 | r1 << 8 | r2 << 16
    // Taps of residue r on axis a form an arithmetic progression:
    //   k = tk0[a][r] + u * kstep[a],  beta = tb0[a][r] - u * bstep[a],  u in [0, ntap[a][r])
    // with kstep = s / gcd(s, d) and bstep = d / gcd(s, d).
    int ntap[3][kMaxRes];
    int tk0[3][kMaxRes];
    int tb0[3][kMaxRes];
    int kstep[3], bstep[3];
    Act act;  // output activation
    // quantized instances only (QLinear scheme; see the kernel's Q8 comments)
    struct Quant {
        const float *w_scale;   // 1 or M values
        const void *w_zp;       // 1 or M values of w's type
        const int *bias;        // M values or null
        const int *wsum;        // [G][T][Mgp]: sum over c of the shifted weights
        const int *xsum;        // [N][G][L0][L1][L2]: sum over the group's channels of the shifted input
        float x_scale, y_scale;
        int x_zp, y_zp, y_lo, y_hi;  // x_zp in the signed (shifted) domain
        unsigned xflip;              // 0x80808080 for uint8 x (to the signed domain), else 0
        int w_u8, w_per_channel;
    } q;
};

__device__ __forceinline__ int floor_div8(int v) { return v >= 0 ? v / 8 : -((-v + 7) / 8); }


// Tile geometry of the phase pixels (j1, j2) a block covers.
struct Tile {
    int q0, q1;          // flattened pixel range in the J1 x J2 plane
    int row_lo, col_lo;  // first row / first column of the tile
    int HR, HC;          // halo rows / columns
    bool seg;            // tile lies inside one row
};

// One block = 4 wave64s; WAVES_M of them split the BM output channels, the others the
// BN phase pixels; each wave owns WM x WN MFMA tiles of 32 x 32.  CC input channels form
// one step (CC/16 MFMA k-steps of 16).  NCH_ITEMS: NCHW halo items (8 channels x 8
// columns) per thread; NHWC_VECS: NHWC halo 16-byte vectors per thread; OCC: blocks per
// compute unit the register and LDS budgets are sized for.
// PAIR (channels-first, stride 2 on the innermost axis, two wave rows): the two wave rows
// compute the two column phases r2 = 0, 1 of the same BM/2 output channels instead of two
// channel halves of one phase, so the block owns whole output rows and stores them with
// 16-byte vectors.
// ROWS8 (channels-first): input rows are whole 16-byte vectors (innermost size a multiple
// of 8), so a halo vector is one 16-byte load; otherwise (an even innermost size) it is
// four 4-byte loads and the columns past the row end are zeroed when the halo is stored.
template <bool CL, int WAVES_M, int WM, int WN, int CC, int NCH_ITEMS, int NHWC_VECS, int OCC, bool Q8 = false>
struct IgCfg {
    static constexpr int WAVES_N = 4 / WAVES_M;
    static constexpr int BM = WAVES_M * WM * 32;
    static constexpr int BN = WAVES_N * WN * 32;
    static constexpr int ROW = CC * 2 + 16;   // LDS bytes per staged row (data + 16 pad)
    static constexpr int CHUNKS = CC / 8;     // 16-byte chunks per row
    static constexpr int KSUB = CC / 16;      // MFMA k-steps per step
    static constexpr int WVEC = BM * CHUNKS / kThreads;
    static constexpr int LDS = lds_budget(OCC);
    // DIRECT (one wave row, float16): every wave reads the weights of its MFMAs straight
    // into registers from the fragment-major packing, so LDS holds no weight tiles but two
    // halo buffers (the next group's halo is stored while the current one is read).
    static constexpr bool DIRECT = WAVES_M == 1 && !Q8;
    static constexpr int HALO_BYTES = DIRECT ? ((LDS - kSinkBytes - tail_bytes(Q8)) / 2) / 16 * 16
                                             : LDS - 2 * BM * ROW - kSinkBytes - tail_bytes(Q8);
    static constexpr int HALO_BUFS = DIRECT ? 2 : 1;
    static_assert(BM * CHUNKS % kThreads == 0, "weight tile must split evenly");
    static_assert(HALO_BYTES > 0, "LDS budget");
};

// Q8 (channels-last): the quantized operation on the int8 MFMA v_mfma_i32_32x32x32_i8.
// Operands are taken to the signed domain (uint8 values XOR 0x80, i.e. minus 128, and
// the zero points with them); input positions outside the input hold the input zero
// point instead of 0, so every iterated tap contributes (x - x_zp) * (w - w_zp) and
//   sum (x - x_zp)(w - w_zp) = sum x w - w_zp * Sx - x_zp * Sw + x_zp * w_zp * Cg * T
// with Sx the sum of the iterated inputs (from the channel sums xsum, per pixel; only
// when some w_zp is non-zero), Sw the sum of the iterated weights (from wsum, per
// channel) and T the iterated tap count.  A step is CC * 2 int8 channels (the same
// 16-byte chunks and LDS rows as the float16 instances).
template <bool CL, int WAVES_M, int WM, int WN, int CC, int NCH_ITEMS, int NHWC_VECS, int OCC, bool PAIR, bool ROWS8,
          bool Q8 = false, bool WDMA = false>
__global__ __launch_bounds__(kThreads, OCC) void igemm_kernel(const _Float16 *x, const _Float16 *__restrict__ wp,
                                                            const _Float16 *__restrict__ bias,
                                                            _Float16 *__restrict__ y, IgArgs p)
{
    using Cfg = IgCfg<CL, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC, Q8>;
    static_assert(!Q8 || (CL && !PAIR && ROWS8), "quantized instances: channels-last");
    using XE = std::conditional_t<Q8, signed char, _Float16>;  // element of x and of the packed weights
    using AccV = std::conditional_t<Q8, i32x16, f32x16>;
    constexpr int CCH = Q8 ? 2 * CC : CC;   // channels per step
    constexpr int CH16 = Q8 ? 16 : 8;       // channels per 16-byte chunk
    const XE *const xe = reinterpret_cast<const XE *>(x);
    const XE *const we = reinterpret_cast<const XE *>(wp);
    constexpr int WAVES_N = Cfg::WAVES_N, BM = Cfg::BM, BN = Cfg::BN, ROW = Cfg::ROW;
    constexpr int CHUNKS = Cfg::CHUNKS, KSUB = Cfg::KSUB, WVEC = Cfg::WVEC;
    (void)WAVES_N;
    static_assert(!PAIR || (!CL && WAVES_M == 2), "column-phase pairs: channels-first, two wave rows");
    static_assert(ROWS8 || (!CL && !PAIR), "narrow-row loads: channels-first, unpaired");
    constexpr int BMM = PAIR ? BM / 2 : BM;  // output channels per block

    // One LDS array: two weight-tile buffers, the halo buffer, and a per-lane sink for
    // halo stores that have no destination (keeps those stores branch-free).  After the
    // main loop the whole array holds the output tile.
    __shared__ __attribute__((aligned(16))) unsigned char lds[Cfg::LDS];
    constexpr bool DIRECT = Cfg::DIRECT;
    // WDMA (the 256 x 256 block, float16 or int8, with four taps per group): the weight tiles are
    // copied from global memory straight into LDS (no registers), two steps ahead, into a
    // ring of three buffers of unpadded 128-byte rows whose 16-byte chunks are permuted
    // per row (see wdma_issue), so fragment reads stay free of bank conflicts.
    static_assert(!WDMA || (!DIRECT && BM == 256 && CC == 64 && WAVES_M == 2), "WDMA: the 256 x 256 block");
    constexpr int WROW = WDMA ? CC * 2 : ROW;  // LDS bytes per weight row
    constexpr int NWBUF = WDMA ? 3 : 2;
    constexpr int HALO_B =
        WDMA ? Cfg::LDS - NWBUF * BM * WROW - kSinkBytes - tail_bytes(Q8) : Cfg::HALO_BYTES;
    static_assert(HALO_B > 0, "LDS budget");
    auto lds_w = [&](int buf) -> unsigned char * { return lds + buf * (BM * WROW); };
    unsigned char *const lds_h = DIRECT ? lds : lds + NWBUF * BM * WROW;  // DIRECT: halo buffer 0
    unsigned char *const lds_sink = lds_h + Cfg::HALO_BUFS * HALO_B;
    float *const sbias = reinterpret_cast<float *>(lds_sink + kSinkBytes);  // kept to the end
    int *const sq_comp = reinterpret_cast<int *>(lds_sink + kSinkBytes);      // Q8: the same region
    float *const sq_mult = reinterpret_cast<float *>(sq_comp + 256);
    int *const sq_wz = sq_comp + 512;
    static_assert(BM <= 256, "bias region");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: a scalar
    const int wm = wave % WAVES_M;
    const int wn = wave / WAVES_M;

    // ---------------- which phase / tile this block computes ----------------
    // Equal phases: each XCD takes a contiguous range of work (the phases of a pixel tile
    // share its L2).  Unequal phases: launch order, heaviest phase first, so the blocks
    // of every weight class spread over all XCDs and the light ones fill in last.
    const int v = p.interleave ? xcd_remap(blockIdx.x, p.nblocks) : int(blockIdx.x);
    int ph, local;
    if (p.interleave) {
        ph = v % p.nphase;
        local = v / p.nphase;
    } else {
        ph = 0;
        while (v >= p.ph_start[ph + 1]) ++ph;
        local = v - p.ph_start[ph];
    }
    const int r0 = p.ph_r[ph] & 0xff, r1 = (p.ph_r[ph] >> 8) & 0xff, r2 = p.ph_r[ph] >> 16;  // PAIR: r2 = 0
    const int k00 = p.tk0[0][r0], k01 = p.tk0[1][r1], k02 = p.tk0[2][r2];
    const int ks0 = p.kstep[0], ks1 = p.kstep[1], ks2 = p.kstep[2];
    const int b00 = p.tb0[0][r0], bs0 = p.bstep[0], bs1 = p.bstep[1], bs2 = p.bstep[2];
    const int J0 = (p.O[0] - r0 + p.s[0] - 1) / p.s[0];
    const int J1 = (p.O[1] - r1 + p.s[1] - 1) / p.s[1];
    const int J2 = (p.O[2] - r2 + p.s[2] - 1) / p.s[2];
    const int nt0 = p.ntap[0][r0], nt1 = p.ntap[1][r1], nt2 = p.ntap[2][r2];

    Tile tl;
    tl.seg = J2 >= BN;
    const int tpr = tl.seg ? (J2 + BN - 1) / BN : 1;
    const int ptiles = tl.seg ? J1 * tpr : (J1 * J2 + BN - 1) / BN;
    int rest = local;
    const int pt = rest % ptiles;
    rest /= ptiles;
    const int j0 = rest % J0;
    rest /= J0;
    const int n = rest % p.N;
    rest /= p.N;
    const int g = rest % p.G;
    const int mt = rest / p.G;

    const int b1max = p.tb0[1][r1], b1min = nt1 ? b1max - (nt1 - 1) * bs1 : b1max;
    int b2max = p.tb0[2][r2], b2min = nt2 ? b2max - (nt2 - 1) * bs2 : b2max;
    if (PAIR) {  // the halo spans the taps of both column phases (same tap count)
        b2max = max(b2max, int(p.tb0[2][1]));
        b2min = min(b2min, p.tb0[2][1] - (nt2 - 1) * bs2);
    }
    // PAIR: column shift of this wave's phase inside the halo
    const int cshift = PAIR ? p.tb0[2][wm] - (nt2 - 1) * bs2 - b2min : 0;
    if (tl.seg) {
        tl.row_lo = pt / tpr;
        tl.col_lo = (pt % tpr) * BN;
        tl.q0 = tl.row_lo * J2 + tl.col_lo;
        tl.q1 = tl.q0 + min(BN, J2 - tl.col_lo);
        tl.HR = 1 + (b1max - b1min);
        tl.HC = (tl.q1 - tl.q0) + (b2max - b2min);
    } else {
        tl.q0 = pt * BN;
        tl.q1 = min(tl.q0 + BN, J1 * J2);
        tl.row_lo = tl.q0 / J2;
        tl.col_lo = 0;
        tl.HR = (tl.q1 - 1) / J2 - tl.row_lo + 1 + (b1max - b1min);
        tl.HC = J2 + (b2max - b2min);
    }
    const int i1o = tl.row_lo + b1min;  // input coordinates of halo (0, 0)
    const int i2o = tl.col_lo + b2min;

    // taps along axis 0 whose input plane j0 + beta lies inside [0, L0)
    int t0_first = 0, t0_end = 0;
    {
        int f = nt0, e = 0;
        for (int t = 0; t < nt0; ++t) {
            const int i0 = j0 + b00 - t * bs0;
            if (i0 >= 0 && i0 < p.L[0]) {
                if (f == nt0) f = t;
                e = t + 1;
            }
        }
        t0_first = f;
        t0_end = (f == nt0) ? f : e;
    }
    const int nsteps = p.nchunk * (t0_end - t0_first) * nt1 * nt2;

    // ---------------- per-lane halo offsets of this wave's pixel columns ----------------
    int hoff[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        int q = tl.q0 + (wn * WN + j) * 32 + (lane & 31);
        if (q >= tl.q1) q = tl.q1 - 1;
        const int row = tl.seg ? tl.row_lo : q / J2;
        const int col = q - row * J2;
        hoff[j] = ((row - tl.row_lo) * tl.HC + (col - tl.col_lo)) * ROW + (lane >> 5) * 16;
    }

    AccV acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int L0 = p.L[0], L1 = p.L[1], L2 = p.L[2];
    const size_t plane_in = size_t(L0) * L1 * L2;

    // ---------------- step order: chunk, axis-0 tap, axis-1 tap, axis-2 tap ----------------
    struct StepIdx {
        int chunk, t0, t1, t2;
    };
    auto advance = [&](StepIdx &q) {
        if (++q.t2 == nt2) {
            q.t2 = 0;
            if (++q.t1 == nt1) {
                q.t1 = 0;
                if (++q.t0 == t0_end) {
                    q.t0 = t0_first;
                    ++q.chunk;
                }
            }
        }
    };

    // ---------------- weight tile: BM rows x CC channels of Wp ----------------
    const size_t wrow0 = size_t(g) * p.T;
    // The packed weights' padded sizes as opaque scalars: the compiler then keeps them
    // (spilling to vector lanes if it must) instead of re-reading them from the kernel
    // arguments inside the loop, where that scalar load's wait also waits for the LDS
    // reads in flight.
    int wCgp = p.Cgp, wMgp = p.Mgp;
    asm volatile("" : "+s"(wCgp), "+s"(wMgp));
    // PAIR: rows [0, BMM) hold column phase 0's tap, rows [BMM, BM) phase 1's tap; the
    // loads k < WVEC/2 of every thread cover exactly the first half.
    static_assert(!PAIR || (WVEC % 2 == 0 && (WVEC / 2) * kThreads == BMM * CHUNKS), "phase halves");
    auto load_w = [&](const StepIdx &q, u32x4 *reg) {
        const int stride_vec = wCgp / CH16;  // 16-byte vectors per Wp row
        if constexpr (!PAIR) {
            const int tflat = ((k00 + q.t0 * ks0) * p.K[1] + (k01 + q.t1 * ks1)) * p.K[2] + (k02 + q.t2 * ks2);
            const size_t row0 = (wrow0 + tflat) * wMgp + size_t(mt) * BM;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(we + row0 * wCgp + size_t(q.chunk) * CCH);
#pragma unroll
            for (int k = 0; k < WVEC; ++k) {
                const int u = tid + k * kThreads;
                reg[k] = src[(u / CHUNKS) * stride_vec + (u % CHUNKS)];
            }
        } else {
            const int tb = ((k00 + q.t0 * ks0) * p.K[1] + (k01 + q.t1 * ks1)) * p.K[2] + q.t2 * ks2;
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // column phase h: WVEC / 2 loads
                const size_t row0 = (wrow0 + tb + p.tk0[2][h]) * wMgp + size_t(mt) * BMM;
                const u32x4 *src = reinterpret_cast<const u32x4 *>(we + row0 * wCgp + size_t(q.chunk) * CCH);
#pragma unroll
                for (int k = 0; k < WVEC / 2; ++k) {
                    const int u = tid + k * kThreads;
                    reg[h * (WVEC / 2) + k] = src[(u / CHUNKS) * stride_vec + (u % CHUNKS)];
                }
            }
        }
    };
    auto store_w = [&](int buf, const u32x4 *reg) {
#pragma unroll
        for (int k = 0; k < WVEC; ++k) {
            const int u = tid + k * kThreads;
            *reinterpret_cast<u32x4 *>(&lds_w(buf)[(u / CHUNKS) * ROW + (u % CHUNKS) * 16]) = reg[k];
        }
    };

    // ---------------- input halo of one (channel chunk, axis-0 tap) group ----------------
    // Fetched into registers during the first step of the previous group and written to
    // the (single) halo buffer between two barriers at the group boundary.  Loads read
    // a clamped, always valid address; a bit mask records which hold real input and
    // zeros are substituted when storing; every store has a destination (a per-lane sink
    // for items past the halo).
    constexpr int HREG = CL ? NHWC_VECS : NCH_ITEMS * 8;
    static_assert(HREG > 0 && HREG <= 32, "halo registers");
    const int va = floor_div8(i2o);
    const int nvc = floor_div8(i2o + tl.HC + 7) - va;
    const int halo_items = CL ? tl.HR * tl.HC * CHUNKS : tl.HR * nvc * CHUNKS;
    // halo item -> (row, column or vector) by multiply-high (items * divisor < 2^32)
    const UDiv dhalo(CL ? tl.HC : nvc);
    // Every halo item of a lane has the same 16-byte channel chunk (CHUNKS divides the
    // block size), so "chunk lies inside C/group" is cbase < ch_lim with a per-lane limit
    // held in a vector register: the loop never re-reads C/group from the kernel arguments
    // (a scalar load there is waited for together with the LDS reads in flight).
    static_assert(kThreads % CHUNKS == 0, "one channel chunk per lane");
    const int ch_lim = p.Cg - (tid % CHUNKS) * CH16;
    // load_halo_part<KB, KE>: loads KB..KE-1 of the HREG halo loads (all of them for
    // <0, HREG>) and returns their validity bits (NHWC: bit per load; NC..: bit per item).
    auto load_halo_part = [&](auto kb, auto ke, int chunk, int t0, u32x4 *reg) -> unsigned {
        constexpr int KB = decltype(kb)::value, KE = decltype(ke)::value;
        const int i0 = j0 + b00 - t0 * bs0;
        const int cbase = chunk * CCH;  // channel offset inside the group
        unsigned valid = 0;
        if (CL) {
            const XE *xb = xe + (size_t(n) * L0 + i0) * L1 * L2 * p.C + size_t(g) * p.Cg + cbase;
#pragma unroll
            for (int k = KB; k < KE; ++k) {
                const int u = tid + k * kThreads;
                const int pix = u / CHUNKS, ch = u % CHUNKS;
                const int hr = dhalo.div(pix), hc = pix - hr * tl.HC;
                const int i1 = i1o + hr, i2 = i2o + hc;
                const bool inside = (u < halo_items) & (i1 >= 0) & (i1 < L1) & (i2 >= 0) & (i2 < L2);
                const bool ok = inside & (cbase < ch_lim);
                const size_t off = ok ? (size_t(i1) * L2 + i2) * p.C + ch * CH16 : 0;
                reg[k] = *reinterpret_cast<const u32x4 *>((ok ? xb : xe) + off);
                // Q8: the bit records the position only (channel padding is zeroed on store)
                valid |= unsigned(Q8 ? inside : ok) << k;
            }
        } else {
            // items (halo row, aligned 8-column vector, channel octet), octet fastest:
            // a wave reads 8 channel planes x 128 contiguous bytes per load; load index
            // = item * 8 + channel of the octet
            const XE *xb = xe + (size_t(n) * p.C + size_t(g) * p.Cg + cbase) * plane_in + size_t(i0) * L1 * L2;
#pragma unroll
            for (int it = KB / 8; it < (KE + 7) / 8; ++it) {
                const int u = tid + it * kThreads;
                const int oct = u % CHUNKS;
                const int rv = u / CHUNKS;
                const int hr = dhalo.div(rv), vc = rv - hr * nvc;
                const int i1 = i1o + hr;
                const int i2 = (va + vc) * 8;
                const bool ok = (u < halo_items) & (i1 >= 0) & (i1 < L1) & (i2 >= 0) & (i2 < L2) & (cbase < ch_lim);
                // branch-free: the offset is computed for every item and masked (a select
                // of the whole address becomes a branch around its arithmetic, which splits
                // the step's schedule and keeps these instructions out of the MFMA stream)
                const size_t mask = size_t(0) - size_t(ok);
                const size_t off = (size_t(oct * 8) * plane_in + size_t(i1) * L2 + size_t(i2)) & mask;
                const XE *src = (ok ? xb : xe) + off;
                const size_t step = plane_in & mask;
                if constexpr (ROWS8) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (it * 8 + k >= KB && it * 8 + k < KE)
                            reg[it * 8 + k] = *reinterpret_cast<const u32x4 *>(src + k * step);
                } else {
                    // a column pair at or past the row end reads a valid address instead
                    // (store_halo replaces its values by zeros)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bool in = ok && i2 + 2 * q < L2;
                        const XE *sq = in ? src + 2 * q : xe;
                        const size_t sstep = in ? step : 0;
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            if (it * 8 + k >= KB && it * 8 + k < KE)
                                reg[it * 8 + k][q] = *reinterpret_cast<const unsigned *>(sq + k * sstep);
                    }
                }
                valid |= unsigned(ok) << it;
            }
        }
        return valid;
    };
    auto load_halo = [&](int chunk, int t0, u32x4 *reg) -> unsigned {
        return load_halo_part(std::integral_constant<int, 0>{}, std::integral_constant<int, HREG>{}, chunk, t0, reg);
    };
    auto store_halo_to = [&](unsigned char *const lds_h, const u32x4 *reg, unsigned valid, int chunk) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        unsigned char *const sink = lds_sink + lane * 16;
        if (CL) {
#pragma unroll
            for (int k = 0; k < NHWC_VECS; ++k) {
                const int u = tid + k * kThreads;
                unsigned char *dst = u < halo_items ? &lds_h[(u / CHUNKS) * ROW + (u % CHUNKS) * 16] : sink;
                if constexpr (Q8) {
                    // channels past C/group hold 0, positions outside the input the input
                    // zero point, the others the input in the signed domain
                    const unsigned fb = unsigned(p.q.x_zp) & 0xffu;
                    const unsigned f4 = fb | (fb << 8) | (fb << 16) | (fb << 24);
                    const u32x4 fill = {f4, f4, f4, f4};
                    const u32x4 flip = {p.q.xflip, p.q.xflip, p.q.xflip, p.q.xflip};
                    const bool chok = (u % CHUNKS) * CH16 < p.Cg - chunk * CCH;
                    *reinterpret_cast<u32x4 *>(dst) = !chok ? zero : (((valid >> k) & 1u) ? (reg[k] ^ flip) : fill);
                } else {
                    (void)chunk;
                    *reinterpret_cast<u32x4 *>(dst) = ((valid >> k) & 1u) ? reg[k] : zero;
                }
            }
        } else {
#pragma unroll
            for (int it = 0; it < NCH_ITEMS; ++it) {
                const int u = tid + it * kThreads;
                const bool ok = (valid >> it) & 1u;
                const bool here = u < halo_items;
                const int oct = u % CHUNKS;
                const int rv = u / CHUNKS;
                const int hr = dhalo.div(rv), vc = rv - hr * nvc;
                const u32x4 *in = reg + it * 8;
                // transpose 8 channels x 8 columns -> 8 columns x 8 channels
#pragma unroll
                for (int pp = 0; pp < 8; ++pp) {
                    const int hc = (va + vc) * 8 + pp - i2o;
                    u32x4 o;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const unsigned lo = in[2 * jj][pp >> 1], hi = in[2 * jj + 1][pp >> 1];
                        o[jj] = (pp & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                    }
                    unsigned char *dst =
                        (here && hc >= 0 && hc < tl.HC) ? &lds_h[(hr * tl.HC + hc) * ROW + oct * 16] : sink;
                    const bool inside = ROWS8 || (va + vc) * 8 + pp < L2;  // past the row end: zero
                    *reinterpret_cast<u32x4 *>(dst) = (ok && inside) ? o : zero;
                }
            }
        }
    };
    auto store_halo = [&](const u32x4 *reg, unsigned valid, int chunk) { store_halo_to(lds_h, reg, valid, chunk); };

    // The bias of the block's channels, staged once (read in the epilogue; the first
    // barrier below, or the epilogue's own, makes it visible).  Q8: per channel the
    // compensation bias - x_zp * Sw + x_zp * w_zp * Cg * T (int32, modulo 2^32), the
    // requantization multiplier and the shifted weight zero point; need_sx: some channel
    // of the block has a non-zero weight zero point.
    int need_sx = 0;
    if constexpr (Q8) {
        const unsigned taps_it = unsigned((t0_end - t0_first) * nt1 * nt2);
        int nz = 0;
        for (int mm = tid; mm < BM; mm += kThreads) {
            const int m = mt * BM + mm;
            int comp = 0, wz = 0;
            float mult = 0.0f;
            if (m < p.Mg) {
                const int mg = g * p.Mg + m;
                const int qi = p.q.w_per_channel ? mg : 0;
                wz = p.q.w_u8 ? int(static_cast<const unsigned char *>(p.q.w_zp)[qi]) - 128
                              : int(static_cast<const signed char *>(p.q.w_zp)[qi]);
                unsigned sw = 0;
                for (int t0 = t0_first; t0 < t0_end; ++t0)
                    for (int t1 = 0; t1 < nt1; ++t1)
                        for (int t2 = 0; t2 < nt2; ++t2) {
                            const int tflat = ((k00 + t0 * ks0) * p.K[1] + (k01 + t1 * ks1)) * p.K[2] + (k02 + t2 * ks2);
                            sw += unsigned(p.q.wsum[(size_t(g) * p.T + tflat) * p.Mgp + m]);
                        }
                unsigned c = p.q.bias ? unsigned(p.q.bias[mg]) : 0u;
                c -= unsigned(p.q.x_zp) * sw;
                c += unsigned(p.q.x_zp) * unsigned(wz) * unsigned(p.Cg) * taps_it;
                comp = __builtin_bit_cast(int, c);
                mult = requant_mult(p.q.x_scale, p.q.w_scale[qi], p.q.y_scale);
            }
            sq_comp[mm] = comp;
            sq_mult[mm] = mult;
            sq_wz[mm] = wz;
            nz |= wz != 0;
        }
        need_sx = __syncthreads_or(nz);
    }
    // float16: the block's bias (one channel per thread) is loaded here and staged in LDS
    // after the main loop, so the first operand loads do not wait for it
    static_assert(BMM <= kThreads, "one bias value per thread");
    // (an unconditional load from a valid address -- x when there is no bias -- so no
    // branch makes the compiler convert, and so wait for, the value here)
    const bool bias_ok = !Q8 && bias && tid < BMM && mt * BMM + tid < p.Mg;
    const _Float16 bias_h =
        bias_ok ? bias[g * p.Mg + mt * BMM + tid] : *reinterpret_cast<const _Float16 *>(bias ? bias : x);

    // ---------------- main loop ----------------
    if constexpr (DIRECT) {
        if (nsteps > 0) {
            // Weights straight from the fragment-major packing into MFMA operand registers:
            // fragment (32 channels of m, 16 input channels) of (g, tap) is 64 lanes x 16
            // bytes, contiguous, in lane order.  A ring of RING steps of fragments is kept in
            // flight, so a fragment is loaded RING - 1 steps before its MFMAs.  No barrier
            // between the steps of a group: the waves meet once per group, when the next
            // group's halo (loaded into registers at the group's first step) has been stored
            // into the other halo buffer.
            constexpr int RING = (WM * KSUB >= 8) ? 2 : 3;
            const int KB = p.Cgp / 16, MB = p.Mgp / 32;
            const f16x8 *const wf = reinterpret_cast<const f16x8 *>(wp);
            auto load_a = [&](const StepIdx &q, f16x8 (&dst)[WM][KSUB]) {
                const int tflat = ((k00 + q.t0 * ks0) * p.K[1] + (k01 + q.t1 * ks1)) * p.K[2] + (k02 + q.t2 * ks2);
                const f16x8 *src =
                    wf + (((size_t(g) * p.T + tflat) * MB + size_t(mt) * (BM / 32)) * KB + size_t(q.chunk) * KSUB) * 64 +
                    lane;
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int h = 0; h < KSUB; ++h) dst[i][h] = src[(size_t(i) * KB + h) * 64];
            };
            auto mma_direct = [&](const StepIdx &c, const unsigned char *hbuf, const f16x8 (&a)[WM][KSUB]) {
                const int toff = ((nt1 - 1 - c.t1) * bs1 * tl.HC + (nt2 - 1 - c.t2) * bs2) * ROW;
                const unsigned char *hb = hbuf + toff;
                f16x8 b[2][WN];
#pragma unroll
                for (int j = 0; j < WN; ++j) b[0][j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j]);
#pragma unroll
                for (int h = 0; h < KSUB; ++h) {
                    const int cb = h & 1, nb = cb ^ 1;
                    if (h + 1 < KSUB) {
#pragma unroll
                        for (int j = 0; j < WN; ++j)
                            b[nb][j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j] + (h + 1) * 32);
                    }
#pragma unroll
                    for (int i = 0; i < WM; ++i)
#pragma unroll
                        for (int j = 0; j < WN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][h], b[cb][j], acc[i][j], 0, 0, 0);
                }
            };
            u32x4 hreg[HREG];
            f16x8 ring[RING][WM][KSUB];
            StepIdx cur = {0, t0_first, 0, 0};
            StepIdx pf = cur;  // the next step whose fragments are loaded
#pragma unroll
            for (int d = 0; d < RING; ++d) {  // issued first: the halo's wait then covers them
                load_a(d < nsteps ? pf : cur, ring[d]);  // past the end: a valid, unused tile
                advance(pf);
            }
            {
                const unsigned v0 = load_halo(0, t0_first, hreg);
                store_halo_to(lds_h, hreg, v0, 0);
            }
            __syncthreads();
            unsigned hvalid = 0;
            int hchunk = 0, gi = 0;
            for (int s0 = 0; s0 < nsteps; s0 += RING) {
#pragma unroll
                for (int u = 0; u < RING; ++u) {
                    const int s = s0 + u;
                    if (s < nsteps) {
                        const bool group_first = cur.t1 == 0 && cur.t2 == 0;
                        const bool group_last = cur.t1 == nt1 - 1 && cur.t2 == nt2 - 1;
                        if (group_first) {  // the next group's halo comes in during this group
                            StepIdx ng = cur;
                            ng.t1 = nt1 - 1;
                            ng.t2 = nt2 - 1;
                            advance(ng);
                            if (ng.chunk < p.nchunk) {
                                hvalid = load_halo(ng.chunk, ng.t0, hreg);
                                hchunk = ng.chunk;
                            }
                        }
                        mma_direct(cur, lds_h + (gi & 1) * Cfg::HALO_BYTES, ring[u]);
                        load_a(s + RING < nsteps ? pf : cur, ring[u]);  // refill: RING steps ahead
                        advance(pf);
                        if (group_last) {
                            if (s + 1 < nsteps) store_halo_to(lds_h + ((gi + 1) & 1) * Cfg::HALO_BYTES, hreg, hvalid, hchunk);
                            __syncthreads();
                            ++gi;
                        }
                        advance(cur);
                    }
                }
            }
        }
    } else if constexpr (WDMA) {
        if (nsteps > 0) {
            // Step s reads weight buffer s % 3; during step s the tile of step s + 2 is copied
            // into buffer (s + 2) % 3, which step s - 1 read last (done: every wave passed the
            // barrier that ended step s - 1).  The barrier that ends step s first waits until
            // this wave's copy of step s + 1's tile has landed: it was issued in step s - 1,
            // so only the copies and halo loads issued in step s may still be in flight
            // (vector memory operations complete in issue order).
            //
            // LDS layout of a tile: row R (output channel of the block) holds 8 chunks of 16
            // bytes (8 float16 or 16 int8 input channels); chunk c is stored at position c ^ f(R) with
            // f(R) = (R & 7) ^ ((R >> 3) & 1), which gives the 16 lanes of one LDS cycle (16
            // consecutive rows, one chunk) 16 distinct bank groups, and 8 consecutive rows 8.
            // One copy instruction of a wave fills 64 consecutive 16-byte slots = 8 rows.
            const int dr = lane >> 3, dp = lane & 7;
            const int dc0 = dp ^ dr, dc1 = dc0 ^ 1;  // source chunk for even / odd instructions
            const int half = PAIR ? (wave >> 1) : 0;  // PAIR: waves 0-1 phase 0 rows, 2-3 phase 1
            const int drow = (PAIR ? (wave & 1) : wave) * 64 + dr;  // Wp row (within the tile) of k = 0
            // byte offsets inside the packed weights (the host plans WDMA for packed weights
            // under 2^31 bytes only)
            constexpr int ES = int(sizeof(XE));  // bytes per element (a 16-byte chunk holds CH16)
            const int doff0 = (drow * wCgp + dc0 * CH16) * ES, doff1 = (drow * wCgp + dc1 * CH16) * ES;
            int tk_half = PAIR ? int(p.tk0[2][half]) : 0;
            asm volatile("" : "+s"(tk_half));
            // Buffer-resource copies (not global-address ones): the compiler counts a
            // global-address copy into LDS as a pending LDS access of unknown order and then
            // waits for every LDS read in flight; these it counts as vector memory only.
            const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<XE *>(we), short(0), p.G * p.T * wMgp * wCgp * ES, 0x00020000);
            auto wdma_issue = [&](const StepIdx &q, int buf) {
                const int tflat = ((k00 + q.t0 * ks0) * p.K[1] + (k01 + q.t1 * ks1)) * p.K[2] +
                                  (PAIR ? q.t2 * ks2 + tk_half : k02 + q.t2 * ks2);
                const int src = (((int(wrow0) + tflat) * wMgp + mt * BMM) * wCgp + q.chunk * CCH) * ES;
                unsigned char *dst = lds_w(buf) + wave * 8 * 1024;
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (__attribute__((address_space(3))) void *)(dst + k * 1024),
                                                             16, (k & 1) ? doff1 : doff0, src + k * 8 * wCgp * ES, 0, 0);
            };
            // fragment (rows i*32 + l of the wave, chunk 2h + (lane >> 5)) of a tile
            const int fl = lane & 31, ff = (fl & 7) ^ ((fl >> 3) & 1);
            const int abase = (wm * WM * 32 + fl) * WROW + (((lane >> 5) ^ (ff & 1)) << 4);
            const int asw = (ff & 6) << 4;
            u32x4 hreg[HREG];
            StepIdx cur = {0, t0_first, 0, 0};
            {
                StepIdx nx = cur;
                advance(nx);
                wdma_issue(cur, 0);
                wdma_issue(nsteps > 1 ? nx : cur, 1);  // one step only: a harmless copy
                const unsigned v0 = load_halo(0, t0_first, hreg);
                store_halo(hreg, v0, 0);
            }
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            auto mma_step_d = [&](const StepIdx &c, int buf, auto pre0, auto pre1) {
                const int toff = ((nt1 - 1 - c.t1) * bs1 * tl.HC + (nt2 - 1 - c.t2) * bs2 + cshift) * ROW;
                const unsigned char *hb = lds_h + toff;
                const unsigned char *wb = lds_w(buf) + abase;
                f16x8 a[2][WM], b[2][WN];
#pragma unroll
                for (int i = 0; i < WM; ++i) a[0][i] = *reinterpret_cast<const f16x8 *>(wb + i * 32 * WROW + asw);
#pragma unroll
                for (int j = 0; j < WN; ++j) b[0][j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j]);
#pragma unroll
                for (int h = 0; h < KSUB; ++h) {
                    const int cb = h & 1, nb = cb ^ 1;
                    if (h + 1 < KSUB) {
                        const int ah = ((h + 1) << 5) ^ asw;
#pragma unroll
                        for (int i = 0; i < WM; ++i) a[nb][i] = *reinterpret_cast<const f16x8 *>(wb + i * 32 * WROW + ah);
#pragma unroll
                        for (int j = 0; j < WN; ++j)
                            b[nb][j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j] + (h + 1) * 32);
                    }
                    if (h == 0 || h == 1) {
                        if (h == 0) pre0();
                        else pre1();
                        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (WM + WN), 0);
#pragma unroll
                        for (int k = 0; k < WM * WN; ++k) {
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        }
                    } else {
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int i = 0; i < WM; ++i)
#pragma unroll
                        for (int j = 0; j < WN; ++j)
                            if constexpr (Q8)
                                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a[cb][i]),
                                                                                 __builtin_bit_cast(i32x4, b[cb][j]),
                                                                                 acc[i][j], 0, 0, 0);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[cb][i], b[cb][j], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // Four taps per (chunk, axis-0 tap) group (the host plans this kernel only then):
            // each step copies the tile of two steps ahead and loads a fixed quarter of the
            // next group's halo (the last step loads its quarter first, so the halo store
            // after it need not wait for that step's copies).
            const int ngroups = nsteps / 4;
            StepIdx grp = cur;
            int wb0 = 0;  // buffer of the group's first step: (4 * gi) % 3
            for (int gi = 0; gi < ngroups; ++gi) {
                StepIdx ng = grp;
                ng.t1 = nt1 - 1;
                ng.t2 = nt2 - 1;
                advance(ng);
                const bool has_ng = gi + 1 < ngroups;
                const int hch = has_ng ? ng.chunk : grp.chunk, ht0 = has_ng ? ng.t0 : grp.t0;  // last: a harmless reload
                unsigned hv = 0;
                auto g4_step = [&](auto U) {
                    constexpr int u = decltype(U)::value;
                    constexpr int PB = HREG * u / 4, PE = HREG * (u + 1) / 4;
                    const int s = gi * 4 + u;
                    StepIdx c = grp;
                    c.t1 = u / nt2;
                    c.t2 = u - c.t1 * nt2;
                    StepIdx n2 = c;  // the step two ahead (within this group or the next)
                    advance(n2);
                    advance(n2);
                    const StepIdx wtile = s + 2 < nsteps ? n2 : c;  // past the end: a harmless copy
                    const int bcur = (wb0 + u) % 3, bnext2 = (wb0 + u + 2) % 3;
                    auto dma = [&] { wdma_issue(wtile, bnext2); };
                    auto halo = [&] {
                        hv |= load_halo_part(std::integral_constant<int, PB>{}, std::integral_constant<int, PE>{},
                                             hch, ht0, hreg);
                    };
                    if constexpr (u == 3) mma_step_d(c, bcur, halo, dma);
                    else mma_step_d(c, bcur, dma, halo);
                    // 8 copies and PE - PB halo loads were issued in this step
                    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(8 + PE - PB) : "memory");
                };
                g4_step(std::integral_constant<int, 0>{});
                g4_step(std::integral_constant<int, 1>{});
                g4_step(std::integral_constant<int, 2>{});
                g4_step(std::integral_constant<int, 3>{});
                if (has_ng) {  // the next group's halo, between two barriers
                    store_halo(hreg, hv, hch);
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                }
                grp = ng;
                wb0 = (wb0 + 1) % 3;
            }
            // the copies past the last step land before the output stage reuses the LDS
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        }
    } else if (nsteps > 0) {
        u32x4 wreg[WVEC];
        u32x4 hreg[HREG];
        StepIdx cur = {0, t0_first, 0, 0};
        // the first weight tile and the first halo are in flight together (the weights,
        // issued first, are stored as soon as they arrive)
        load_w(cur, wreg);
        {
            const unsigned v0 = load_halo(0, t0_first, hreg);
            store_w(0, wreg);
            store_halo(hreg, v0, 0);
        }
        __syncthreads();
        // MFMAs of one step: weight tile from buffer buf, the halo window of the step's taps.
        // pre_w() issues the next weight tile's global loads, pre_h() a part of the next
        // halo, post() the weight tile's LDS writes; they are spread between the MFMAs of
        // the first, the second and the last k-step (one load per MFMA, one LDS write per
        // two MFMAs) rather than issued in bursts, so no wave waits at issue for the memory
        // pipes the four waves share.  The weight loads stay ahead of the halo loads (the
        // k-step boundary is a scheduling fence): loads complete in issue order, and the
        // LDS writes must not wait for the halo.
        auto mma_step = [&](const StepIdx &cur, int buf, auto pre_w, auto pre_h, auto post) {
            // tap shift inside the halo: (beta - beta_min) rows and columns
            const int toff = ((nt1 - 1 - cur.t1) * bs1 * tl.HC + (nt2 - 1 - cur.t2) * bs2 + cshift) * ROW;
            const unsigned char *hb = lds_h + toff;
            const unsigned char *wb = lds_w(buf) + (wm * WM * 32 + (lane & 31)) * ROW + (lane >> 5) * 16;
            f16x8 a[2][WM], b[2][WN];
#pragma unroll
            for (int i = 0; i < WM; ++i) a[0][i] = *reinterpret_cast<const f16x8 *>(wb + i * 32 * ROW);
#pragma unroll
            for (int j = 0; j < WN; ++j) b[0][j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j]);
#pragma unroll
            for (int h = 0; h < KSUB; ++h) {
                const int cb = h & 1, nb = cb ^ 1;
                if (h + 1 < KSUB) {  // fragments of the next k-step, read under this one's MFMAs
#pragma unroll
                    for (int i = 0; i < WM; ++i)
                        a[nb][i] = *reinterpret_cast<const f16x8 *>(wb + i * 32 * ROW + (h + 1) * 32);
#pragma unroll
                    for (int j = 0; j < WN; ++j)
                        b[nb][j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j] + (h + 1) * 32);
                }
                if (h == 0 || (h == 1 && h < KSUB - 1)) {
                    if (h == 0) pre_w();
                    else pre_h();
                    // fragment reads first, then alternate one global load and one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (WM + WN), 0);
#pragma unroll
                    for (int k = 0; k < WM * WN; ++k) {
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                } else if (h == KSUB - 1) {
                    if (KSUB == 2) pre_h();
                    post();
#pragma unroll
                    for (int k = 0; k < WM * WN / 2; ++k) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                    }
                } else {
                    // fence: the reads above are issued before these MFMAs
                    __builtin_amdgcn_sched_barrier(0);
                }
                // the MFMAs keep source order (each accumulator is touched once per k-step)
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int j = 0; j < WN; ++j)
                        if constexpr (Q8)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a[cb][i]),
                                                                             __builtin_bit_cast(i32x4, b[cb][j]),
                                                                             acc[i][j], 0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[cb][i], b[cb][j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        if (!Q8 && nt1 * nt2 == 4) {
            // Four taps per (chunk, axis-0 tap) group: one group per iteration, unrolled.
            // Each step loads the next step's weight tile and then a fixed quarter of the
            // next group's halo, all unconditionally, so every wait for a weight tile
            // leaves the halo quarter issued after it in flight.  (Float16 only: the int8
            // instances keep the one-group-at-a-time halo.)
            const int ngroups = nsteps / 4;
            StepIdx grp = cur;
            for (int gi = 0; gi < ngroups; ++gi) {
                StepIdx ng = grp;
                ng.t1 = nt1 - 1;
                ng.t2 = nt2 - 1;
                advance(ng);
                const bool has_ng = gi + 1 < ngroups;
                const int hch = has_ng ? ng.chunk : grp.chunk, ht0 = has_ng ? ng.t0 : grp.t0;  // last: a harmless reload
                unsigned hv = 0;
                auto g4_step = [&](auto U) {
                    constexpr int u = decltype(U)::value;
                    constexpr int PB = HREG * u / 4, PE = HREG * (u + 1) / 4;
                    const int s = gi * 4 + u;
                    StepIdx c = grp;
                    c.t1 = u / nt2;
                    c.t2 = u - c.t1 * nt2;
                    StepIdx nx = c;
                    advance(nx);
                    const StepIdx wnext = s + 1 < nsteps ? nx : c;  // the last step reloads a valid tile
                    mma_step(
                        c, s & 1, [&] { load_w(wnext, wreg); },
                        [&] {
                            hv |= load_halo_part(std::integral_constant<int, PB>{}, std::integral_constant<int, PE>{},
                                                 hch, ht0, hreg);
                        },
                        [&] { store_w((s + 1) & 1, wreg); });
                    __syncthreads();
                };
                g4_step(std::integral_constant<int, 0>{});
                g4_step(std::integral_constant<int, 1>{});
                g4_step(std::integral_constant<int, 2>{});
                g4_step(std::integral_constant<int, 3>{});
                if (has_ng) {  // the next group's halo, between two barriers
                    store_halo(hreg, hv, hch);
                    __syncthreads();
                }
                grp = ng;
            }
        } else {
            StepIdx nxt = cur;
            advance(nxt);
            unsigned hvalid = 0;
            int hchunk = 0;  // channel chunk of the halo held in registers
            for (int s = 0; s < nsteps; ++s) {
                const bool group_first = cur.t1 == 0 && cur.t2 == 0;
                const bool group_last = cur.t1 == nt1 - 1 && cur.t2 == nt2 - 1;
                // The next step's weight tile is loaded first: loads complete in issue
                // order, so waiting for it at the end of this step does not wait for the
                // halo loads.
                load_w(s + 1 < nsteps ? nxt : cur, wreg);  // the last step reloads a valid tile
                if (group_first) {  // the halo of the next group, if any, comes in meanwhile
                    StepIdx ng = cur;
                    ng.t1 = nt1 - 1;
                    ng.t2 = nt2 - 1;
                    advance(ng);
                    if (ng.chunk < p.nchunk) {
                        hvalid = load_halo(ng.chunk, ng.t0, hreg);
                        hchunk = ng.chunk;
                    }
                }
                // issue the prefetch loads here, ahead of the MFMAs (no later sinking)
                asm volatile("" ::: "memory");
                mma_step(cur, s & 1, [] {}, [] {}, [&] { store_w((s + 1) & 1, wreg); });
                __syncthreads();
                if (group_last && s + 1 < nsteps) {  // refresh the halo between two barriers
                    store_halo(hreg, hvalid, hchunk);
                    __syncthreads();
                }
                cur = nxt;
                advance(nxt);
            }
        }
    }

    if constexpr (!Q8)
        if (tid < BMM) sbias[tid] = bias_ok ? float(bias_h) : 0.0f;  // made visible by the output stage's barrier
    // The output stage, instantiated once per activation kind (one uniform switch picks
    // the instance), so no value pays for a dispatch.
    auto output_stage = [&](auto fin) {
        // lane and thread index recomputed here (two instructions) instead of being kept
        // live across the main loop, where the register allocator spills them to memory
        const int lane = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
        const int tid = wave * 64 + lane;
        // ---------------- epilogue: bias, round once, store ----------------
        // Accumulator element r of tile (i, j) belongs to channel i*32 + (r/4)*8 + (lane/32)*4
        // + r%4 of the wave's rows; the bias is added in float32 before the one rounding.
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        if constexpr (CL && WAVES_M != 2) __syncthreads();  // the staged bias is visible
        const int mwave = PAIR ? 0 : wm * WM * 32;  // first channel of the wave inside the tile
        auto bias_of = [&](int i, int rg, float *bv) {
            const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sbias[mwave + i * 32 + rg * 8 + (lane >> 5) * 4]);
    #pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = b4[e];
        };
        const int O1 = p.O[1], O2 = p.O[2];
        const size_t opix = size_t(p.O[0]) * O1 * O2;
        const int o0 = r0 + p.s[0] * j0;
        const int npix = tl.q1 - tl.q0;
        const int mvalid = min(BMM, p.Mg - mt * BMM);
        auto pixel_offset = [&](int pl) -> size_t {  // output pixel index of tile pixel pl
            const int q = tl.q0 + pl;
            const int row = tl.seg ? tl.row_lo : q / J2;
            const int col = q - row * J2;
            return (size_t(o0) * O1 + (r1 + p.s[1] * row)) * O2 + (r2 + p.s[2] * col);
        };
        if constexpr (CL && WAVES_M != 2) {
            // Channels-last, one wave row: straight from the accumulators.  A lane holds 4 consecutive
            // channels of one pixel per (tile, row group); lanes l and l + 32 hold adjacent
            // quadruples, so each store instruction writes 16 contiguous bytes per pixel.
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const bool vec = (p.M % 4 == 0) && ((g * p.Mg + mt * BM) % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % 8 == 0);
            const int mrow = wm * WM * 32;  // first channel of the wave inside the tile
            _Float16 *yp[WN];
    #pragma unroll
            for (int j = 0; j < WN; ++j) {
                const int pl = min((wn * WN + j) * 32 + (lane & 31), npix - 1);
                yp[j] = y + (size_t(n) * opix + pixel_offset(pl)) * p.M + g * p.Mg + mt * BM;
            }
    #pragma unroll
            for (int i = 0; i < WM; ++i)
    #pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int ml = mrow + i * 32 + rg * 8 + (lane >> 5) * 4;
                    float bv[4];
                    bias_of(i, rg, bv);
    #pragma unroll
                    for (int j = 0; j < WN; ++j) {
                        if ((wn * WN + j) * 32 + (lane & 31) >= npix) continue;
                        _Float16 v[4];
    #pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = _Float16(fin(acc[i][j][rg * 4 + e] + bv[e]));
                        if (vec && ml + 4 <= mvalid) {
                            const unsigned w0 = unsigned(__builtin_bit_cast(unsigned short, v[0])) |
                                                (unsigned(__builtin_bit_cast(unsigned short, v[1])) << 16);
                            const unsigned w1 = unsigned(__builtin_bit_cast(unsigned short, v[2])) |
                                                (unsigned(__builtin_bit_cast(unsigned short, v[3])) << 16);
                            *reinterpret_cast<u32x2 *>(yp[j] + ml) = u32x2{w0, w1};
                        } else {
    #pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (ml + e < mvalid) yp[j][ml + e] = v[e];
                        }
                    }
                }
            return;
        }
        // Channels-first, and channels-last with two wave rows: the block's output tile goes
        // through LDS (free once the main loop is done) and is stored with 16-byte vectors
        // along the contiguous direction (pixels; channels for channels-last, where a wave
        // then writes whole 128-byte lines instead of 8 bytes per lane and pixel).
        // Two wave rows (PACKED): tile layout [pixel][m] (PAIR: [column phase][pixel][m]),
        // channels innermost with a pitch of BMM + 4 elements: a lane's 4 consecutive
        // channels of one pixel are one 8-byte write, and a pitch of an odd number of 8-byte
        // words spreads the writes of 32 consecutive pixels over all banks; the store loop
        // regroups 8 pixels (PAIR: 4 pixels x 2 phases) of each channel into one 16-byte
        // vector.  One wave row (64-channel tiles, where the epilogue weighs less): layout
        // [m][pixel] with a pitch of BN + 8 elements, written per element.
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        constexpr bool PACKED = WAVES_M == 2;
        constexpr int CP = BMM + 4, TP = BN + 8;
        static_assert(CP % 8 == 4, "pitch: an odd number of 8-byte words");
        // the staged bias starts after the operand buffers and the sink
        constexpr int kBiasOffset =
            (DIRECT ? 0 : NWBUF * BM * WROW) + Cfg::HALO_BUFS * HALO_B + kSinkBytes;
        static_assert((PACKED ? (PAIR ? 2 : 1) * BN * CP : BMM * TP) * 2 <= kBiasOffset,
                      "output tile must fit in LDS below the bias");
        __syncthreads();  // every wave is done reading the operand buffers
        _Float16 *const stile = reinterpret_cast<_Float16 *>(lds);
    #pragma unroll
        for (int i = 0; i < WM; ++i)
    #pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int ml = (PAIR ? 0 : wm * WM * 32) + i * 32 + rg * 8 + (lane >> 5) * 4;  // 4 consecutive channels
                float bv[4];
                bias_of(i, rg, bv);
    #pragma unroll
                for (int j = 0; j < WN; ++j) {
                    const int pl = (wn * WN + j) * 32 + (lane & 31);
                    if constexpr (PACKED) {
                        float v[4];
    #pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = fin(acc[i][j][rg * 4 + e] + bv[e]);
                        // one rounding to nearest even per value (packed conversion)
                        const f16x2 lo = __builtin_convertvector(f32x2{v[0], v[1]}, f16x2);
                        const f16x2 hi = __builtin_convertvector(f32x2{v[2], v[3]}, f16x2);
                        *reinterpret_cast<u32x2 *>(&stile[((PAIR ? wm * BN : 0) + pl) * CP + ml]) =
                            u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
                    } else {
    #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            stile[(ml + e) * TP + pl] = _Float16(fin(acc[i][j][rg * 4 + e] + bv[e]));
                    }
                }
            }
        __syncthreads();
        if constexpr (CL) {
            // 8 channels of one pixel per lane and store; a pixel's channels of the tile are
            // contiguous in Y.  The 16-byte output stores of the epilogue are streaming
            // stores: Y is written once and read by no block.
            const bool vec = (p.M % 8 == 0) && ((g * p.Mg + mt * BM) % 8 == 0) && (mvalid % 8 == 0) &&
                             (reinterpret_cast<uintptr_t>(y) % 16 == 0);
            _Float16 *const yt = y + size_t(n) * opix * p.M + g * p.Mg + mt * BM;
            if (vec) {
                const int nc8 = mvalid / 8;
                for (int u = tid; u < npix * nc8; u += kThreads) {
                    const int pl = u / nc8, c8 = u - pl * nc8;
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(&stile[pl * CP + c8 * 8]);
                    const u32x2 hi = *reinterpret_cast<const u32x2 *>(&stile[pl * CP + c8 * 8 + 4]);
                    __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y},
                                                reinterpret_cast<u32x4 *>(yt + pixel_offset(pl) * p.M + c8 * 8));
                }
            } else {
                for (int u = tid; u < npix * mvalid; u += kThreads) {
                    const int pl = u / mvalid, ml = u - pl * mvalid;
                    yt[pixel_offset(pl) * p.M + ml] = stile[pl * CP + ml];
                }
            }
            return;
        }
        // 16-bit element (c & 1) of word w, for channel c of a staged quadruple
        auto lo_hi = [](unsigned a, unsigned b, int c) {  // a -> low half, b -> high half
            return (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        };

        if (PAIR) {
            // both column phases of each tile pixel: 2 * npix consecutive outputs per tile row
            // segment; 16-byte vectors when rows are whole vectors (then no vector crosses a row)
            const bool vec = (O2 % 8 == 0) && (tl.q0 % 4 == 0) && (npix % 4 == 0) &&
                             (reinterpret_cast<uintptr_t>(y) % 16 == 0);
            if (vec) {
                // A lane takes 4 channels x 4 pixels x 2 phases (four 16-byte stores); a wave
                // covers 8 channel quads x 8 pixel quads, so per channel 8 lanes write 128
                // contiguous bytes.
                const int mq = (mvalid + 3) / 4, pq = npix / 4;
                const int nbp = (pq + 7) / 8, nblk = ((mq + 7) / 8) * nbp;
                for (int blk = wave; blk < nblk; blk += kThreads / 64) {
                    const int m4 = (blk / nbp) * 8 + (lane >> 3);
                    const int v4 = (blk % nbp) * 8 + (lane & 7);
                    if (m4 >= mq || v4 >= pq) continue;
                    u32x2 d0[4], d1[4];  // phase 0 / phase 1: the 4 channels of pixel 4 * v4 + k
    #pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        d0[k] = *reinterpret_cast<const u32x2 *>(&stile[(4 * v4 + k) * CP + 4 * m4]);
                        d1[k] = *reinterpret_cast<const u32x2 *>(&stile[(BN + 4 * v4 + k) * CP + 4 * m4]);
                    }
                    _Float16 *const yq = y + (size_t(n) * p.M + g * p.Mg + mt * BMM + 4 * m4) * opix + pixel_offset(4 * v4);
    #pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (4 * m4 + c >= mvalid) break;
                        u32x4 o;
    #pragma unroll
                        for (int k = 0; k < 4; ++k)
                            o[k] = lo_hi(c < 2 ? d0[k].x : d0[k].y, c < 2 ? d1[k].x : d1[k].y, c);
                        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(yq + size_t(c) * opix));
                    }
                }
            } else {
                for (int u = tid; u < mvalid * 2 * npix; u += kThreads) {
                    const int ml = u / (2 * npix), e2 = u - ml * (2 * npix);
                    y[(size_t(n) * p.M + g * p.Mg + mt * BMM + ml) * opix + pixel_offset(e2 >> 1) + (e2 & 1)] =
                        stile[((e2 & 1) * BN + (e2 >> 1)) * CP + ml];
                }
            }
        } else {
            // runs of pixels per channel: contiguous in Y only along a row with unit stride
            const bool vec = p.s[2] == 1 && !tl.seg && (J2 % 8 == 0) && (tl.q0 % 8 == 0) && (O2 % 8 == 0) && r2 == 0 &&
                             (npix % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
            if (vec && !PACKED) {
                const int per = npix / 8;
                for (int u = tid; u < mvalid * per; u += kThreads) {
                    const int ml = u / per, p8 = u - ml * per;
                    const size_t off = (size_t(n) * p.M + g * p.Mg + mt * BM + ml) * opix + pixel_offset(p8 * 8);
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&stile[ml * TP + p8 * 8]),
                                                reinterpret_cast<u32x4 *>(y + off));
                }
            } else if (vec) {
                // A lane takes 4 channels x 8 pixels (four 16-byte stores); a wave covers 8
                // channel quads x 8 pixel octets, so per channel 8 lanes write 128 contiguous
                // bytes.
                const int mq = (mvalid + 3) / 4, po = npix / 8;
                const int nbp = (po + 7) / 8, nblk = ((mq + 7) / 8) * nbp;
                for (int blk = wave; blk < nblk; blk += kThreads / 64) {
                    const int m4 = (blk / nbp) * 8 + (lane >> 3);
                    const int p8 = (blk % nbp) * 8 + (lane & 7);
                    if (m4 >= mq || p8 >= po) continue;
                    u32x2 d[8];  // the 4 channels of pixel 8 * p8 + k
    #pragma unroll
                    for (int k = 0; k < 8; ++k) d[k] = *reinterpret_cast<const u32x2 *>(&stile[(8 * p8 + k) * CP + 4 * m4]);
                    _Float16 *const yq = y + (size_t(n) * p.M + g * p.Mg + mt * BM + 4 * m4) * opix + pixel_offset(8 * p8);
    #pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (4 * m4 + c >= mvalid) break;
                        u32x4 o;
    #pragma unroll
                        for (int k = 0; k < 4; ++k)
                            o[k] = lo_hi(c < 2 ? d[2 * k].x : d[2 * k].y, c < 2 ? d[2 * k + 1].x : d[2 * k + 1].y, c);
                        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(yq + size_t(c) * opix));
                    }
                }
            } else {
                // Phase-strided or ragged rows: a wave stores 64 consecutive tile pixels of
                // one channel (lane = pixel), so each store instruction touches the few
                // output lines those pixels span; the pixel offsets are computed once per
                // 64-pixel block and reused for every channel.
                for (int pb = 0; pb < npix; pb += 64) {
                    const int pl = pb + lane;
                    if (pl >= npix) continue;
                    _Float16 *const yq = y + (size_t(n) * p.M + g * p.Mg + mt * BM) * opix + pixel_offset(pl);
                    for (int ml = wave; ml < mvalid; ml += 4)
                        yq[size_t(ml) * opix] = stile[PACKED ? pl * CP + ml : ml * TP + pl];
                }
            }
        }
    };
    if constexpr (Q8) {
        // ---------------- quantized epilogue: compensation, requantization, store ----------------
        // (the staged per-channel values were made visible by the staging's own barrier)
        const int O1 = p.O[1], O2 = p.O[2];
        const size_t opix = size_t(p.O[0]) * O1 * O2;
        const int o0 = r0 + p.s[0] * j0;
        const int npix = tl.q1 - tl.q0;
        const int mvalid = min(BM, p.Mg - mt * BM);
        const int mrow = wm * WM * 32;
        unsigned char *const yb = reinterpret_cast<unsigned char *>(y);
        const bool vec = (p.M % 4 == 0) && ((g * p.Mg + mt * BM) % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % 4 == 0);
        unsigned char *yp[WN];
        unsigned sx[WN];  // sum of the iterated shifted inputs of the lane's pixels
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int pl = min((wn * WN + j) * 32 + (lane & 31), npix - 1);
            const int q = tl.q0 + pl;
            const int row = tl.seg ? tl.row_lo : q / J2;
            const int col = q - row * J2;
            yp[j] = yb + ((size_t(n) * opix + (size_t(o0) * O1 + (r1 + p.s[1] * row)) * O2 + (r2 + p.s[2] * col)) * p.M +
                          g * p.Mg + mt * BM);
            unsigned acc_s = 0;
            if (need_sx) {
                for (int t0 = t0_first; t0 < t0_end; ++t0) {
                    const int i0 = j0 + b00 - t0 * bs0;
                    for (int t1 = 0; t1 < nt1; ++t1) {
                        const int i1 = row + p.tb0[1][r1] - t1 * bs1;
                        for (int t2 = 0; t2 < nt2; ++t2) {
                            const int i2 = col + p.tb0[2][r2] - t2 * bs2;
                            const bool inside = i1 >= 0 && i1 < L1 && i2 >= 0 && i2 < L2;
                            acc_s += inside ? unsigned(p.q.xsum[(((size_t(n) * p.G + g) * L0 + i0) * L1 + i1) * L2 + i2])
                                            : unsigned(p.Cg) * unsigned(p.q.x_zp);
                        }
                    }
                }
            }
            sx[j] = acc_s;
        }
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int ml = mrow + i * 32 + rg * 8 + (lane >> 5) * 4;  // 4 consecutive channels
                const i32x4 cp = *reinterpret_cast<const i32x4 *>(&sq_comp[ml]);
                const i32x4 wz = *reinterpret_cast<const i32x4 *>(&sq_wz[ml]);
                float mult[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) mult[e] = sq_mult[ml + e];
#pragma unroll
                for (int j = 0; j < WN; ++j) {
                    if ((wn * WN + j) * 32 + (lane & 31) >= npix) continue;
                    unsigned packed = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const unsigned a = unsigned(acc[i][j][rg * 4 + e]) + unsigned(cp[e]) - unsigned(wz[e]) * sx[j];
                        const int code = requantize(a, mult[e], p.q.y_zp, p.q.y_lo, p.q.y_hi);
                        packed |= (unsigned(code) & 0xffu) << (8 * e);
                    }
                    if (vec && ml + 4 <= mvalid) {
                        *reinterpret_cast<unsigned *>(yp[j] + ml) = packed;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (ml + e < mvalid) yp[j][ml + e] = (unsigned char)(packed >> (8 * e));
                    }
                }
            }
    } else {
        (void)need_sx;
        with_activation(p.act, output_stage);
    }
}

// Wp[g][t][m][c] = W[g*Cg + c][m][t], zero outside c < Cg, m < Mg.  One thread writes
// 8 consecutive c (16 bytes); consecutive threads take consecutive taps so that the
// 8 strided reads of W are coalesced across the wave.  conv: W is a forward
// convolution's weight (M, C/group, k) whose stride-1 adjoint this call computes, read
// with its taps reversed: Wp[g][t][m][c] = Wconv[g*Mg + m][c][T-1-t].
// frag: the fragment-major packing read by the one-wave-row instances, in which the MFMA
// operand fragment (32 rows m, 16 channels c) of (g, t) is 64 lanes x 8 values in lane
// order (lane = 32 * ((c % 16) / 8) + m % 32):
//   Wf[g][t][m / 32][c / 16][lane][c % 8]
struct PackArgs {
    int G, Cg, Mg, Cgp, Mgp, T, conv, frag;
    long long total;  // G * (Cgp/8) * Mgp * T
};

__global__ __launch_bounds__(256) void pack_w_kernel(const _Float16 *__restrict__ w, _Float16 *__restrict__ wp,
                                                     PackArgs a)
{
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= a.total) return;
    int t, m, cv, g;
    if (a.total <= 0x7fffffffLL) {  // 32-bit index arithmetic (64-bit division is a long sequence)
        unsigned rest = unsigned(u);
        t = int(rest % unsigned(a.T));
        rest /= unsigned(a.T);
        m = int(rest % unsigned(a.Mgp));
        rest /= unsigned(a.Mgp);
        cv = int(rest % unsigned(a.Cgp / 8));
        g = int(rest / unsigned(a.Cgp / 8));
    } else {
        t = int(u % a.T);
        long long rest = u / a.T;
        m = int(rest % a.Mgp);
        rest /= a.Mgp;
        cv = int(rest % (a.Cgp / 8));
        g = int(rest / (a.Cgp / 8));
    }
    unsigned short v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int c = cv * 8 + k;
        const size_t src = a.conv ? ((size_t(g) * a.Mg + m) * a.Cg + c) * a.T + (a.T - 1 - t)
                                  : ((size_t(g) * a.Cg + c) * a.Mg + m) * a.T + t;
        // unconditional load from a valid address, masked afterwards: loads under a
        // branch are waited for one at a time
        const bool ok = c < a.Cg && m < a.Mg;
        const _Float16 e = w[ok ? src : 0];
        v[k] = ok ? __builtin_bit_cast(unsigned short, e) : (unsigned short)0;
    }
    const size_t gt = size_t(g) * a.T + t;
    _Float16 *dst = a.frag ? wp + (((gt * (a.Mgp / 32) + m / 32) * (a.Cgp / 16) + cv / 2) * 64 + (cv & 1) * 32 + m % 32) * 8
                           : wp + (gt * a.Mgp + m) * a.Cgp + cv * 8;
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = unsigned(v[2 * k]) | (unsigned(v[2 * k + 1]) << 16);
    *reinterpret_cast<u32x4 *>(dst) = o;
}

// Quantized weights: Wp[g][t][m][c] = w[g*Cg + c][m][t] in the signed domain (uint8
// values XOR 0x80), zero outside c < Cg, m < Mg; one thread writes 16 consecutive c.
struct PackQArgs {
    int G, Cg, Mg, Cgp, Mgp, T, w_u8;
    long long total;  // G * (Cgp/16) * Mgp * T
};

__global__ __launch_bounds__(256) void pack_wq_kernel(const unsigned char *__restrict__ w, signed char *__restrict__ wp,
                                                      PackQArgs a)
{
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= a.total) return;
    int t, m, cv, g;
    if (a.total <= 0x7fffffffLL) {  // 32-bit index arithmetic (64-bit division is a long sequence)
        unsigned rest = unsigned(u);
        t = int(rest % unsigned(a.T));
        rest /= unsigned(a.T);
        m = int(rest % unsigned(a.Mgp));
        rest /= unsigned(a.Mgp);
        cv = int(rest % unsigned(a.Cgp / 16));
        g = int(rest / unsigned(a.Cgp / 16));
    } else {
        t = int(u % a.T);
        long long rest = u / a.T;
        m = int(rest % a.Mgp);
        rest /= a.Mgp;
        cv = int(rest % (a.Cgp / 16));
        g = int(rest / (a.Cgp / 16));
    }
    const unsigned flip = a.w_u8 ? 0x80u : 0u;
    u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int c = cv * 16 + k;
        const bool ok = c < a.Cg && m < a.Mg;  // unconditional load, masked afterwards
        const unsigned raw = w[ok ? ((size_t(g) * a.Cg + c) * a.Mg + m) * a.T + t : 0];
        o[k >> 2] |= (ok ? (raw ^ flip) : 0u) << (8 * (k & 3));
    }
    *reinterpret_cast<u32x4 *>(wp + ((size_t(g) * a.T + t) * a.Mgp + m) * a.Cgp + cv * 16) = o;
}

// wsum[g][t][m] = sum over c of Wp[g][t][m][c] (signed bytes); one wave per row.
__global__ __launch_bounds__(256) void wsum_kernel(const signed char *__restrict__ wp, int *__restrict__ wsum,
                                                   long long rows, int Cgp)
{
    const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;  // the whole wave
    const u32x4 *src = reinterpret_cast<const u32x4 *>(wp + size_t(r) * Cgp);
    int sum = 0;
    for (int v = lane; v < Cgp / 16; v += 64) {
        const u32x4 q = src[v];
#pragma unroll
        for (int k = 0; k < 4; ++k) sum = __builtin_amdgcn_sdot4(int(q[k]), 0x01010101, sum, false);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) wsum[r] = sum;
}

// xsum[n][g][pixel] = sum over the group's channels of x in the signed domain
// (channels-last x: the channels of a pixel are contiguous).  Only the per-pixel
// correction of non-zero weight zero points reads it: when every weight zero point is 0
// in the signed domain, every block returns at once.
__global__ __launch_bounds__(256) void xsum_kernel(const unsigned char *__restrict__ x, int *__restrict__ xsum,
                                                   long long total, int G, int Cg, long long pixels, unsigned flip,
                                                   const unsigned char *__restrict__ w_zp, int wq_len, int w_u8)
{
    int nz = 0;
    for (int i = threadIdx.x; i < wq_len; i += blockDim.x)
        nz |= (w_u8 ? int(w_zp[i]) - 128 : int((signed char)w_zp[i])) != 0;
    if (!__syncthreads_or(nz)) return;
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= total) return;  // u = (n * G + g) * pixels + pixel
    const long long pix = u % pixels;
    const long long ng = u / pixels;
    const int g = int(ng % G);
    const long long n = ng / G;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t(n) * pixels + pix) * size_t(G) * Cg + size_t(g) * Cg);
    int sum = 0;
    for (int v = 0; v < Cg / 16; ++v) {
        const u32x4 q = src[v];
#pragma unroll
        for (int k = 0; k < 4; ++k) sum = __builtin_amdgcn_sdot4(int(q[k] ^ flip), 0x01010101, sum, false);
    }
    xsum[u] = sum;
}

// ---------------- host-side planning ----------------
struct Config {
    int waves_m, wm, wn, cc, nch_items, nhwc_vecs, occ;
    int bm() const { return waves_m * wm * 32; }
    int bn() const { return (4 / waves_m) * wn * 32; }
    int row() const { return cc * 2 + 16; }
    int chunks() const { return cc / 8; }
    bool direct(bool q8) const { return waves_m == 1 && !q8; }
    // the halo budget of the WDMA instance (three unpadded weight buffers)
    int halo_bytes_wdma(bool q8 = false) const { return lds_budget(occ) - 3 * bm() * cc * 2 - kSinkBytes - tail_bytes(q8); }
    int halo_bytes(bool q8 = false) const
    {
        return direct(q8) ? ((lds_budget(occ) - kSinkBytes - tail_bytes(q8)) / 2) / 16 * 16
                          : lds_budget(occ) - 2 * bm() * row() - kSinkBytes - tail_bytes(q8);
    }
    bool operator==(const Config &o) const
    {
        return waves_m == o.waves_m && wm == o.wm && wn == o.wn && cc == o.cc && nch_items == o.nch_items &&
               nhwc_vecs == o.nhwc_vecs && occ == o.occ;
    }
};

// The two compiled configurations (their template arguments must match launch_igemm).
constexpr Config kWide{2, 4, 4, 64, 2, 14, 1};    // 256 x 256 block, 128 x 128 per wave, 64 ch/step
constexpr Config kNarrow{1, 2, 4, 32, 2, 12, 1};  // 64 x 512 block, 64 x 128 per wave, 32 ch/step
constexpr Config kHalf{2, 2, 4, 64, 2, 14, 1};    // 128 x 256 block, 64 x 128 per wave, 64 ch/step
constexpr Config kMid{1, 2, 2, 32, 2, 12, 2};     // 64 x 256 block, 64 x 64 per wave, 32 ch/step, two blocks per CU
constexpr Config kSmall{1, 2, 1, 64, 2, 8, 2};    // 64 x 128 block, 64 x 32 per wave, two blocks per CU

// Candidates from the largest tile to the smallest.  Larger tiles re-read less and keep
// the MFMA pipes busier, but a launch with fewer blocks than the chip has block slots
// leaves compute units idle for its whole duration, which costs more (measured on a 2-D
// decoder layer, 1 to 8 images of 512 x 64 x 64 into 256 channels, and on 3-D layers of
// 2 x 128 x 16 x 32 x 32 into 64 channels).
constexpr Config kConfigs[] = {kWide, kHalf, kNarrow, kMid, kSmall};

struct Plan {
    Config cfg;
    bool pair;  // column-phase pairs (see IgCfg)
    bool wdma;  // the 256 x 256 block with weight tiles copied straight into LDS (see WDMA)
    IgArgs a;
    size_t ws_bytes;
};

// q8: the quantized instances (int8 elements, CC * 2 channels per step).
bool make_plan_cfg(const Geom &g, bool cl, const Config &cfg, Plan *pl, std::string *why, bool q8 = false)
{
    auto no = [&](const char *m) {
        *why = m;
        return false;
    };
    const int BN = cfg.bn();
    std::memset(&pl->a, 0, sizeof(pl->a));
    IgArgs &a = pl->a;
    for (int t = 0; t < kAxes; ++t) {
        if (g.s[t] > kMaxRes) return no("stride larger than 8");
        a.L[t] = int(g.L[t]);
        a.O[t] = int(g.O[t]);
        a.s[t] = int(g.s[t]);
        a.K[t] = int(g.K[t]);
        const int64_t gsd = std::__gcd(g.s[t], g.d[t]);
        a.kstep[t] = int(g.s[t] / gsd);
        a.bstep[t] = int(g.d[t] / gsd);
        if (g.K[t] > 32767 || g.d[t] / gsd > 32767) return no("kernel or dilation too large");
        for (int r = 0; r < g.s[t]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, t, r, &ph) || ph.ntaps > kMaxTap) return no("more than 8 taps per phase");
            a.ntap[t][r] = ph.ntaps;
            a.tk0[t][r] = ph.ntaps ? ph.k[0] : 0;
            a.tb0[t][r] = ph.ntaps ? ph.beta[0] : 0;
            for (int k = 0; k < ph.ntaps; ++k)  // the progression the kernel walks
                if (ph.k[k] != ph.k[0] + k * a.kstep[t] || ph.beta[k] != ph.beta[0] - k * a.bstep[t])
                    return no("internal: taps are not an arithmetic progression");
            if (ph.ntaps && (ph.beta[0] > 32767 || ph.beta[0] < -32767)) return no("pads too large");
        }
    }
    a.N = int(g.N);
    a.C = int(g.C);
    a.M = int(g.M);
    a.G = int(g.G);
    a.Cg = int(g.Cg);
    a.Mg = int(g.Mg);
    a.T = int(g.taps());
    const int cch = q8 ? 2 * cfg.cc : cfg.cc;  // channels per step
    a.nchunk = int((g.Cg + cch - 1) / cch);
    a.Cgp = a.nchunk * cch;
    // Column-phase pairs: channels-first output, stride 2 on the innermost axis, an even
    // output width (both phases then have the same pixel grid), equal tap counts and input
    // rows of whole 16-byte vectors.
    const bool pair = !q8 && !cl && cfg.waves_m == 2 && g.s[2] == 2 && g.O[2] % 2 == 0 &&
                      a.ntap[2][0] == a.ntap[2][1] && g.L[2] % 8 == 0;
    const int BMM = pair ? cfg.bm() / 2 : cfg.bm();
    a.mtiles = int((g.Mg + BMM - 1) / BMM);
    a.Mgp = a.mtiles * BMM;

    // phases with outputs, heaviest (most taps) first
    struct PhaseInfo {
        int r[3], taps, blocks;
    };
    PhaseInfo list[kMaxPh];
    int nph = 0;
    // WDMA: the 256 x 256 float16 block, rows of whole 16-byte vectors (or channels-last),
    // every phase with taps having four taps per (chunk, axis-0 tap) group, and the halo
    // within the smaller budget
    bool wdma = cfg == kWide && (cl || g.L[2] % 8 == 0);
    for (int r0 = 0; r0 < g.s[0]; ++r0)
        for (int r1 = 0; r1 < g.s[1]; ++r1)
            for (int r2 = 0; r2 < (pair ? 1 : g.s[2]); ++r2) {  // a pair is listed as r2 = 0
                if (r0 >= g.O[0] || r1 >= g.O[1] || r2 >= g.O[2]) continue;
                if (nph == kMaxPh) return no("more than 64 phases");
                PhaseInfo &pi = list[nph++];
                pi.r[0] = r0;
                pi.r[1] = r1;
                pi.r[2] = r2;
                pi.taps = a.ntap[0][r0] * a.ntap[1][r1] * a.ntap[2][r2];
                const int J0 = int((g.O[0] - r0 + g.s[0] - 1) / g.s[0]);
                const int J1 = int((g.O[1] - r1 + g.s[1] - 1) / g.s[1]);
                const int J2 = int((g.O[2] - r2 + g.s[2] - 1) / g.s[2]);
                const bool seg = J2 >= BN;
                const long long ptiles =
                    seg ? (long long)J1 * ((J2 + BN - 1) / BN) : ((long long)J1 * J2 + BN - 1) / BN;
                const long long blocks = ptiles * J0 * g.N * g.G * a.mtiles;
                if (blocks > (1ll << 30)) return no("too many blocks");
                pi.blocks = int(blocks);
                // halo capacity check (largest tile of this phase)
                const int n1 = a.ntap[1][r1], n2 = a.ntap[2][r2];
                const int e1 = n1 ? (n1 - 1) * a.bstep[1] : 0;
                int e2 = n2 ? (n2 - 1) * a.bstep[2] : 0;
                if (pair && n2)  // union of both phases' columns
                    e2 = std::max<int>(a.tb0[2][0], a.tb0[2][1]) - std::min<int>(a.tb0[2][0], a.tb0[2][1]) + e2;
                // rows a tile spans: tiles start at multiples of BN, so inside a row at
                // offsets that are multiples of gcd(BN, J2); the worst start is J2 - gcd
                const int rmax = J2 - std::__gcd(BN, J2);
                const int HR = seg ? 1 + e1 : std::min<int>(J1, (rmax + BN + J2 - 1) / J2) + e1;
                const int HC = seg ? BN + e2 : J2 + e2;
                if ((long long)HR * HC * cfg.row() > cfg.halo_bytes(q8)) return no("input halo exceeds LDS");
                if (pi.taps > 0 && (n1 * n2 != 4 || (long long)HR * HC * cfg.row() > cfg.halo_bytes_wdma(q8)))
                    wdma = false;
                if (cl && (long long)HR * HC * cfg.chunks() > (long long)cfg.nhwc_vecs * kThreads)
                    return no("input halo exceeds the loads of one block");
                const int nvc = (HC + 7) / 8 + 1;
                if (!cl && (long long)HR * nvc * cfg.chunks() > (long long)cfg.nch_items * kThreads)
                    return no("input halo exceeds the loads of one block");
            }
    std::stable_sort(list, list + nph, [](const PhaseInfo &x, const PhaseInfo &y) { return x.taps > y.taps; });
    a.nphase = nph;
    long long total = 0;
    bool uniform = true;
    for (int i = 0; i < nph; ++i) {
        a.ph_start[i] = int(total);
        a.ph_r[i] = list[i].r[0] | (list[i].r[1] << 8) | (list[i].r[2] << 16);
        total += list[i].blocks;
        uniform = uniform && list[i].blocks == list[0].blocks && list[i].taps == list[0].taps;
    }
    a.ph_start[nph] = int(total);
    if (total > INT32_MAX) return no("too many blocks");
    a.nblocks = int(total);
    a.interleave = uniform ? 1 : 0;
    pl->cfg = cfg;
    pl->pair = pair;
    pl->wdma = wdma;
    pl->ws_bytes = size_t(a.G) * a.T * a.Mgp * a.Cgp * (q8 ? 1 : sizeof(_Float16));
    if (pl->ws_bytes >= (size_t(1) << 31)) pl->wdma = false;  // its copies use 32-bit byte offsets
    return true;
}

// The largest tile that pads the output channels little (Mgp / Mg within 15 % of the
// least padding any servable tile has) and still gives every block slot of the chip (256
// compute units x blocks per unit) a block; if none does, the least-padded tile with the
// most blocks.
constexpr int kNumConfigs = int(sizeof(kConfigs) / sizeof(kConfigs[0]));
constexpr int kMpTile = kNumConfigs;      // the forced-tile index of the all-phase kernel
constexpr int kTsTile = kNumConfigs + 1;  // the forced-tile index of the tap-split kernel
std::atomic<int> g_forced_tile{-1};  // index into kConfigs, kMpTile, kTsTile, or -1: automatic

// tiles with quantized (int8) instances
bool has_q8(const Config &c) { return c == kWide || c == kHalf || c == kSmall; }

bool make_plan(const Geom &g, bool cl, Plan *pl, std::string *why, bool q8 = false)
{
    const int forced = g_forced_tile.load(std::memory_order_relaxed);
    if (forced == kMpTile || forced == kTsTile) {
        *why = forced == kMpTile ? "the all-phase kernel is forced" : "the tap-split kernel is forced";
        return false;
    }
    if (forced >= 0) {
        if (q8 && !has_q8(kConfigs[forced])) {
            *why = "the forced tile has no int8 instance";
            return false;
        }
        return make_plan_cfg(g, cl, kConfigs[forced], pl, why, q8);
    }
    constexpr int kCUs = 256;
    constexpr int kN = kNumConfigs;
    Plan cand[kN];
    bool ok[kN];
    double waste[kN], best_waste = 1e30;
    for (int i = 0; i < kN; ++i) {
        std::string w;
        ok[i] = (!q8 || has_q8(kConfigs[i])) && make_plan_cfg(g, cl, kConfigs[i], &cand[i], &w, q8);
        if (q8 && !has_q8(kConfigs[i])) w = "no int8 instance";
        if (!ok[i]) {
            if (i == 0 || why->empty()) *why = w;
            continue;
        }
        waste[i] = double(cand[i].a.Mgp) / double(g.Mg);
        best_waste = std::min(best_waste, waste[i]);
    }
    int pick = -1;
    for (int i = 0; i < kN; ++i) {
        if (!ok[i] || waste[i] > 1.15 * best_waste) continue;
        if (cand[i].a.nblocks >= kCUs * kConfigs[i].occ) {
            pick = i;
            break;
        }
        if (pick < 0 || cand[i].a.nblocks > cand[pick].a.nblocks) pick = i;
    }
    if (pick < 0) return false;
    *pl = cand[pick];
    return true;
}

template <bool CL, int WAVES_M, int WM, int WN, int CC, int NCH_ITEMS, int NHWC_VECS, int OCC, bool PAIR = false,
          bool ROWS8 = true, bool Q8 = false, bool WDMA = false>
void launch_cfg(const IgArgs &a, const _Float16 *x, const _Float16 *wp, const _Float16 *b, _Float16 *y,
                hipStream_t st)
{
    hipLaunchKernelGGL((igemm_kernel<CL, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC, PAIR, ROWS8, Q8, WDMA>),
                       dim3(unsigned(a.nblocks)), dim3(kThreads), 0, st, x, wp, b, y, a);
}

// Launches the instance of one configuration for the plan's layout (and column-phase
// pairing, which exists for the two-wave-row configurations only).
template <int WAVES_M, int WM, int WN, int CC, int NCH_ITEMS, int NHWC_VECS, int OCC>
bool launch_config(const Config &c, const Plan &pl, bool cl, const _Float16 *x, const _Float16 *wp,
                   const _Float16 *b, _Float16 *y, hipStream_t st)
{
    if (!(c == Config{WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC})) return false;
    if constexpr (WAVES_M == 2 && WM == 4 && WN == 4 && CC == 64) {
        if (pl.wdma) {
            if (cl)
                launch_cfg<true, 2, 4, 4, 64, NCH_ITEMS, NHWC_VECS, OCC, false, true, false, true>(pl.a, x, wp, b, y, st);
            else if (pl.pair)
                launch_cfg<false, 2, 4, 4, 64, NCH_ITEMS, NHWC_VECS, OCC, true, true, false, true>(pl.a, x, wp, b, y, st);
            else
                launch_cfg<false, 2, 4, 4, 64, NCH_ITEMS, NHWC_VECS, OCC, false, true, false, true>(pl.a, x, wp, b, y, st);
            return true;
        }
    }
    if (cl)
        launch_cfg<true, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC>(pl.a, x, wp, b, y, st);
    else if (pl.a.L[2] % 8 != 0)
        launch_cfg<false, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC, false, false>(pl.a, x, wp, b, y, st);
    else if (!pl.pair)
        launch_cfg<false, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC>(pl.a, x, wp, b, y, st);
    else if constexpr (WAVES_M == 2)
        launch_cfg<false, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC, true>(pl.a, x, wp, b, y, st);
    else
        return false;
    return true;
}

// The int8 (quantized, channels-last) instance of one configuration.
template <int WAVES_M, int WM, int WN, int CC, int NCH_ITEMS, int NHWC_VECS, int OCC>
bool launch_config_q8(const Config &c, const Plan &pl, const void *x, const void *wp, void *y, hipStream_t st)
{
    if (!(c == Config{WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC})) return false;
    if constexpr (WAVES_M == 2 && WM == 4 && WN == 4 && CC == 64) {
        if (pl.wdma) {
            launch_cfg<true, 2, 4, 4, 64, NCH_ITEMS, NHWC_VECS, OCC, false, true, true, true>(
                pl.a, static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(wp), nullptr,
                static_cast<_Float16 *>(y), st);
            return true;
        }
    }
    launch_cfg<true, WAVES_M, WM, WN, CC, NCH_ITEMS, NHWC_VECS, OCC, false, true, true>(
        pl.a, static_cast<const _Float16 *>(x), static_cast<const _Float16 *>(wp), nullptr, static_cast<_Float16 *>(y),
        st);
    return true;
}

}  // namespace

bool igemm_supports(const Geom &g, ct_dtype dt, bool cl, const void *x, std::string *why)
{
    // An empty input (a spatial size of 0: the outputs are bias alone) never reaches the
    // MFMA kernels: their halo and operand loads read through x's base pointer, which an
    // empty tensor need not give a valid address for.
    if (g.x_elems() <= 0) {
        *why = "empty input";
        return false;
    }
    if (dt == CT_FLOAT32) return igemm32_supports(g, cl, why);
    if (dt != CT_FLOAT16) {
        *why = "float16 and float32 only";
        return false;
    }
    if (g.Cg < 8 || g.Cg % 8 != 0) {
        *why = "C/group must be a multiple of 8";
        return false;
    }
    if (cl ? (g.C % 8 != 0) : (g.L[2] % 2 != 0)) {
        *why = cl ? "C must be a multiple of 8" : "innermost input size must be even";
        return false;
    }
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) {
        *why = "x must be 16-byte aligned";
        return false;
    }
    const int forced = g_forced_tile.load(std::memory_order_relaxed);
    if (forced == kMpTile) return mphase_supports(g, cl, why);
    if (forced == kTsTile) return tapsplit_supports(g, cl, why);
    Plan pl;
    if (make_plan(g, cl, &pl, why)) return true;
    std::string alt_why;
    return forced < 0 && (mphase_supports(g, cl, &alt_why) || tapsplit_supports(g, cl, &alt_why));
}

namespace {
// The all-phase kernel serves strided calls with few output channels per group, where
// the per-class kernel's blocks are short and every class re-reads the same input.
bool use_mphase(const Geom &g, bool cl)
{
    const int forced = g_forced_tile.load(std::memory_order_relaxed);
    std::string why;
    if (forced == kMpTile) return true;
    if (forced >= 0) return false;
    Plan pl;
    const bool classic = make_plan(g, cl, &pl, &why);
    return mphase_supports(g, cl, &why) && (!classic || g.Mg <= 64);
}
// The tap-split kernel serves stride-1 3-D calls with few output channels per group, where
// the phase kernel's blocks repeat every weight load in each wave and reload the input
// halo for every tap group.
bool use_tapsplit(const Geom &g, bool cl)
{
    const int forced = g_forced_tile.load(std::memory_order_relaxed);
    std::string why;
    if (forced == kTsTile) return true;
    if (forced >= 0) return false;
    if (!tapsplit_supports(g, cl, &why)) return false;
    Plan pl;
    return !make_plan(g, cl, &pl, &why) || (g.nsp == 3 && g.Mg <= 64);
}
}  // namespace

size_t igemm_workspace_bytes(const Geom &g, ct_dtype dt)
{
    if (dt != CT_FLOAT16) return 0;  // the float32 kernel reads W in place
    Plan pl;
    std::string why;
    // the largest packed weights of any tile and layout (tiles pad M differently), so a
    // workspace stays large enough whichever tile a later call uses
    size_t bytes = 0;
    for (const Config &c : kConfigs)
        for (const bool cl : {false, true})
            if (make_plan_cfg(g, cl, c, &pl, &why)) bytes = std::max(bytes, pl.ws_bytes);
    for (const bool cl : {false, true})
        bytes = std::max({bytes, mphase_workspace_bytes(g, cl), tapsplit_workspace_bytes(g, cl)});
    return bytes;
}

int igemm_tile_count() { return kNumConfigs + 2; }

void igemm_force_tile(int tile) { g_forced_tile.store(tile, std::memory_order_relaxed); }

int igemm_forced_tile() { return g_forced_tile.load(std::memory_order_relaxed); }

ct_status launch_igemm(const Geom &g, ct_dtype dt, bool cl, const void *x, const void *w, const void *bias,
                       void *y, const Act &act, void *workspace, size_t ws_bytes, hipStream_t st, std::string *err,
                       bool w_conv)
{
    if (dt == CT_FLOAT32) return launch_igemm32(g, cl, x, w, bias, y, act, st, err);
    const bool mp = use_mphase(g, cl);
    if (mp || use_tapsplit(g, cl)) {
        const size_t need = mp ? mphase_workspace_bytes(g, cl) : tapsplit_workspace_bytes(g, cl);
        if (need == 0) {
            std::string why;
            if (mp)
                mphase_supports(g, cl, &why);
            else
                tapsplit_supports(g, cl, &why);
            *err = why;
            return CT_EUNSUPPORTED;
        }
        void *wsp = workspace;
        if (!wsp) {
            hipError_t e = scratch_malloc(&wsp, need, st);
            if (e != hipSuccess) {
                *err = std::string("workspace allocation failed: ") + hipGetErrorString(e);
                return CT_EDEVICE;
            }
        } else if (ws_bytes < need) {
            *err = "workspace is smaller than convtranspose_workspace_size() reports";
            return CT_EINVAL;
        }
        ct_status s = mp ? launch_mphase(g, cl, x, w, bias, y, act, wsp, need, st, err, w_conv)
                         : launch_tapsplit(g, cl, x, w, bias, y, act, wsp, need, st, err, w_conv);
        if (!workspace) {
            const hipError_t f = hipFreeAsync(wsp, st);
            if (s == CT_OK && f != hipSuccess) {
                *err = std::string("scratch release failed: ") + hipGetErrorString(f);
                s = CT_EDEVICE;
            }
        }
        return s;
    }
    Plan pl;
    if (!make_plan(g, cl, &pl, err)) return CT_EUNSUPPORTED;
    pl.a.act = act;
    bool owned = false;
    void *wsp = workspace;
    if (!wsp) {
        hipError_t e = scratch_malloc(&wsp, pl.ws_bytes, st);
        if (e != hipSuccess) {
            *err = std::string("workspace allocation failed: ") + hipGetErrorString(e);
            return CT_EDEVICE;
        }
        owned = true;
    } else if (ws_bytes < pl.ws_bytes) {
        *err = "workspace is smaller than convtranspose_workspace_size() reports";
        return CT_EINVAL;
    }
    PackArgs pa;
    pa.G = pl.a.G;
    pa.Cg = pl.a.Cg;
    pa.Mg = pl.a.Mg;
    pa.Cgp = pl.a.Cgp;
    pa.Mgp = pl.a.Mgp;
    pa.T = pl.a.T;
    pa.conv = w_conv ? 1 : 0;
    pa.frag = pl.cfg.direct(false) ? 1 : 0;
    pa.total = (long long)pa.G * (pa.Cgp / 8) * pa.Mgp * pa.T;
    const _Float16 *wt = static_cast<const _Float16 *>(w);
    _Float16 *wpk = static_cast<_Float16 *>(wsp);
    hipLaunchKernelGGL(pack_w_kernel, dim3(unsigned((pa.total + 255) / 256)), dim3(256), 0, st, wt, wpk, pa);
    const _Float16 *xt = static_cast<const _Float16 *>(x);
    const _Float16 *bt = static_cast<const _Float16 *>(bias);
    _Float16 *yt = static_cast<_Float16 *>(y);
    const Config c = pl.cfg;
    mark_before(st);
    // (the template arguments repeat the Config constants above)
    const bool launched = launch_config<2, 4, 4, 64, 2, 14, 1>(c, pl, cl, xt, wpk, bt, yt, st) ||
                          launch_config<1, 2, 4, 32, 2, 12, 1>(c, pl, cl, xt, wpk, bt, yt, st) ||
                          launch_config<2, 2, 4, 64, 2, 14, 1>(c, pl, cl, xt, wpk, bt, yt, st) ||
                          launch_config<1, 2, 2, 32, 2, 12, 2>(c, pl, cl, xt, wpk, bt, yt, st) ||
                          launch_config<1, 2, 1, 64, 2, 8, 2>(c, pl, cl, xt, wpk, bt, yt, st);
    mark_after(st);
    hipError_t e = launched ? hipGetLastError() : hipErrorInvalidConfiguration;
    if (owned) {
        const hipError_t f = hipFreeAsync(wsp, st);
        if (e == hipSuccess) e = f;
    }
    if (e != hipSuccess) {
        *err = std::string("implicit-GEMM launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

ct_status launch_pack_w_frag(const Geom &g, const void *w, void *wp, int Cgp, int Mgp, bool w_conv, hipStream_t st,
                             std::string *err)
{
    PackArgs pa;
    pa.G = int(g.G);
    pa.Cg = int(g.Cg);
    pa.Mg = int(g.Mg);
    pa.Cgp = Cgp;
    pa.Mgp = Mgp;
    pa.T = int(g.taps());
    pa.conv = w_conv ? 1 : 0;
    pa.frag = 1;
    pa.total = (long long)pa.G * (pa.Cgp / 8) * pa.Mgp * pa.T;
    if (pa.total > 0)
        hipLaunchKernelGGL(pack_w_kernel, dim3(unsigned((pa.total + 255) / 256)), dim3(256), 0, st,
                           static_cast<const _Float16 *>(w), static_cast<_Float16 *>(wp), pa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("weight re-layout launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct

namespace ct {

// Largest depth (C/group x taps of one phase) whose int8 products cannot overflow the
// MFMA's int32 accumulator: depth * 128 * 128 < 2^31.
constexpr int64_t kMaxQ8Depth = (int64_t(1) << 31) / (128 * 128) - 1;

// Byte transpose of a batch of [rows][cols] matrices into [cols][rows] (channels-first
// <-> channels-last for 8-bit tensors), through a 64 x 64 LDS tile per block.
// VEC: rows and columns are multiples of 16 (and the buffers 16-byte aligned), so each
// thread moves one 16-byte vector in and one out; otherwise bytes, bounds-checked.
template <bool VEC>
__global__ __launch_bounds__(256) void transpose8_kernel(const unsigned char *__restrict__ src,
                                                         unsigned char *__restrict__ dst, long long rows,
                                                         long long cols)
{
    __shared__ unsigned char tile[64][65];
    const long long r0 = (long long)blockIdx.y * 64, c0 = (long long)blockIdx.x * 64;
    const size_t base = size_t(blockIdx.z) * size_t(rows) * size_t(cols);
    const int t = threadIdx.x;
    if constexpr (VEC) {
        const int rr = t / 4, cq = (t % 4) * 16;  // row of the tile, first of 16 columns
        if (r0 + rr < rows && c0 + cq < cols) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(src + base + size_t(r0 + rr) * cols + c0 + cq);
#pragma unroll
            for (int e = 0; e < 16; ++e) tile[rr][cq + e] = (unsigned char)(v[e >> 2] >> (8 * (e & 3)));
        }
        __syncthreads();
        const int cc = t / 4, rq = (t % 4) * 16;  // output row (= input column), first of 16 bytes
        if (c0 + cc < cols && r0 + rq < rows) {
            u32x4 o = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; ++e) o[e >> 2] |= unsigned(tile[rq + e][cc]) << (8 * (e & 3));
            *reinterpret_cast<u32x4 *>(dst + base + size_t(c0 + cc) * rows + r0 + rq) = o;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {  // 64 rows x 64 columns, consecutive threads on consecutive columns
            const int e = t + k * 256, rr = e / 64, cc = e % 64;
            if (r0 + rr < rows && c0 + cc < cols) tile[rr][cc] = src[base + size_t(r0 + rr) * cols + c0 + cc];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = t + k * 256, cc = e / 64, rr = e % 64;
            if (r0 + rr < rows && c0 + cc < cols) dst[base + size_t(c0 + cc) * rows + r0 + rr] = tile[rr][cc];
        }
    }
}

void transpose8(const void *src, void *dst, long long batch, long long rows, long long cols, hipStream_t st)
{
    if (batch * rows * cols == 0) return;
    const dim3 grid(unsigned((cols + 63) / 64), unsigned((rows + 63) / 64), unsigned(batch));
    const bool vec = rows % 16 == 0 && cols % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dst) % 16 == 0;
    if (vec)
        hipLaunchKernelGGL(transpose8_kernel<true>, grid, dim3(256), 0, st, static_cast<const unsigned char *>(src),
                           static_cast<unsigned char *>(dst), rows, cols);
    else
        hipLaunchKernelGGL(transpose8_kernel<false>, grid, dim3(256), 0, st, static_cast<const unsigned char *>(src),
                           static_cast<unsigned char *>(dst), rows, cols);
}

// Channels-first calls run the channels-last kernel between two transposes (x in, y out)
// through scratch.
bool qigemm_supports(const Geom &g, bool cl, const void *x, std::string *why)
{
    // the transposes' grids: (pixels or M) / 64 x (C or output pixels) / 64 x N
    if (!cl && ((g.C + 63) / 64 > 65535 || (g.out_pixels() + 63) / 64 > 65535 || g.N > 65535)) {
        *why = "too large for the layout transposes";
        return false;
    }
    if (g.Cg % 16 != 0 || g.C % 16 != 0) {
        *why = "C/group must be a multiple of 16";
        return false;
    }
    if (cl && reinterpret_cast<uintptr_t>(x) % 16 != 0) {
        *why = "x must be 16-byte aligned";
        return false;
    }
    int64_t taps = 1;
    for (int a = 0; a < kAxes; ++a) {
        int64_t most = 0;
        for (int r = 0; r < g.s[a]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, a, r, &ph)) {
                *why = "more than 16 taps per phase";
                return false;
            }
            most = std::max<int64_t>(most, ph.ntaps);
        }
        taps *= most;
    }
    if (g.Cg * taps > kMaxQ8Depth) {
        *why = "depth too large for exact int32 accumulation";
        return false;
    }
    Plan pl;
    return make_plan(g, true, &pl, why, true);
}


ct_status launch_qigemm(const Geom &g, bool cl, const void *x, const void *w, void *y, const QuantCall &qc,
                        hipStream_t st, std::string *err)
{
    Plan pl;
    if (!make_plan(g, true, &pl, err, true)) return CT_EUNSUPPORTED;
    IgArgs &a = pl.a;
    // workspace: packed weights, their channel sums, the input's channel sums; for
    // channels-first calls also x and y in channels-last order
    const size_t wp_bytes = (pl.ws_bytes + 255) / 256 * 256;
    const size_t wsum_elems = size_t(a.G) * a.T * a.Mgp;
    const size_t wsum_bytes = (wsum_elems * 4 + 255) / 256 * 256;
    const long long pixels = (long long)g.in_pixels();
    const long long xsum_elems = (long long)g.N * g.G * pixels;
    const size_t xsum_bytes = (size_t(std::max<long long>(xsum_elems, 1)) * 4 + 255) / 256 * 256;
    const size_t xt_bytes = cl ? 0 : (size_t(g.x_elems()) + 255) / 256 * 256;
    const size_t yt_bytes = cl ? 0 : (size_t(g.y_elems()) + 255) / 256 * 256;
    const size_t total = wp_bytes + wsum_bytes + xsum_bytes + xt_bytes + yt_bytes;
    void *ws = nullptr;
    hipError_t e = scratch_malloc(&ws, total, st);
    if (e != hipSuccess) {
        *err = std::string("workspace allocation failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    signed char *wpk = static_cast<signed char *>(ws);
    int *wsum = reinterpret_cast<int *>(static_cast<char *>(ws) + wp_bytes);
    int *xsum = reinterpret_cast<int *>(static_cast<char *>(ws) + wp_bytes + wsum_bytes);
    void *const y_final = y;
    if (!cl) {  // x (N, C, pixels) -> (N, pixels, C); the kernel writes y as (N, pixels, M)
        char *xt = static_cast<char *>(ws) + wp_bytes + wsum_bytes + xsum_bytes;
        transpose8(x, xt, g.N, g.C, pixels, st);
        x = xt;
        y = xt + xt_bytes;
    }

    PackQArgs pa;
    pa.G = a.G;
    pa.Cg = a.Cg;
    pa.Mg = a.Mg;
    pa.Cgp = a.Cgp;
    pa.Mgp = a.Mgp;
    pa.T = a.T;
    pa.w_u8 = qc.w_type == CT_UINT8;
    pa.total = (long long)pa.G * (pa.Cgp / 16) * pa.Mgp * pa.T;
    hipLaunchKernelGGL(pack_wq_kernel, dim3(unsigned((pa.total + 255) / 256)), dim3(256), 0, st,
                       static_cast<const unsigned char *>(w), wpk, pa);
    hipLaunchKernelGGL(wsum_kernel, dim3(unsigned((wsum_elems + 3) / 4)), dim3(256), 0, st, wpk, wsum,
                       (long long)wsum_elems, a.Cgp);
    const unsigned xflip = qc.x_type == CT_UINT8 ? 0x80808080u : 0u;
    if (xsum_elems > 0)
        hipLaunchKernelGGL(xsum_kernel, dim3(unsigned((xsum_elems + 255) / 256)), dim3(256), 0, st,
                           static_cast<const unsigned char *>(x), xsum, xsum_elems, a.G, a.Cg, pixels, xflip,
                           static_cast<const unsigned char *>(qc.w_zp), int(qc.wq_len), qc.w_type == CT_UINT8 ? 1 : 0);

    a.q.w_scale = qc.w_scale;
    a.q.w_zp = qc.w_zp;
    a.q.bias = qc.bias;
    a.q.wsum = wsum;
    a.q.xsum = xsum;
    a.q.x_scale = qc.x_scale;
    a.q.y_scale = qc.y_scale;
    a.q.x_zp = qc.x_type == CT_UINT8 ? qc.x_zp - 128 : qc.x_zp;
    a.q.y_zp = qc.y_zp;
    a.q.y_lo = qc.y_type == CT_INT8 ? -128 : 0;
    a.q.y_hi = qc.y_type == CT_INT8 ? 127 : 255;
    a.q.xflip = xflip;
    a.q.w_u8 = qc.w_type == CT_UINT8;
    a.q.w_per_channel = qc.wq_len == g.M && g.M != 1;
    const Config c = pl.cfg;
    mark_before(st);
    // (the template arguments repeat the Config constants above)
    const bool launched = launch_config_q8<2, 4, 4, 64, 2, 14, 1>(c, pl, x, wpk, y, st) ||
                          launch_config_q8<2, 2, 4, 64, 2, 14, 1>(c, pl, x, wpk, y, st) ||
                          launch_config_q8<1, 2, 1, 64, 2, 8, 2>(c, pl, x, wpk, y, st);
    mark_after(st);
    if (!cl) transpose8(y, y_final, g.N, g.out_pixels(), g.M, st);
    e = launched ? hipGetLastError() : hipErrorInvalidConfiguration;
    const hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = f;
    if (e != hipSuccess) {
        *err = std::string("int8 implicit-GEMM launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
