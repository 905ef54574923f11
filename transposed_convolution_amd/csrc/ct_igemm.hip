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
// Kernel structure (one workgroup = 4 wave64s, one phase, BM output channels x BN phase
// pixels of one (n, j0) plane):
//   * W is first re-laid out by pack_w_kernel into Wp[g][tap][m][c] (c contiguous,
//     zero padded to whole 32-channel chunks and whole channel tiles), so every weight
//     tile is a run of 16-byte loads.
//   * For each 32-channel chunk and each valid tap along axis 0, the input "halo" that
//     the tile's taps along axes 1 and 2 touch is staged once in LDS as
//     [row][col][32 channels]; every (t1, t2) tap then reads a shifted window of it.
//   * The MFMA v_mfma_f32_32x32x16_f16 runs with the weight tile as A (32 channels of
//     m) and the shifted halo window as B (32 pixels); float32 accumulators.
//   * Weight tiles and halos are double-buffered in LDS and prefetched into registers
//     one step ahead.  LDS rows are 80 bytes (64 data + 16 pad): 16-byte reads of 8 or
//     16 consecutive rows then fall in distinct bank groups.
//   * Epilogue: + bias, one round-to-nearest-even conversion, store.
//   * Blocks are re-ordered so that the blocks an XCD receives (hardware round-robin)
//     are consecutive in work order: all phases of one pixel tile share that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "ct_internal.hpp"

namespace ct {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCC = 32;                  // input channels per depth chunk
constexpr int kRow = 80;                 // LDS bytes per staged row (32 halves + pad)
constexpr int kMaxRes = 8;               // largest stride handled per axis
constexpr int kMaxTap = 8;               // largest tap count per residue and axis
constexpr int kMaxPh = 64;               // largest number of phases
constexpr int kHaloBytes = 56 * 1024;    // one halo buffer

struct IgArgs {
    int N, C, M, Cg, Mg, Cgp, Mgp, T, G;
    int L[3], O[3], s[3], K[3];
    int nchunk, mtiles;
    int nphase, interleave, nblocks;
    int ph_start[kMaxPh + 1];
    unsigned char ph_r[kMaxPh][3];
    // Taps of residue r on axis a form an arithmetic progression:
    //   k = tk0[a][r] + u * kstep[a],  beta = tb0[a][r] - u * bstep[a],  u in [0, ntap[a][r])
    // with kstep = s / gcd(s, d) and bstep = d / gcd(s, d).
    signed char ntap[3][kMaxRes];
    short tk0[3][kMaxRes];
    short tb0[3][kMaxRes];
    short kstep[3], bstep[3];
};

__device__ __forceinline__ int floor_div8(int v) { return v >= 0 ? v / 8 : -((-v + 7) / 8); }

// Block b goes to XCD b % 8; give each XCD a contiguous range of work indices.
__device__ __forceinline__ int xcd_remap(int b, int nb)
{
    const int q = nb >> 3, rem = nb & 7, x = b & 7, k = b >> 3;
    return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + k;
}

// Tile geometry of the phase pixels (j1, j2) a block covers.
struct Tile {
    int q0, q1;          // flattened pixel range in the J1 x J2 plane
    int row_lo, col_lo;  // first row / first column of the tile
    int HR, HC;          // halo rows / columns
    bool seg;            // tile lies inside one row
};

// WAVES wave64s per block, WAVES_M of them along output channels; each wave owns
// WM x WN MFMA tiles of 32 x 32.  NCH_ITEMS: NCHW halo items (8 channels x 8 columns)
// per thread; NHWC_VECS: NHWC halo 16-byte vectors per thread.  Together with the tile
// they bound the halo a block stages.
template <bool CL, int WAVES, int WAVES_M, int WM, int WN, int NCH_ITEMS, int NHWC_VECS>
__global__ __launch_bounds__(WAVES * 64, 1) void igemm_kernel(const _Float16 *__restrict__ x,
                                                            const _Float16 *__restrict__ wp,
                                                            const _Float16 *__restrict__ bias,
                                                            _Float16 *__restrict__ y, IgArgs p)
{
    constexpr int kThreads = WAVES * 64;
    constexpr int WAVES_N = WAVES / WAVES_M;
    constexpr int BM = WAVES_M * WM * 32;
    constexpr int BN = WAVES_N * WN * 32;
    // weight-tile 16-byte vectors per thread (threads past the tile load a valid
    // address and store into the sink)
    constexpr int WVEC = (BM * 4 + kThreads - 1) / kThreads;

    __shared__ __attribute__((aligned(16))) unsigned char lds_w[2][BM * kRow];
    __shared__ __attribute__((aligned(16))) unsigned char lds_h[2][kHaloBytes];
    // per-lane sink for halo stores that have no destination (keeps the stores branch-free)
    __shared__ __attribute__((aligned(16))) unsigned char lds_sink[64 * 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M;
    const int wn = wave / WAVES_M;

    // ---------------- which phase / tile this block computes ----------------
    const int v = xcd_remap(blockIdx.x, p.nblocks);
    int ph, local;
    if (p.interleave) {
        ph = v % p.nphase;
        local = v / p.nphase;
    } else {
        ph = 0;
        while (v >= p.ph_start[ph + 1]) ++ph;
        local = v - p.ph_start[ph];
    }
    const int r0 = p.ph_r[ph][0], r1 = p.ph_r[ph][1], r2 = p.ph_r[ph][2];
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
    const int b2max = p.tb0[2][r2], b2min = nt2 ? b2max - (nt2 - 1) * bs2 : b2max;
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
        hoff[j] = ((row - tl.row_lo) * tl.HC + (col - tl.col_lo)) * kRow + (lane >> 5) * 16;
    }

    f32x16 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---------------- loaders ----------------
    const int L0 = p.L[0], L1 = p.L[1], L2 = p.L[2];
    const size_t plane_in = size_t(L0) * L1 * L2;

    // Step order: chunk, then axis-0 tap, then axis-1 tap, then axis-2 tap.
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
    const size_t wrow0 = size_t(g) * p.T;
    auto load_w = [&](const StepIdx &q, u32x4 *reg) {
        const int tflat = ((k00 + q.t0 * ks0) * p.K[1] + (k01 + q.t1 * ks1)) * p.K[2] + (k02 + q.t2 * ks2);
        const size_t row0 = (wrow0 + tflat) * p.Mgp + size_t(mt) * BM;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(wp + row0 * p.Cgp + size_t(q.chunk) * kCC);
        const int stride_vec = p.Cgp / 8;  // 16-byte vectors per Wp row
#pragma unroll
        for (int k = 0; k < WVEC; ++k) {
            const int u = min(tid + k * kThreads, BM * 4 - 1);
            reg[k] = src[(u >> 2) * stride_vec + (u & 3)];
        }
    };
    auto store_w = [&](int buf, const u32x4 *reg) {
#pragma unroll
        for (int k = 0; k < WVEC; ++k) {
            const int u = tid + k * kThreads;
            unsigned char *dst = u < BM * 4 ? &lds_w[buf][(u >> 2) * kRow + (u & 3) * 16] : lds_sink + lane * 16;
            *reinterpret_cast<u32x4 *>(dst) = reg[k];
        }
    };

    // Halo of one (channel chunk, axis-0 tap) group.  It is fetched during the first
    // step of the previous group and stored into the other halo buffer (free for that
    // whole group) at the end of that step.  Loads read a clamped, always valid address
    // and a bit mask records which hold real input; zeros are substituted when storing,
    // and every store has a destination (a per-lane sink for items past the halo), so
    // no loaded value is merged or consumed before the MFMAs of the step are issued.
    constexpr int HREG = CL ? NHWC_VECS : NCH_ITEMS * 8;
    static_assert(HREG > 0 && HREG <= 32, "halo registers");
    const int va = floor_div8(i2o);
    const int nvc = floor_div8(i2o + tl.HC + 7) - va;
    const int halo_items = CL ? tl.HR * tl.HC * 4 : tl.HR * 4 * nvc;
    auto load_halo = [&](int chunk, int t0, u32x4 *reg) -> unsigned {
        const int i0 = j0 + b00 - t0 * bs0;
        const int cbase = chunk * kCC;  // channel offset inside the group
        unsigned valid = 0;
        if (CL) {
            const _Float16 *xb = x + (size_t(n) * L0 + i0) * L1 * L2 * p.C + size_t(g) * p.Cg + cbase;
#pragma unroll
            for (int k = 0; k < NHWC_VECS; ++k) {
                const int u = tid + k * kThreads;
                const int pix = u >> 2, ch = u & 3;
                const int hr = pix / tl.HC, hc = pix - hr * tl.HC;
                const int i1 = i1o + hr, i2 = i2o + hc;
                const bool ok = u < halo_items && i1 >= 0 && i1 < L1 && i2 >= 0 && i2 < L2 && cbase + ch * 8 < p.Cg;
                const size_t off = ok ? (size_t(i1) * L2 + i2) * p.C + ch * 8 : 0;
                reg[k] = *reinterpret_cast<const u32x4 *>((ok ? xb : x) + off);
                valid |= unsigned(ok) << k;
            }
        } else {
            // items: (halo row, channel octet, aligned 8-column vector)
            const _Float16 *xb = x + (size_t(n) * p.C + size_t(g) * p.Cg + cbase) * plane_in + size_t(i0) * L1 * L2;
#pragma unroll
            for (int it = 0; it < NCH_ITEMS; ++it) {
                const int u = tid + it * kThreads;
                const int hr = u / (4 * nvc);
                const int rem2 = u - hr * 4 * nvc;
                const int oct = rem2 / nvc, vc = rem2 - oct * nvc;
                const int i1 = i1o + hr;
                const int i2 = (va + vc) * 8;
                const bool ok = u < halo_items && i1 >= 0 && i1 < L1 && i2 >= 0 && i2 < L2 && cbase + oct * 8 < p.Cg;
                const _Float16 *src = ok ? xb + size_t(oct * 8) * plane_in + size_t(i1) * L2 + i2 : x;
                const size_t step = ok ? plane_in : 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) reg[it * 8 + k] = *reinterpret_cast<const u32x4 *>(src + k * step);
                valid |= unsigned(ok) << it;
            }
        }
        return valid;
    };
    auto store_halo = [&](int buf, const u32x4 *reg, unsigned valid) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        unsigned char *const sink = lds_sink + lane * 16;
        if (CL) {
#pragma unroll
            for (int k = 0; k < NHWC_VECS; ++k) {
                const int u = tid + k * kThreads;
                unsigned char *dst = u < halo_items ? &lds_h[buf][(u >> 2) * kRow + (u & 3) * 16] : sink;
                *reinterpret_cast<u32x4 *>(dst) = ((valid >> k) & 1u) ? reg[k] : zero;
            }
        } else {
#pragma unroll
            for (int it = 0; it < NCH_ITEMS; ++it) {
                const int u = tid + it * kThreads;
                const bool ok = (valid >> it) & 1u;
                const bool here = u < halo_items;
                const int hr = u / (4 * nvc);
                const int rem2 = u - hr * 4 * nvc;
                const int oct = rem2 / nvc, vc = rem2 - oct * nvc;
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
                    unsigned char *dst = (here && hc >= 0 && hc < tl.HC)
                                             ? &lds_h[buf][(hr * tl.HC + hc) * kRow + oct * 16]
                                             : sink;
                    *reinterpret_cast<u32x4 *>(dst) = ok ? o : zero;
                }
            }
        }
    };

    // ---------------- main loop ----------------
    if (nsteps > 0) {
        u32x4 wreg[WVEC];
        u32x4 hreg[HREG];
        StepIdx cur = {0, t0_first, 0, 0};
        {
            const unsigned v0 = load_halo(0, t0_first, hreg);
            store_halo(0, hreg, v0);
        }
        load_w(cur, wreg);
        store_w(0, wreg);
        __syncthreads();
        StepIdx nxt = cur;
        advance(nxt);
        int hbuf = 0;
        for (int s = 0; s < nsteps; ++s) {
            // the halo of the next group is fetched during the first step of this one
            bool fetch = false;
            unsigned hvalid = 0;
            if (cur.t1 == 0 && cur.t2 == 0) {
                StepIdx ng = cur;
                ng.t1 = nt1 - 1;
                ng.t2 = nt2 - 1;
                advance(ng);
                fetch = ng.chunk < p.nchunk;
                if (fetch) hvalid = load_halo(ng.chunk, ng.t0, hreg);
            }
            load_w(s + 1 < nsteps ? nxt : cur, wreg);  // the last step reloads a valid tile
            // issue the prefetch loads here, ahead of the MFMAs (no later sinking)
            asm volatile("" ::: "memory");

            // tap shift inside the halo: (beta - beta_min) rows and columns
            const int toff = ((nt1 - 1 - cur.t1) * bs1 * tl.HC + (nt2 - 1 - cur.t2) * bs2) * kRow;
            const unsigned char *hb = lds_h[hbuf] + toff;
            const unsigned char *wb = lds_w[s & 1] + (wm * WM * 32 + (lane & 31)) * kRow + (lane >> 5) * 16;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f16x8 a[WM], b[WN];
#pragma unroll
                for (int i = 0; i < WM; ++i)
                    a[i] = *reinterpret_cast<const f16x8 *>(wb + i * 32 * kRow + h * 32);
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    b[j] = *reinterpret_cast<const f16x8 *>(hb + hoff[j] + h * 32);
#pragma unroll
                for (int i = 0; i < WM; ++i)
#pragma unroll
                    for (int j = 0; j < WN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
            }

            if (fetch) store_halo(hbuf ^ 1, hreg, hvalid);
            store_w((s + 1) & 1, wreg);
            __syncthreads();
            cur = nxt;
            advance(nxt);
            if (cur.t1 == 0 && cur.t2 == 0) hbuf ^= 1;
        }
    }

    // ---------------- epilogue: bias, round once, store ----------------
    const int O1 = p.O[1], O2 = p.O[2];
    const size_t opix = size_t(p.O[0]) * O1 * O2;
    const int o0 = r0 + p.s[0] * j0;
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        const int q = tl.q0 + (wn * WN + j) * 32 + (lane & 31);
        if (q >= tl.q1) continue;
        const int row = tl.seg ? tl.row_lo : q / J2;
        const int col = q - row * J2;
        const int o1 = r1 + p.s[1] * row, o2 = r2 + p.s[2] * col;
        const size_t pix = (size_t(o0) * O1 + o1) * O2 + o2;
#pragma unroll
        for (int i = 0; i < WM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int mloc = mt * BM + wm * WM * 32 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (mloc >= p.Mg) continue;
                const int m = g * p.Mg + mloc;
                float val = acc[i][j][r];
                if (bias) val += float(bias[m]);
                const size_t off = CL ? ((size_t(n) * opix + pix) * p.M + m) : ((size_t(n) * p.M + m) * opix + pix);
                y[off] = _Float16(val);
            }
        }
    }
}

// Wp[g][t][m][c] = W[g*Cg + c][m][t], zero outside c < Cg, m < Mg.  One thread writes
// 8 consecutive c (16 bytes); consecutive threads take consecutive taps so that the
// 8 strided reads of W are coalesced across the wave.
struct PackArgs {
    int G, Cg, Mg, Cgp, Mgp, T;
    long long total;  // G * (Cgp/8) * Mgp * T
};

__global__ __launch_bounds__(256) void pack_w_kernel(const _Float16 *__restrict__ w, _Float16 *__restrict__ wp,
                                                     PackArgs a)
{
    const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= a.total) return;
    const int t = int(u % a.T);
    long long rest = u / a.T;
    const int m = int(rest % a.Mgp);
    rest /= a.Mgp;
    const int cv = int(rest % (a.Cgp / 8));
    const int g = int(rest / (a.Cgp / 8));
    unsigned short v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int c = cv * 8 + k;
        const _Float16 e =
            (c < a.Cg && m < a.Mg) ? w[((size_t(g) * a.Cg + c) * a.Mg + m) * a.T + t] : _Float16(0.0f);
        v[k] = __builtin_bit_cast(unsigned short, e);
    }
    _Float16 *dst = wp + ((size_t(g) * a.T + t) * a.Mgp + m) * a.Cgp + cv * 8;
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = unsigned(v[2 * k]) | (unsigned(v[2 * k + 1]) << 16);
    *reinterpret_cast<u32x4 *>(dst) = o;
}

// ---------------- host-side planning ----------------
struct Config {
    int waves, waves_m, wm, wn, nch_items, nhwc_vecs;
    int threads() const { return waves * 64; }
    int bm() const { return waves_m * wm * 32; }
    int bn() const { return (waves / waves_m) * wn * 32; }
};

// Both configurations run 8 waves (two per SIMD) so that one wave's loads and index
// arithmetic overlap the other's MFMAs.
Config pick_config(const Geom &g)
{
    if (g.Mg > 64) return Config{8, 2, 4, 2, 1, 6};  // 256 x 256 block, 128 x 64 per wave
    return Config{8, 1, 2, 2, 1, 6};                 // 64 x 512 block, 64 x 64 per wave
}

struct Plan {
    Config cfg;
    IgArgs a;
    size_t ws_bytes;
};

bool make_plan(const Geom &g, Plan *pl, std::string *why)
{
    auto no = [&](const char *m) {
        *why = m;
        return false;
    };
    const Config cfg = pick_config(g);
    const int BM = cfg.bm(), BN = cfg.bn();
    std::memset(&pl->a, 0, sizeof(pl->a));
    IgArgs &a = pl->a;
    for (int t = 0; t < kAxes; ++t) {
        if (g.s[t] > kMaxRes) return no("stride larger than 8");
        a.L[t] = int(g.L[t]);
        a.O[t] = int(g.O[t]);
        a.s[t] = int(g.s[t]);
        a.K[t] = int(g.K[t]);
        const int64_t gsd = std::__gcd(g.s[t], g.d[t]);
        a.kstep[t] = short(g.s[t] / gsd);
        a.bstep[t] = short(g.d[t] / gsd);
        if (g.K[t] > 32767 || g.d[t] / gsd > 32767) return no("kernel or dilation too large");
        for (int r = 0; r < g.s[t]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, t, r, &ph) || ph.ntaps > kMaxTap) return no("more than 8 taps per phase");
            a.ntap[t][r] = (signed char)ph.ntaps;
            a.tk0[t][r] = short(ph.ntaps ? ph.k[0] : 0);
            a.tb0[t][r] = short(ph.ntaps ? ph.beta[0] : 0);
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
    a.nchunk = int((g.Cg + kCC - 1) / kCC);
    a.Cgp = a.nchunk * kCC;
    a.mtiles = int((g.Mg + BM - 1) / BM);
    a.Mgp = a.mtiles * BM;

    // phases with outputs, heaviest (most taps) first
    struct PhaseInfo {
        int r[3], taps, blocks;
    };
    PhaseInfo list[kMaxPh];
    int nph = 0;
    for (int r0 = 0; r0 < g.s[0]; ++r0)
        for (int r1 = 0; r1 < g.s[1]; ++r1)
            for (int r2 = 0; r2 < g.s[2]; ++r2) {
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
                const int e2 = n2 ? (n2 - 1) * a.bstep[2] : 0;
                const int HR = seg ? 1 + e1 : std::min<int>(J1, (BN + J2 - 1) / J2 + 1) + e1;
                const int HC = seg ? BN + e2 : J2 + e2;
                if ((long long)HR * HC * kRow > kHaloBytes) return no("input halo exceeds LDS");
                if ((long long)HR * HC * 4 > (long long)cfg.nhwc_vecs * cfg.threads()) return no("halo too large");
                const int nvc = (HC + 7) / 8 + 1;
                if ((long long)HR * 4 * nvc > (long long)cfg.nch_items * cfg.threads()) return no("halo too large");
            }
    std::stable_sort(list, list + nph, [](const PhaseInfo &x, const PhaseInfo &y) { return x.taps > y.taps; });
    a.nphase = nph;
    long long total = 0;
    bool uniform = true;
    for (int i = 0; i < nph; ++i) {
        a.ph_start[i] = int(total);
        a.ph_r[i][0] = (unsigned char)list[i].r[0];
        a.ph_r[i][1] = (unsigned char)list[i].r[1];
        a.ph_r[i][2] = (unsigned char)list[i].r[2];
        total += list[i].blocks;
        uniform = uniform && list[i].blocks == list[0].blocks;
    }
    a.ph_start[nph] = int(total);
    if (total > INT32_MAX) return no("too many blocks");
    a.nblocks = int(total);
    a.interleave = uniform ? 1 : 0;
    pl->cfg = cfg;
    pl->ws_bytes = size_t(a.G) * a.T * a.Mgp * a.Cgp * sizeof(_Float16);
    return true;
}

template <bool CL, int WAVES, int WAVES_M, int WM, int WN, int NCH_ITEMS, int NHWC_VECS>
void launch_cfg(const IgArgs &a, const _Float16 *x, const _Float16 *wp, const _Float16 *b, _Float16 *y,
                hipStream_t st)
{
    hipLaunchKernelGGL((igemm_kernel<CL, WAVES, WAVES_M, WM, WN, NCH_ITEMS, NHWC_VECS>),
                       dim3(unsigned(a.nblocks)), dim3(WAVES * 64), 0, st, x, wp, b, y, a);
}

}  // namespace

bool igemm_supports(const Geom &g, ct_dtype dt, bool cl, const void *x, std::string *why)
{
    if (dt != CT_FLOAT16) {
        *why = "float16 only";
        return false;
    }
    if (g.Cg < 8 || g.Cg % 8 != 0) {
        *why = "C/group must be a multiple of 8";
        return false;
    }
    if (cl ? (g.C % 8 != 0) : (g.L[2] % 8 != 0)) {
        *why = cl ? "C must be a multiple of 8" : "innermost input size must be a multiple of 8";
        return false;
    }
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) {
        *why = "x must be 16-byte aligned";
        return false;
    }
    Plan pl;
    return make_plan(g, &pl, why);
}

size_t igemm_workspace_bytes(const Geom &g)
{
    Plan pl;
    std::string why;
    return make_plan(g, &pl, &why) ? pl.ws_bytes : 0;
}

ct_status launch_igemm(const Geom &g, ct_dtype, bool cl, const void *x, const void *w, const void *bias,
                       void *y, void *workspace, size_t ws_bytes, hipStream_t st, std::string *err)
{
    Plan pl;
    if (!make_plan(g, &pl, err)) return CT_EUNSUPPORTED;
    bool owned = false;
    void *wsp = workspace;
    if (!wsp) {
        hipError_t e = hipMallocAsync(&wsp, pl.ws_bytes, st);
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
    pa.total = (long long)pa.G * (pa.Cgp / 8) * pa.Mgp * pa.T;
    const _Float16 *wt = static_cast<const _Float16 *>(w);
    _Float16 *wpk = static_cast<_Float16 *>(wsp);
    hipLaunchKernelGGL(pack_w_kernel, dim3(unsigned((pa.total + 255) / 256)), dim3(256), 0, st, wt, wpk, pa);
    const _Float16 *xt = static_cast<const _Float16 *>(x);
    const _Float16 *bt = static_cast<const _Float16 *>(bias);
    _Float16 *yt = static_cast<_Float16 *>(y);
    const Config c = pl.cfg;
    mark_before(st);
    if (c.waves_m == 2) {
        if (cl) launch_cfg<true, 8, 2, 4, 2, 1, 6>(pl.a, xt, wpk, bt, yt, st);
        else launch_cfg<false, 8, 2, 4, 2, 1, 6>(pl.a, xt, wpk, bt, yt, st);
    } else {
        if (cl) launch_cfg<true, 8, 1, 2, 2, 1, 6>(pl.a, xt, wpk, bt, yt, st);
        else launch_cfg<false, 8, 1, 2, 2, 1, 6>(pl.a, xt, wpk, bt, yt, st);
    }
    mark_after(st);
    hipError_t e = hipGetLastError();
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

}  // namespace ct
