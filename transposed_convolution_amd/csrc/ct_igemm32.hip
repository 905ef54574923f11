// ct_igemm32.hip -- stride-phase implicit GEMM for float32 on MFMA (gfx950).
//
// The same decomposition as the float16 kernel (webgpu-kernels "ai.onnx.ConvTranspose"
// README, Implementation variants: the stride-phase route and the implicit-gather GEMM
// reducing over input channels x taps with direct output stores): output positions of
// one residue class modulo the stride on every axis ("phase") form a dense stride-1
// correlation with that phase's taps, i.e. a GEMM with rows = output channels, columns =
// the phase's output pixels (over all images) and depth = input channels x phase taps.
// No zero-inserted input or column matrix is formed: the depth slices of both operands
// are gathered straight into LDS.
//
// One block = 4 wave64s computing a 64 (output channels) x 64 (phase pixels) tile with
// v_mfma_f32_32x32x2_f32 (exact float32 products, float32 accumulation), 32 x 32 per wave.
// Depth advances 16 (channel, tap) pairs per step; the operands of the next step are
// gathered into registers while the current step's MFMAs run.  Any rank 1..3, stride,
// dilation, padding and group; channels-first or channels-last storage.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "ct_internal.hpp"

namespace ct {
namespace {

constexpr int kThreads32 = 256;
constexpr int kBM = 64, kBN = 64, kKC = 16;  // tile: channels x pixels x depth per step
constexpr int kRPT = kKC / 4;                 // depth rows gathered per thread and step
constexpr int kMaxRes32 = 16, kMaxTap32 = 16, kMaxPh32 = 64;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// the word padding slots of a gather read (outside the input, channels past C/group,
// output channels past M/group); a global-memory variable like x and w, so the selected
// pointer keeps the global address space (a constant-space one would turn the gathers
// into flat loads, which the compiler waits for one at a time).  Never written.
__device__ float kZero32 = 0.0f;

struct I32Args {
    int N, C, M, G, Cg, Mg, cl;
    int L[3], O[3], s[3], K[3];
    int mtiles, nphase;
    int ph_start[kMaxPh32 + 1];
    unsigned char ph_r[kMaxPh32][3];
    // per phase and axis: tap count, first tap and its input offset (the residue tables
    // below looked up once on the host), so the kernel reads them in one round
    signed char ph_nt[kMaxPh32][3];
    short ph_tk[kMaxPh32][3], ph_tb[kMaxPh32][3];
    // taps of residue r on axis a: k = tk0 + u * kstep, input offset beta = tb0 - u * bstep
    signed char ntap[3][kMaxRes32];
    short tk0[3][kMaxRes32], tb0[3][kMaxRes32];
    short kstep[3], bstep[3];
    Act act;  // output activation
};

// ALL = 0: depth streamed through two LDS buffers, one step ahead.  ALL > 0 (calls whose
// depth is at most ALL steps, e.g. 64 channels x 2 taps): every step's operands are
// gathered at once, staged once and reduced without further barriers, so the block waits
// for one round of loads instead of one per step.
// OFF: the element-offset type, 32-bit when X and W hold fewer than 2^30 elements (one
// 32-bit add per element and loads addressed from a scalar base), else 64-bit.
template <int ALL, typename OFF>
__global__ __launch_bounds__(kThreads32) void igemm32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                                             const float *__restrict__ bias, float *__restrict__ y,
                                                             I32Args p)
{
    constexpr int NBUF = ALL > 0 ? ALL : 2;
    __shared__ float As[NBUF][kKC][kBM + 4];  // [depth][channel]
    __shared__ float Bs[NBUF][kKC][kBN + 4];  // [depth][pixel]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // ---- work item: phase, pixel tile, channel tile, group ----
    const int v = blockIdx.x;
    // the phase: lane i compares the block against boundary i (one vector read of the
    // boundaries, no chain of dependent argument reads), the ballot counts the passed ones
    static_assert(kMaxPh32 <= 64, "one boundary per lane");
    const bool passed = lane >= 1 && lane < p.nphase && v >= p.ph_start[lane];
    const int ph = __builtin_amdgcn_readfirstlane(__builtin_popcountll(__ballot(passed)));
    int local = v - p.ph_start[ph];
    int r[3], J[3], nt[3];
    for (int a = 0; a < 3; ++a) {
        r[a] = p.ph_r[ph][a];
        J[a] = (p.O[a] - r[a] + p.s[a] - 1) / p.s[a];
        nt[a] = p.ph_nt[ph][a];
    }
    const int T = nt[0] * nt[1] * nt[2];
    const int P = p.N * J[0] * J[1] * J[2];
    const int ptiles = (P + kBN - 1) / kBN;
    const int pt = local % ptiles;
    local /= ptiles;
    const int mt = local % p.mtiles;
    const int g = local / p.mtiles;
    // depth order: tap-major, d = t * Cgp + c with Cgp = C/group rounded up to 16, so the
    // 16 depth rows of a step share one tap (wave-uniform) and hold consecutive channels
    const int Cgp = (p.Cg + kKC - 1) / kKC * kKC;
    const int depth = Cgp * T;
    const int Ktot = p.K[0] * p.K[1] * p.K[2];

    // ---- this thread's gather slots: one channel (A) and one pixel (B), kRPT depth rows ----
    const int col = tid % 64, row0 = tid / 64;  // depth rows row0 + 4 i
    const int m_a = mt * kBM + col;              // output channel inside the group
    int jn, jj[3];
    bool q_ok;
    {
        int q = pt * kBN + col;
        q_ok = q < P;
        if (!q_ok) q = 0;
        jj[2] = q % J[2];
        q /= J[2];
        jj[1] = q % J[1];
        q /= J[1];
        jj[0] = q % J[0];
        jn = q / J[0];
    }
    const OFF in_pix = OFF(p.L[0]) * p.L[1] * p.L[2];
    const bool m_ok = m_a < p.Mg;
    // element (channel c, tap) of this thread's operands: A at w + a_base + c * MgK + tap
    // offset, B at x + b_base + c * cstride + pixel offset of the tap
    const OFF MgK = OFF(p.Mg) * Ktot;
    const OFF a_base = OFF(g) * p.Cg * MgK + OFF(m_ok ? m_a : 0) * Ktot;
    const OFF cstride = p.cl ? 1 : in_pix;
    const OFF b_base = p.cl ? OFF(jn) * in_pix * p.C + OFF(g) * p.Cg : (OFF(jn) * p.C + OFF(g) * p.Cg) * in_pix;
    // Every load is issued unconditionally from a valid address: loads under a branch
    // are waited for one at a time.
    // the phase's tap progressions, read from the arguments once
    int tk[3], tb[3], ks[3], bs[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) {
        tk[a] = p.ph_tk[ph][a];
        tb[a] = jj[a] + p.ph_tb[ph][a];
        ks[a] = p.kstep[a];
        bs[a] = p.bstep[a];
    }
    auto gather = [&](int step, float (&areg)[kRPT], float (&breg)[kRPT]) {
        // the step's tap (uniform) and this thread's input pixel for it
        const int t = (step * kKC) / Cgp, cb = step * kKC - t * Cgp;
        const int t2 = t % nt[2], tq = t / nt[2];
        const int t1 = tq % nt[1], t0 = tq / nt[1];
        const int k0 = tk[0] + t0 * ks[0], k1 = tk[1] + t1 * ks[1], k2 = tk[2] + t2 * ks[2];
        const int tapoff = (k0 * p.K[1] + k1) * p.K[2] + k2;
        const int i0 = tb[0] - t0 * bs[0];
        const int i1 = tb[1] - t1 * bs[1];
        const int i2 = tb[2] - t2 * bs[2];
        const bool pin = q_ok && i0 >= 0 && i0 < p.L[0] && i1 >= 0 && i1 < p.L[1] && i2 >= 0 && i2 < p.L[2];
        const OFF pix = pin ? (OFF(i0) * p.L[1] + i1) * p.L[2] + i2 : 0;
        const OFF pixoff = p.cl ? pix * p.C : pix;
        // running offsets of channel cb + row0 + 4 i (one add per element); a padding slot
        // reads the zero word instead, so no select waits for the loaded value and every
        // load of the step (of all steps, in the one-round instance) stays in flight
        OFF ao = a_base + OFF(cb + row0) * MgK + tapoff;
        OFF bo = b_base + OFF(cb + row0) * cstride + pixoff;
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
            const bool cok = cb + row0 + 4 * i < p.Cg;
            areg[i] = *((cok && m_ok) ? w + ao : &kZero32);
            breg[i] = *((cok && pin) ? x + bo : &kZero32);
            ao += 4 * MgK;
            bo += 4 * cstride;
        }
    };
    auto stage = [&](int buf, const float (&areg)[kRPT], const float (&breg)[kRPT]) {
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
            As[buf][row0 + 4 * i][col] = areg[i];
            Bs[buf][row0 + 4 * i][col] = breg[i];
        }
    };
    auto mma_step = [&](int buf, f32x16 &acc) {
#pragma unroll
        for (int k = 0; k < kKC; k += 2) {
            const float a = As[buf][k + (lane >> 5)][wm * 32 + (lane & 31)];
            const float b = Bs[buf][k + (lane >> 5)][wn * 32 + (lane & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
    };

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    const int nsteps = (depth + kKC - 1) / kKC;
    if constexpr (ALL > 0) {
        float ar[ALL][kRPT], br[ALL][kRPT];
#pragma unroll
        for (int st = 0; st < ALL; ++st)
            if (st < nsteps) gather(st, ar[st], br[st]);
#pragma unroll
        for (int st = 0; st < ALL; ++st)
            if (st < nsteps) stage(st, ar[st], br[st]);
        __syncthreads();
#pragma unroll
        for (int st = 0; st < ALL; ++st)
            if (st < nsteps) mma_step(st, acc);
    } else if (nsteps > 0) {
        float areg[kRPT], breg[kRPT];
        gather(0, areg, breg);
        stage(0, areg, breg);
        __syncthreads();
        for (int st = 0; st < nsteps; ++st) {
            const int buf = st & 1;
            if (st + 1 < nsteps) gather(st + 1, areg, breg);  // next step's operands, in flight under the MFMAs
            mma_step(buf, acc);
            if (st + 1 < nsteps) stage(buf ^ 1, areg, breg);
            __syncthreads();
        }
    }

    // ---- epilogue: bias, store (result row = channel, column = pixel) ----
    int q = pt * kBN + wn * 32 + (lane & 31);
    if (q >= P) return;
    int o[3];
    o[2] = r[2] + p.s[2] * (q % J[2]);
    q /= J[2];
    o[1] = r[1] + p.s[1] * (q % J[1]);
    q /= J[1];
    o[0] = r[0] + p.s[0] * (q % J[0]);
    const int n = q / J[0];
    const size_t opix = size_t(p.O[0]) * p.O[1] * p.O[2];
    const size_t pix = (size_t(o[0]) * p.O[1] + o[1]) * p.O[2] + o[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int ml = mt * kBM + wm * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (ml >= p.Mg) continue;
        const int m = g * p.Mg + ml;
        const float val = p.act(acc[e] + (bias ? bias[m] : 0.0f));
        if (p.cl) y[(size_t(n) * opix + pix) * p.M + m] = val;
        else y[(size_t(n) * p.M + m) * opix + pix] = val;
    }
}

bool make_plan32(const Geom &g, bool cl, I32Args *a, int *blocks, std::string *why)
{
    std::memset(a, 0, sizeof(*a));
    a->N = int(g.N);
    a->C = int(g.C);
    a->M = int(g.M);
    a->G = int(g.G);
    a->Cg = int(g.Cg);
    a->Mg = int(g.Mg);
    a->cl = cl ? 1 : 0;
    for (int t = 0; t < kAxes; ++t) {
        if (g.s[t] > kMaxRes32) {
            *why = "stride larger than 16";
            return false;
        }
        a->L[t] = int(g.L[t]);
        a->O[t] = int(g.O[t]);
        a->s[t] = int(g.s[t]);
        a->K[t] = int(g.K[t]);
        const int64_t gsd = std::__gcd(g.s[t], g.d[t]);
        a->kstep[t] = short(g.s[t] / gsd);
        a->bstep[t] = short(g.d[t] / gsd);
        for (int r = 0; r < g.s[t]; ++r) {
            AxisPhase ph;
            if (!axis_phase(g, t, r, &ph) || ph.ntaps > kMaxTap32) {
                *why = "more than 16 taps per phase";
                return false;
            }
            a->ntap[t][r] = (signed char)ph.ntaps;
            a->tk0[t][r] = short(ph.ntaps ? ph.k[0] : 0);
            a->tb0[t][r] = short(ph.ntaps ? ph.beta[0] : 0);
            for (int k = 0; k < ph.ntaps; ++k)
                if (ph.k[k] != ph.k[0] + k * a->kstep[t] || ph.beta[k] != ph.beta[0] - k * a->bstep[t]) {
                    *why = "internal: taps are not an arithmetic progression";
                    return false;
                }
        }
    }
    if (g.K[0] > 32767 || g.K[1] > 32767 || g.K[2] > 32767) {
        *why = "kernel too large";
        return false;
    }
    // depth (C/group rounded up to 16, times the phase's taps) in an int
    if ((g.Cg + kKC) * g.taps() > INT32_MAX) {
        *why = "C/group x taps too large";
        return false;
    }
    a->mtiles = int((g.Mg + kBM - 1) / kBM);
    int64_t total = 0;
    int nph = 0;
    for (int r0 = 0; r0 < g.s[0]; ++r0)
        for (int r1 = 0; r1 < g.s[1]; ++r1)
            for (int r2 = 0; r2 < g.s[2]; ++r2) {
                if (r0 >= g.O[0] || r1 >= g.O[1] || r2 >= g.O[2]) continue;
                if (nph == kMaxPh32) {
                    *why = "more than 64 phases";
                    return false;
                }
                const int64_t J0 = (g.O[0] - r0 + g.s[0] - 1) / g.s[0], J1 = (g.O[1] - r1 + g.s[1] - 1) / g.s[1],
                              J2 = (g.O[2] - r2 + g.s[2] - 1) / g.s[2];
                const int64_t P = g.N * J0 * J1 * J2;
                if (P > INT32_MAX) {
                    *why = "too many pixels";
                    return false;
                }
                a->ph_start[nph] = int(total);
                a->ph_r[nph][0] = (unsigned char)r0;
                a->ph_r[nph][1] = (unsigned char)r1;
                a->ph_r[nph][2] = (unsigned char)r2;
                const int rr[3] = {r0, r1, r2};
                for (int ax = 0; ax < 3; ++ax) {
                    a->ph_nt[nph][ax] = a->ntap[ax][rr[ax]];
                    a->ph_tk[nph][ax] = a->tk0[ax][rr[ax]];
                    a->ph_tb[nph][ax] = a->tb0[ax][rr[ax]];
                }
                total += (P + kBN - 1) / kBN * a->mtiles * g.G;
                ++nph;
            }
    if (total > INT32_MAX) {
        *why = "too many blocks";
        return false;
    }
    a->nphase = nph;
    a->ph_start[nph] = int(total);
    *blocks = int(total);
    return true;
}

}  // namespace

bool igemm32_supports(const Geom &g, bool cl, std::string *why)
{
    // the gathers load element 0 of x and w for masked slots: both must be non-empty
    if (g.x_elems() <= 0 || g.w_elems() <= 0) {
        *why = "empty input or weights";
        return false;
    }
    I32Args a;
    int blocks = 0;
    return make_plan32(g, cl, &a, &blocks, why);
}

ct_status launch_igemm32(const Geom &g, bool cl, const void *x, const void *w, const void *bias, void *y,
                         const Act &act, hipStream_t st, std::string *err)
{
    I32Args a;
    int blocks = 0;
    if (!make_plan32(g, cl, &a, &blocks, err)) return CT_EUNSUPPORTED;
    a.act = act;
    mark_before(st);
    // deepest phase: C/group (rounded up to 16) x its taps; at most 8 steps -> the one-round instance
    int64_t max_depth = 0;
    for (int ph = 0; ph < a.nphase; ++ph)
        max_depth = std::max<int64_t>(max_depth, int64_t((a.Cg + kKC - 1) / kKC * kKC) * a.ntap[0][a.ph_r[ph][0]] *
                                                     a.ntap[1][a.ph_r[ph][1]] * a.ntap[2][a.ph_r[ph][2]]);
    // 32-bit element offsets when every offset stays below 2^30 elements
    const bool off32 = g.x_elems() < (int64_t(1) << 30) && g.w_elems() < (int64_t(1) << 30);
    const auto *xf = static_cast<const float *>(x);
    const auto *wf = static_cast<const float *>(w);
    const auto *bf = static_cast<const float *>(bias);
    auto *yf = static_cast<float *>(y);
    if (blocks > 0) {
        const dim3 grid = dim3(unsigned(blocks)), block = dim3(kThreads32);
        if (max_depth <= 8 * kKC && off32)
            hipLaunchKernelGGL((igemm32_kernel<8, unsigned>), grid, block, 0, st, xf, wf, bf, yf, a);
        else if (max_depth <= 8 * kKC)
            hipLaunchKernelGGL((igemm32_kernel<8, size_t>), grid, block, 0, st, xf, wf, bf, yf, a);
        else if (off32)
            hipLaunchKernelGGL((igemm32_kernel<0, unsigned>), grid, block, 0, st, xf, wf, bf, yf, a);
        else
            hipLaunchKernelGGL((igemm32_kernel<0, size_t>), grid, block, 0, st, xf, wf, bf, yf, a);
    }
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("float32 implicit-GEMM launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
