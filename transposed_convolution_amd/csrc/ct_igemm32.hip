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
constexpr int kMaxRes32 = 16, kMaxTap32 = 16, kMaxPh32 = 64;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct I32Args {
    int N, C, M, G, Cg, Mg, cl;
    int L[3], O[3], s[3], K[3];
    int mtiles, nphase;
    int ph_start[kMaxPh32 + 1];
    unsigned char ph_r[kMaxPh32][3];
    // taps of residue r on axis a: k = tk0 + u * kstep, input offset beta = tb0 - u * bstep
    signed char ntap[3][kMaxRes32];
    short tk0[3][kMaxRes32], tb0[3][kMaxRes32];
    short kstep[3], bstep[3];
    Act act;  // output activation
};

__global__ __launch_bounds__(kThreads32) void igemm32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                                                             const float *__restrict__ bias, float *__restrict__ y,
                                                             I32Args p)
{
    __shared__ float As[2][kKC][kBM + 4];  // [depth][channel]
    __shared__ float Bs[2][kKC][kBN + 4];  // [depth][pixel]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // ---- work item: phase, pixel tile, channel tile, group ----
    const int v = blockIdx.x;
    int ph = 0;
    while (v >= p.ph_start[ph + 1]) ++ph;
    int local = v - p.ph_start[ph];
    int r[3], J[3], nt[3];
    for (int a = 0; a < 3; ++a) {
        r[a] = p.ph_r[ph][a];
        J[a] = (p.O[a] - r[a] + p.s[a] - 1) / p.s[a];
        nt[a] = p.ntap[a][r[a]];
    }
    const int T = nt[0] * nt[1] * nt[2];
    const int P = p.N * J[0] * J[1] * J[2];
    const int ptiles = (P + kBN - 1) / kBN;
    const int pt = local % ptiles;
    local /= ptiles;
    const int mt = local % p.mtiles;
    const int g = local / p.mtiles;
    const int depth = p.Cg * T;
    const int Ktot = p.K[0] * p.K[1] * p.K[2];

    // ---- this thread's gather slots: one channel (A) and one pixel (B), 4 depth rows ----
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
    const size_t in_pix = size_t(p.L[0]) * p.L[1] * p.L[2];

    float areg[4], breg[4];
    auto gather = [&](int step) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = step * kKC + row0 + 4 * i;
            float av = 0.0f, bv = 0.0f;
            if (d < depth) {
                const int c = d / T;
                int t = d - c * T;
                const int t2 = t % nt[2];
                t /= nt[2];
                const int t1 = t % nt[1];
                const int t0 = t / nt[1];
                const int k0 = p.tk0[0][r[0]] + t0 * p.kstep[0], k1 = p.tk0[1][r[1]] + t1 * p.kstep[1],
                          k2 = p.tk0[2][r[2]] + t2 * p.kstep[2];
                const int gc = g * p.Cg + c;
                if (m_a < p.Mg) av = w[(size_t(gc) * p.Mg + m_a) * Ktot + (k0 * p.K[1] + k1) * p.K[2] + k2];
                const int i0 = jj[0] + p.tb0[0][r[0]] - t0 * p.bstep[0];
                const int i1 = jj[1] + p.tb0[1][r[1]] - t1 * p.bstep[1];
                const int i2 = jj[2] + p.tb0[2][r[2]] - t2 * p.bstep[2];
                if (q_ok && i0 >= 0 && i0 < p.L[0] && i1 >= 0 && i1 < p.L[1] && i2 >= 0 && i2 < p.L[2]) {
                    const size_t pix = (size_t(i0) * p.L[1] + i1) * p.L[2] + i2;
                    bv = p.cl ? x[(size_t(jn) * in_pix + pix) * p.C + gc] : x[(size_t(jn) * p.C + gc) * in_pix + pix];
                }
            }
            areg[i] = av;
            breg[i] = bv;
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            As[buf][row0 + 4 * i][col] = areg[i];
            Bs[buf][row0 + 4 * i][col] = breg[i];
        }
    };

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    const int nsteps = (depth + kKC - 1) / kKC;
    if (nsteps > 0) {
        gather(0);
        stage(0);
        __syncthreads();
        for (int st = 0; st < nsteps; ++st) {
            const int buf = st & 1;
            if (st + 1 < nsteps) gather(st + 1);  // next step's operands, in flight under the MFMAs
#pragma unroll
            for (int k = 0; k < kKC; k += 2) {
                const float a = As[buf][k + (lane >> 5)][wm * 32 + (lane & 31)];
                const float b = Bs[buf][k + (lane >> 5)][wn * 32 + (lane & 31)];
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
            }
            if (st + 1 < nsteps) stage(buf ^ 1);
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
    if (blocks > 0)
        hipLaunchKernelGGL(igemm32_kernel, dim3(unsigned(blocks)), dim3(kThreads32), 0, st,
                           static_cast<const float *>(x), static_cast<const float *>(w),
                           static_cast<const float *>(bias), static_cast<float *>(y), a);
    mark_after(st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        *err = std::string("float32 implicit-GEMM launch failed: ") + hipGetErrorString(e);
        return CT_EDEVICE;
    }
    return CT_OK;
}

}  // namespace ct
