// Generic path: output-stationary gather over per-axis phase tables.
//
// One thread owns one output position (n, od, oh, ow) and CPT consecutive
// output channels of one group; it walks only the taps of its phase on each
// axis (residue r of o + p mod s; see convt_internal.h) and every input channel
// of the group, then applies the epilogue and stores each element once.  No
// atomics; every output element is written by exactly one thread.
// "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d, dilation 2): the
// thread-per-(b, oc, o) gather kernel that skips non-dividing taps; writes
// coalesce along the innermost axis because consecutive lanes take consecutive
// ow.  Any ndim (padded to 3 axes), groups, stride, padding, output padding and
// dilation within the table limits.
#include <hip/hip_runtime.h>

#include "convt_internal.h"
#include "epilogue.hpp"

namespace convt {
namespace {

constexpr int kBlock = 256;

struct GenericParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, k_vol;
    int in_sp, out_sp;
    int co_chunks;
    int n0; // first batch index of this launch
};

template <int CPT, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_generic(const GenericParams P,
                                                    const float *__restrict__ x,
                                                    const float *__restrict__ w,
                                                    const float *__restrict__ bias,
                                                    const float *add, float *y) {
    const int sp = blockIdx.x * kBlock + threadIdx.x;
    if (sp >= P.out_sp) return;
    const int g = blockIdx.y / P.co_chunks;
    const int co0 = (blockIdx.y % P.co_chunks) * CPT;
    const int n = P.n0 + blockIdx.z;

    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int ow = sp % AW.L_out;
    const int t2 = sp / AW.L_out;
    const int oh = t2 % AH.L_out;
    const int od = t2 / AH.L_out;

    const int td = od + AD.p, th = oh + AH.p, tw = ow + AW.p;
    const int rd = td % AD.s, qd = td / AD.s;
    const int rh = th % AH.s, qh = th / AH.s;
    const int rw = tw % AW.s, qw = tw / AW.s;

    float acc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = 0.0f;

    const float *xg = x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig) * P.in_sp;
    const float *wg = w + ((int64_t)g * P.Cig * P.Cog + co0) * P.k_vol;
    const int ncol = min(CPT, P.Cog - co0);

    for (int jd = AD.tap_start[rd]; jd < AD.tap_start[rd + 1]; ++jd) {
        const int id = qd - AD.tap_c[jd];
        if (id < 0 || id >= AD.L_in) continue;
        for (int jh = AH.tap_start[rh]; jh < AH.tap_start[rh + 1]; ++jh) {
            const int ih = qh - AH.tap_c[jh];
            if (ih < 0 || ih >= AH.L_in) continue;
            for (int jw = AW.tap_start[rw]; jw < AW.tap_start[rw + 1]; ++jw) {
                const int iw = qw - AW.tap_c[jw];
                if (iw < 0 || iw >= AW.L_in) continue;
                const int kidx = (AD.tap_k[jd] * AH.K + AH.tap_k[jh]) * AW.K + AW.tap_k[jw];
                const float *xp = xg + (id * AH.L_in + ih) * AW.L_in + iw;
                const float *wp = wg + kidx;
                for (int ci = 0; ci < P.Cig; ++ci) {
                    const float xv = xp[(int64_t)ci * P.in_sp];
                    const float *wc = wp + (int64_t)ci * P.Cog * P.k_vol;
#pragma unroll
                    for (int j = 0; j < CPT; ++j)
                        if (j < ncol) acc[j] = fmaf(xv, wc[j * P.k_vol], acc[j]);
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        if (j >= ncol) break;
        const int co = g * P.Cog + co0 + j;
        const int64_t idx = ((int64_t)n * P.C_out + co) * P.out_sp + sp;
        const float b = bias ? bias[co] : 0.0f;
        const float a = FUSED ? add[idx] : 0.0f;
        y[idx] = epilogue<FUSED>(acc[j], b, a);
    }
}

template <int CPT>
int launch_cpt(const convt_plan &Pl, const GenericParams &base, const float *x, const float *w,
               const float *bias, const float *add, float *y, hipStream_t st) {
    GenericParams P = base;
    P.co_chunks = (int)((Pl.Cog + CPT - 1) / CPT);
    const unsigned gx = (unsigned)((Pl.out_sp + kBlock - 1) / kBlock);
    const unsigned gy = (unsigned)(Pl.G * P.co_chunks);
    for (int64_t n0 = 0; n0 < Pl.N; n0 += 65535) {
        P.n0 = (int)n0;
        const unsigned gz = (unsigned)(Pl.N - n0 < 65535 ? Pl.N - n0 : 65535);
        dim3 grid(gx, gy, gz);
        if (add)
            hipLaunchKernelGGL((k_generic<CPT, true>), grid, dim3(kBlock), 0, st, P, x, w, bias,
                               add, y);
        else
            hipLaunchKernelGGL((k_generic<CPT, false>), grid, dim3(kBlock), 0, st, P, x, w, bias,
                               add, y);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

int pick_cpt(int64_t Cog) { return Cog >= 8 ? 8 : Cog >= 4 ? 4 : Cog >= 2 ? 2 : 1; }

} // namespace

bool generic_supports(const convt_plan &P) {
    const int cpt = pick_cpt(P.Cog);
    return P.G * ((P.Cog + cpt - 1) / cpt) <= 65535;
}

int launch_generic(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                   const float *add, float *y, void *stream) {
    GenericParams P;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.Cig = (int)Pl.Cig;
    P.Cog = (int)Pl.Cog;
    P.k_vol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    P.co_chunks = 1;
    P.n0 = 0;
    hipStream_t st = (hipStream_t)stream;
    switch (pick_cpt(Pl.Cog)) {
    case 8: return launch_cpt<8>(Pl, P, x, w, bias, add, y, st);
    case 4: return launch_cpt<4>(Pl, P, x, w, bias, add, y, st);
    case 2: return launch_cpt<2>(Pl, P, x, w, bias, add, y, st);
    default: return launch_cpt<1>(Pl, P, x, w, bias, add, y, st);
    }
}

} // namespace convt
