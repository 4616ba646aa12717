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

// ------------------------------------------------------- phase-class variant
// Same gather, but a workgroup covers output positions of one phase class
// (one residue per axis) only, consecutive lanes taking consecutive positions q
// along W.  All lanes of a wave then walk the same tap list, the weights they
// use are the same for the whole wave (scalar loads, broadcast), and each
// input load, coalesced along W, feeds CPT FMAs.  P1's parity-class blocking
// ("Kimi-K2.6 l1_p72" transcript, ConvTranspose3d): a block never mixes
// classes, so trip counts stay uniform.
constexpr int kMaxPhaseCls = 32;
#ifndef CONVT_GEN_POS
#define CONVT_GEN_POS 2
#endif
constexpr int kPhasePos = CONVT_GEN_POS; // positions per thread

int pick_cpt(int64_t Cog) { return Cog >= 8 ? 8 : Cog >= 4 ? 4 : Cog >= 2 ? 2 : 1; }

struct PhaseParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, k_vol;
    int in_sp, out_sp;
    int co_chunks;
    int n0;
    int n_cls;
    int cls_r[kMaxPhaseCls][kAxes];  // residue per axis
    int cls_q0[kMaxPhaseCls][kAxes]; // first q per axis (its output lies in [0, L_out))
    int cls_nq[kMaxPhaseCls][kAxes]; // number of q per axis
    int cls_blk0[kMaxPhaseCls + 1];  // first workgroup (grid x) of each class
    int max_taps;                    // taps of the class with the most
    int tap_stride;                  // staged floats per tap (see tap_stride())
};
constexpr int kMaxPhaseLds = 32768; // bytes of staged weights per workgroup

template <int CPT, int NPOS, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_generic_phase(const PhaseParams P,
                                                          const float *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ bias,
                                                          const float *add, float *y) {
    // Each thread computes NPOS positions of the class, kBlock apart (so each
    // of its loads still coalesces with the neighbouring lanes'), sharing
    // every weight read among NPOS*CPT FMAs.
    int c = 0;
    while (c + 1 < P.n_cls && (int)blockIdx.x >= P.cls_blk0[c + 1]) ++c;
    const int nqd = P.cls_nq[c][0], nqh = P.cls_nq[c][1], nqw = P.cls_nq[c][2];
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int rd = P.cls_r[c][0], rh = P.cls_r[c][1], rw = P.cls_r[c][2];
    bool live[NPOS];
    int qd[NPOS], qh[NPOS], qw[NPOS];
#pragma unroll
    for (int u = 0; u < NPOS; ++u) {
        const int l = ((int)blockIdx.x - P.cls_blk0[c]) * (kBlock * NPOS) + u * kBlock + (int)threadIdx.x;
        live[u] = l < nqd * nqh * nqw;
        const int iqw = l % nqw;
        const int t2 = l / nqw;
        const int iqh = t2 % nqh;
        const int iqd = t2 / nqh;
        qd[u] = P.cls_q0[c][0] + iqd;
        qh[u] = P.cls_q0[c][1] + iqh;
        qw[u] = P.cls_q0[c][2] + iqw;
    }

    const int g = blockIdx.y / P.co_chunks;
    const int co0 = (blockIdx.y % P.co_chunks) * CPT;
    const int n = P.n0 + blockIdx.z;
    const int ncol = min(CPT, P.Cog - co0);

    float acc[NPOS][CPT];
#pragma unroll
    for (int u = 0; u < NPOS; ++u)
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[u][j] = 0.0f;

    // The workgroup's weights, [class tap][input channel][column], staged once:
    // every lane reads the same ones, so the reads below are broadcasts.
    // Columns past the group's last channel repeat it (never stored).
    extern __shared__ __attribute__((aligned(16))) float wl[];
    const int Td = AD.tap_start[rd + 1] - AD.tap_start[rd];
    const int Th = AH.tap_start[rh + 1] - AH.tap_start[rh];
    const int Tw = AW.tap_start[rw + 1] - AW.tap_start[rw];
    {
        const float *wg = w + ((int64_t)g * P.Cig * P.Cog + co0) * P.k_vol;
        const int nw = Td * Th * Tw * P.Cig * CPT;
        for (int i = threadIdx.x; i < nw; i += kBlock) {
            const int j = i % CPT, t = i / CPT;
            const int ci = t % P.Cig, tap = t / P.Cig;
            const int tw = tap % Tw, tdh = tap / Tw;
            const int th = tdh % Th, td = tdh / Th;
            const int kidx = (AD.tap_k[AD.tap_start[rd] + td] * AH.K + AH.tap_k[AH.tap_start[rh] + th]) *
                                 AW.K + AW.tap_k[AW.tap_start[rw] + tw];
            wl[i] = wg[((int64_t)ci * P.Cog + min(j, ncol - 1)) * P.k_vol + kidx];
        }
    }
    __syncthreads();

    const float *xg = x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig) * P.in_sp;
    const float *wt = wl;
    for (int jd = AD.tap_start[rd]; jd < AD.tap_start[rd + 1]; ++jd) {
        for (int jh = AH.tap_start[rh]; jh < AH.tap_start[rh + 1]; ++jh) {
            for (int jw = AW.tap_start[rw]; jw < AW.tap_start[rw + 1]; ++jw, wt += P.Cig * CPT) {
                bool ok[NPOS];
                const float *xp[NPOS];
#pragma unroll
                for (int u = 0; u < NPOS; ++u) {
                    const int id = qd[u] - AD.tap_c[jd], ih = qh[u] - AH.tap_c[jh], iw = qw[u] - AW.tap_c[jw];
                    ok[u] = live[u] && id >= 0 && id < AD.L_in && ih >= 0 && ih < AH.L_in && iw >= 0 &&
                            iw < AW.L_in;
                    // lanes outside the input read the group's first element and use 0
                    xp[u] = xg + (ok[u] ? (id * AH.L_in + ih) * AW.L_in + iw : 0);
                }
#pragma unroll 4
                for (int ci = 0; ci < P.Cig; ++ci) {
                    float xv[NPOS];
#pragma unroll
                    for (int u = 0; u < NPOS; ++u) {
                        const float xr = xp[u][(int64_t)ci * P.in_sp];
                        xv[u] = ok[u] ? xr : 0.0f;
                    }
                    const float *wc = wt + ci * CPT;
#pragma unroll
                    for (int j = 0; j < CPT; ++j) {
                        const float wv = wc[j];
#pragma unroll
                        for (int u = 0; u < NPOS; ++u) acc[u][j] = fmaf(xv[u], wv, acc[u][j]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int u = 0; u < NPOS; ++u) {
        if (!live[u]) continue;
        const int od = qd[u] * AD.s + rd - AD.p, oh = qh[u] * AH.s + rh - AH.p, ow = qw[u] * AW.s + rw - AW.p;
        const int sp = (od * AH.L_out + oh) * AW.L_out + ow;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if (j >= ncol) break;
            const int co = g * P.Cog + co0 + j;
            const int64_t idx = ((int64_t)n * P.C_out + co) * P.out_sp + sp;
            const float b = bias ? bias[co] : 0.0f;
            const float a = FUSED ? add[idx] : 0.0f;
            y[idx] = epilogue<FUSED>(acc[u][j], b, a);
        }
    }
}

// Same gather with the channel contraction on the matrix cores and input rows
// shared along H, for CPT = 4 or 8.
//
// v_mfma_f32_4x4x1f32 runs 16 independent 4x4x1 outer products per wave:
// lane 4b+j supplies column j of block b's B and receives row i of block b's
// result in accumulator register i.  With the A operand broadcast from one
// block (CBSZ = 4, ABID = that block) every block multiplies the same four
// weights w[ci][co0+4h .. co0+4h+3] by its lanes' inputs, so each lane keeps
// the output of its own position for four channels: one instruction per input
// channel and 4-channel block instead of four FMAs.  One broadcast register
// holds the weights of 64/CPT input channels (16 blocks of 4): lane l of the
// staged row [ci0..ci0+64/CPT)[0..CPT) is block l/4, row l%4.
//
// A thread owns one (qd, qw) of its class and R consecutive q along H.  When
// the H taps of every residue have the offsets c = 0, 1, .., T-1 (dilation 1
// on H gives exactly that), output row qh0 + r takes tap j from input row
// qh0 + r - j, so the R + TH - 1 input rows qh0 - TH + 1 .. qh0 + R - 1 feed
// all R x T (row, tap) pairs: each input value loaded serves up to
// min(R, T) MFMAs per 4-channel block.
typedef float v4f __attribute__((ext_vector_type(4)));

template <int ABID>
__device__ __forceinline__ v4f mfma4_bcast(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 4, ABID, 0);
}

// Input loads through a buffer resource over the group's channels of one
// sample: a load past num_records returns zero, so a lane outside the input
// takes an out-of-range offset instead of a select; the channel goes in the
// scalar offset, so all channels of a row share one offset register.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000; // raw (untyped) buffer access
constexpr unsigned kOutOfRange = 0x80000000u;

// One window row (u = ih - (qh0 - TH + 1)), channels ci0 + CL: one MFMA per
// (output row r whose tap j = r + TH-1-U exists, 4-channel block h).  The
// block index is an instruction immediate, hence the compile-time recursion.
template <int CL, int CH, int H, int R, int TH, int U>
__device__ __forceinline__ void rows_channels(const float (&wa)[TH], const float (&xv)[CH],
                                              v4f (&acc)[R][H]) {
    if constexpr (CL < CH) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = r + TH - 1 - U;
            if (j < 0 || j >= TH) continue;
            acc[r][0] = mfma4_bcast<CL * H>(wa[j], xv[CL], acc[r][0]);
            if constexpr (H > 1) acc[r][1] = mfma4_bcast<CL * H + 1>(wa[j], xv[CL], acc[r][1]);
        }
        rows_channels<CL + 1, CH, H, R, TH, U>(wa, xv, acc);
    }
}

// Window rows U .. R + TH - 2 for the channel chunk at scalar byte offset soff
// (nci of its CH channels exist; all of them when FULLCH).
template <int U, int CH, int H, int R, int TH, bool FULLCH>
__device__ __forceinline__ void rows_window(const float (&wa)[TH], rsrc_t rx, unsigned voff_dw,
                                            bool okdw, int ih0, int L_inH, int L_inW, unsigned soff,
                                            unsigned ch_bytes, int nci, v4f (&acc)[R][H]) {
    if constexpr (U < R + TH - 1) {
        const int ih = ih0 + U;
        const bool ok = okdw && ih >= 0 && ih < L_inH;
        const unsigned vo = ok ? 4u * (voff_dw + (unsigned)(ih * L_inW)) : kOutOfRange;
        float xv[CH];
#pragma unroll
        for (int cl = 0; cl < CH; ++cl) {
            if (!FULLCH && cl >= nci) {
                xv[cl] = 0.0f;
                continue;
            }
            xv[cl] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vo, soff + cl * ch_bytes, 0));
        }
        rows_channels<0, CH, H, R, TH, U>(wa, xv, acc);
        rows_window<U + 1, CH, H, R, TH, FULLCH>(wa, rx, voff_dw, okdw, ih0, L_inH, L_inW, soff, ch_bytes,
                                                 nci, acc);
    }
}

// Every class of a launch has exactly TH taps on H (or none on some axis: then
// it only takes the bias).  FULLCH: Cig is a multiple of the channel chunk.
template <int CPT, int R, int TH, bool FULLCH, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_generic_rows(const PhaseParams P,
                                                         const float *__restrict__ x,
                                                         const float *__restrict__ w,
                                                         const float *__restrict__ bias,
                                                         const float *add, float *y) {
    static_assert(CPT == 4 || CPT == 8, "one or two 4-channel blocks");
    constexpr int H = CPT / 4;  // 4-channel blocks per thread
    constexpr int CH = 16 / H;  // input channels per broadcast register (CH * CPT = 64)
    int c = 0;
    while (c + 1 < P.n_cls && (int)blockIdx.x >= P.cls_blk0[c + 1]) ++c;
    const int nqd = P.cls_nq[c][0], nqh = P.cls_nq[c][1], nqw = P.cls_nq[c][2];
    const int nqhb = (nqh + R - 1) / R;
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int rd = P.cls_r[c][0], rh = P.cls_r[c][1], rw = P.cls_r[c][2];
    const int l = ((int)blockIdx.x - P.cls_blk0[c]) * kBlock + (int)threadIdx.x;
    const bool live = l < nqd * nqhb * nqw;
    const int iqw = l % nqw;
    const int t2 = l / nqw;
    const int iqhb = t2 % nqhb;
    const int iqd = t2 / nqhb;
    const int qd = P.cls_q0[c][0] + iqd;
    const int qh0 = P.cls_q0[c][1] + iqhb * R;
    const int qw = P.cls_q0[c][2] + iqw;

    const int g = blockIdx.y / P.co_chunks;
    const int co0 = (blockIdx.y % P.co_chunks) * CPT;
    const int n = P.n0 + blockIdx.z;
    const int ncol = min(CPT, P.Cog - co0);

    v4f acc[R][H];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int h = 0; h < H; ++h) acc[r][h] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int Td = AD.tap_start[rd + 1] - AD.tap_start[rd];
    const int Th = AH.tap_start[rh + 1] - AH.tap_start[rh];
    const int Tw = AW.tap_start[rw + 1] - AW.tap_start[rw];
    if (Td * Th * Tw > 0) {
        // Staged weights, [class tap (d, h, w)][input channel][column] with
        // each tap's rows padded with zeros to tap_stride (a multiple of 64)
        // floats; columns past the group's last channel repeat it (never
        // stored).  Th == TH here.
        extern __shared__ __attribute__((aligned(16))) float wl[];
        const int TS = P.tap_stride;
        {
            const float *wg = w + ((int64_t)g * P.Cig * P.Cog + co0) * P.k_vol;
            const int nw = Td * TH * Tw * TS;
            for (int i = threadIdx.x; i < nw; i += kBlock) {
                const int tap = i / TS, rem = i % TS;
                const int j = rem % CPT, ci = rem / CPT;
                float v = 0.0f;
                if (ci < P.Cig) {
                    const int tw = tap % Tw, tdh = tap / Tw;
                    const int th = tdh % TH, td = tdh / TH;
                    const int kidx = (AD.tap_k[AD.tap_start[rd] + td] * AH.K + AH.tap_k[AH.tap_start[rh] + th]) *
                                         AW.K + AW.tap_k[AW.tap_start[rw] + tw];
                    v = wg[((int64_t)ci * P.Cog + min(j, ncol - 1)) * P.k_vol + kidx];
                }
                wl[i] = v;
            }
        }
        __syncthreads();

        const int lane = threadIdx.x & 63;
        const rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig) * P.in_sp), (short)0,
            (int)(4 * P.Cig * P.in_sp), kRsrcWord3);
        const unsigned ch_bytes = 4u * (unsigned)P.in_sp;
        const int ih0 = qh0 - (TH - 1);
        for (int td = 0; td < Td; ++td) {
            const int id = qd - AD.tap_c[AD.tap_start[rd] + td];
            const bool okd = live && id >= 0 && id < AD.L_in;
            for (int tw = 0; tw < Tw; ++tw) {
                const int iw = qw - AW.tap_c[AW.tap_start[rw] + tw];
                const bool okdw = okd && iw >= 0 && iw < AW.L_in;
                const unsigned voff_dw = okdw ? (unsigned)(id * AH.L_in * AW.L_in + iw) : 0u;
                for (int ci0 = 0; ci0 < P.Cig; ci0 += CH) {
                    // the class's H taps of this (d, w) tap pair, channels
                    // ci0..; ci0 * CPT is a multiple of 64 below Cig * CPT <= TS
                    float wa[TH];
#pragma unroll
                    for (int j = 0; j < TH; ++j) wa[j] = wl[((td * TH + j) * Tw + tw) * TS + ci0 * CPT + lane];
                    rows_window<0, CH, H, R, TH, FULLCH>(wa, rx, voff_dw, okdw, ih0, AH.L_in, AW.L_in,
                                                         (unsigned)ci0 * ch_bytes, ch_bytes, P.Cig - ci0, acc);
                }
            }
        }
    }

    if (!live) return;
    const int od = qd * AD.s + rd - AD.p, ow = qw * AW.s + rw - AW.p;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (iqhb * R + r >= nqh) break;
        const int oh = (qh0 + r) * AH.s + rh - AH.p;
        const int sp = (od * AH.L_out + oh) * AW.L_out + ow;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if (j >= ncol) break;
            const int co = g * P.Cog + co0 + j;
            const int64_t idx = ((int64_t)n * P.C_out + co) * P.out_sp + sp;
            const float b = bias ? bias[co] : 0.0f;
            const float a = FUSED ? add[idx] : 0.0f;
            y[idx] = epilogue<FUSED>(acc[r][j / 4][j % 4], b, a);
        }
    }
}

constexpr int kRows = 4;     // H rows per thread in k_generic_rows
constexpr int kRowsMaxTH = 5; // largest H tap count instantiated

// Largest H tap count of the shape if k_generic_rows applies, else 0: 4-channel
// blocks, a group's input below 2 GiB, at least kRows outputs along H, and on H
// every residue's taps at offsets 0, 1, .., T-1.
int rows_th(const convt_plan &Pl) {
    if (pick_cpt(Pl.Cog) < 4) return 0;
    if (4 * Pl.Cig * Pl.in_sp > 0x7fffffff) return 0; // byte offsets in the buffer resource
    const AxisPlan &A = Pl.ax[1];
    if (A.L_out < kRows) return 0; // nothing to share along H (1D shapes)
    int th = 1;
    for (int r = 0; r < A.s; ++r) {
        const int T = A.tap_start[r + 1] - A.tap_start[r];
        for (int j = 0; j < T; ++j)
            if (A.tap_c[A.tap_start[r] + j] != j) return 0;
        th = T > th ? T : th;
    }
    return th <= kRowsMaxTH ? th : 0;
}

// Floats per staged tap: the FMA kernel packs Cig*CPT; the matrix kernel pads
// to whole 64-float broadcast registers.
int tap_stride(int64_t Cig, int cpt, bool rows) {
    const int64_t n = Cig * cpt;
    return (int)(rows ? (n + 63) / 64 * 64 : n);
}

// Fills the class table; false when the shape has more classes than it holds.
// rows > 0 lays the class out for k_generic_rows (rows q along H per thread),
// else for k_generic_phase (kPhasePos positions per thread).
// th_only > 0 keeps only the classes whose launch key (below) is th_only.
int rows_key(const AxisPlan *A, const int r[kAxes]) {
    int taps = 1;
    for (int a = 0; a < kAxes; ++a) taps *= A[a].tap_start[r[a] + 1] - A[a].tap_start[r[a]];
    // bias-only classes go with the 1-tap launch, which skips their contraction
    return taps == 0 ? 1 : A[1].tap_start[r[1] + 1] - A[1].tap_start[r[1]];
}

bool phase_classes(const convt_plan &Pl, PhaseParams &P, int rows, int th_only = 0) {
    P.n_cls = 0;
    P.max_taps = 1;
    int blocks = 0;
    const AxisPlan *A = Pl.ax;
    for (int rd = 0; rd < A[0].s; ++rd)
        for (int rh = 0; rh < A[1].s; ++rh)
            for (int rw = 0; rw < A[2].s; ++rw) {
                const int r[kAxes] = {rd, rh, rw};
                int q0[kAxes], nq[kAxes];
                bool empty = false;
                for (int a = 0; a < kAxes; ++a) {
                    // q with 0 <= q*s + r - p < L_out
                    const int lo = A[a].p - r[a];
                    q0[a] = lo <= 0 ? 0 : (lo + A[a].s - 1) / A[a].s;
                    const int o0 = q0[a] * A[a].s + r[a] - A[a].p;
                    nq[a] = o0 < A[a].L_out ? (A[a].L_out - 1 - o0) / A[a].s + 1 : 0;
                    empty |= nq[a] == 0;
                }
                if (empty) continue;
                if (th_only > 0 && rows_key(A, r) != th_only) continue;
                if (P.n_cls == kMaxPhaseCls) return false;
                const int c = P.n_cls++;
                for (int a = 0; a < kAxes; ++a) {
                    P.cls_r[c][a] = r[a];
                    P.cls_q0[c][a] = q0[a];
                    P.cls_nq[c][a] = nq[a];
                }
                P.cls_blk0[c] = blocks;
                int taps = 1;
                for (int a = 0; a < kAxes; ++a) taps *= A[a].tap_start[r[a] + 1] - A[a].tap_start[r[a]];
                P.max_taps = taps > P.max_taps ? taps : P.max_taps;
                const int64_t per_thread = rows > 0 ? 1 : kPhasePos;
                const int64_t pos = (int64_t)nq[0] * (rows > 0 ? (nq[1] + rows - 1) / rows : nq[1]) * nq[2];
                blocks += (int)((pos + kBlock * per_thread - 1) / (kBlock * per_thread));
            }
    P.cls_blk0[P.n_cls] = blocks;
    // the staged weights of the class with the most taps must fit in LDS
    P.tap_stride = tap_stride(Pl.Cig, pick_cpt(Pl.Cog), rows > 0);
    return (int64_t)P.max_taps * P.tap_stride * 4 <= kMaxPhaseLds;
}

template <typename Launch>
int launch_classes(const convt_plan &Pl, PhaseParams &P, int cpt, Launch &&launch) {
    P.co_chunks = (int)((Pl.Cog + cpt - 1) / cpt);
    const unsigned gx = (unsigned)P.cls_blk0[P.n_cls];
    const unsigned gy = (unsigned)(Pl.G * P.co_chunks);
    if (gx == 0) return 0;
    for (int64_t n0 = 0; n0 < Pl.N; n0 += 65535) {
        P.n0 = (int)n0;
        const unsigned gz = (unsigned)(Pl.N - n0 < 65535 ? Pl.N - n0 : 65535);
        const size_t lds = (size_t)P.max_taps * P.tap_stride * sizeof(float);
        launch(dim3(gx, gy, gz), lds);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

template <int CPT>
int launch_phase(const convt_plan &Pl, PhaseParams &P, const float *x, const float *w,
                 const float *bias, const float *add, float *y, hipStream_t st) {
    return launch_classes(Pl, P, CPT, [&](dim3 grid, size_t lds) {
        if (add)
            hipLaunchKernelGGL((k_generic_phase<CPT, kPhasePos, true>), grid, dim3(kBlock), lds, st, P, x, w,
                               bias, add, y);
        else
            hipLaunchKernelGGL((k_generic_phase<CPT, kPhasePos, false>), grid, dim3(kBlock), lds, st, P, x, w,
                               bias, add, y);
    });
}

template <int CPT, int TH>
int launch_rows(const convt_plan &Pl, PhaseParams &P, const float *x, const float *w,
                const float *bias, const float *add, float *y, hipStream_t st) {
    constexpr int CH = 64 / CPT;
    const bool full = Pl.Cig % CH == 0;
    return launch_classes(Pl, P, CPT, [&](dim3 grid, size_t lds) {
        if (full) {
            if (add)
                hipLaunchKernelGGL((k_generic_rows<CPT, kRows, TH, true, true>), grid, dim3(kBlock), lds, st, P,
                                   x, w, bias, add, y);
            else
                hipLaunchKernelGGL((k_generic_rows<CPT, kRows, TH, true, false>), grid, dim3(kBlock), lds, st, P,
                                   x, w, bias, add, y);
        } else {
            if (add)
                hipLaunchKernelGGL((k_generic_rows<CPT, kRows, TH, false, true>), grid, dim3(kBlock), lds, st, P,
                                   x, w, bias, add, y);
            else
                hipLaunchKernelGGL((k_generic_rows<CPT, kRows, TH, false, false>), grid, dim3(kBlock), lds, st, P,
                                   x, w, bias, add, y);
        }
    });
}

// One launch per H tap count present (bias-only classes with the first), each
// over the classes with exactly that many H taps.
template <int CPT>
int launch_rows_all(int th_max, const convt_plan &Pl, PhaseParams &Q, const float *x, const float *w,
                    const float *bias, const float *add, float *y, hipStream_t st) {
    static_assert(kRowsMaxTH == 5, "one case per instantiated H tap count");
    for (int th = 1; th <= th_max; ++th) {
        PhaseParams P = Q;
        if (!phase_classes(Pl, P, kRows, th)) return (int)hipErrorInvalidValue; // checked in rows_plan
        if (P.n_cls == 0) continue;
        int e = 0;
        switch (th) {
        case 1: e = launch_rows<CPT, 1>(Pl, P, x, w, bias, add, y, st); break;
        case 2: e = launch_rows<CPT, 2>(Pl, P, x, w, bias, add, y, st); break;
        case 3: e = launch_rows<CPT, 3>(Pl, P, x, w, bias, add, y, st); break;
        case 4: e = launch_rows<CPT, 4>(Pl, P, x, w, bias, add, y, st); break;
        default: e = launch_rows<CPT, 5>(Pl, P, x, w, bias, add, y, st); break;
        }
        if (e) return e;
    }
    return 0;
}

// The rows kernel applies and every per-tap-count launch fits its tables and LDS.
int rows_plan(const convt_plan &Pl) {
    const int th = rows_th(Pl);
    if (th == 0) return 0;
    for (int t = 1; t <= th; ++t) {
        PhaseParams P;
        if (!phase_classes(Pl, P, kRows, t)) return 0;
    }
    return th;
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

} // namespace

const char *generic_kernel_name(const convt_plan &Pl) {
    PhaseParams P;
    if (rows_plan(Pl) > 0) return "k_generic_rows";
    if (phase_classes(Pl, P, 0)) return "k_generic_phase";
    return "k_generic";
}

bool generic_supports(const convt_plan &P) {
    const int cpt = pick_cpt(P.Cog);
    return P.G * ((P.Cog + cpt - 1) / cpt) <= 65535;
}

int launch_generic(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                   const float *add, float *y, void *stream) {
    {
        PhaseParams Q;
        const int th = rows_plan(Pl);
        const bool rows = th > 0;
        if (rows || phase_classes(Pl, Q, 0)) {
            for (int a = 0; a < kAxes; ++a) Q.ax[a] = Pl.ax[a];
            Q.C_in = (int)Pl.C_in;
            Q.C_out = (int)Pl.C_out;
            Q.Cig = (int)Pl.Cig;
            Q.Cog = (int)Pl.Cog;
            Q.k_vol = (int)Pl.k_vol;
            Q.in_sp = (int)Pl.in_sp;
            Q.out_sp = (int)Pl.out_sp;
            hipStream_t st = (hipStream_t)stream;
            if (rows) {
                if (pick_cpt(Pl.Cog) == 8) return launch_rows_all<8>(th, Pl, Q, x, w, bias, add, y, st);
                return launch_rows_all<4>(th, Pl, Q, x, w, bias, add, y, st);
            }
            switch (pick_cpt(Pl.Cog)) {
            case 8: return launch_phase<8>(Pl, Q, x, w, bias, add, y, st);
            case 4: return launch_phase<4>(Pl, Q, x, w, bias, add, y, st);
            case 2: return launch_phase<2>(Pl, Q, x, w, bias, add, y, st);
            default: return launch_phase<1>(Pl, Q, x, w, bias, add, y, st);
            }
        }
    }
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
