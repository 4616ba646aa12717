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
static_assert(kBlock == 4 * 64, "weight staging deals rows to four waves");

struct GenericParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, k_vol;
    int in_sp, out_sp;
    int co_chunks;
    int n0; // first batch index of this launch
};

template <int CPT, int EPI>
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
        const float a = epi_add(EPI) ? add[idx] : 0.0f;
        y[idx] = epilogue<EPI>(acc[j], b, a);
    }
}

// --------------------------------------------------------- channels last
// Any shape with x (N, L_in..., C_in) and y, add_input (N, L_out..., C_out):
// one thread per output element, the channel fastest, so a wave's stores
// cover contiguous channels of consecutive positions, and the threads of one
// position read the same input value (one broadcast load per tap and input
// channel).  The gather walks the element's phase taps as k_generic does.
template <int EPI>
__global__ __launch_bounds__(kBlock) void k_generic_nxc(const GenericParams P, int64_t total,
                                                        const float *__restrict__ x,
                                                        const float *__restrict__ w,
                                                        const float *__restrict__ bias,
                                                        const float *add, float *y) {
    const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (idx >= total) return;
    const int co = (int)(idx % P.C_out);
    const int64_t t = idx / P.C_out;
    const int sp = (int)(t % P.out_sp);
    const int64_t n = t / P.out_sp;
    const int g = co / P.Cog, co_l = co - g * P.Cog;

    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int ow = sp % AW.L_out;
    const int t2 = sp / AW.L_out;
    const int oh = t2 % AH.L_out;
    const int od = t2 / AH.L_out;
    const int td = od + AD.p, th = oh + AH.p, tw = ow + AW.p;
    const int rd = td % AD.s, qd = td / AD.s;
    const int rh = th % AH.s, qh = th / AH.s;
    const int rw = tw % AW.s, qw = tw / AW.s;

    float acc = 0.0f;
    const float *xn = x + n * P.in_sp * P.C_in + (int64_t)g * P.Cig;
    const float *wg = w + ((int64_t)g * P.Cig * P.Cog + co_l) * P.k_vol;
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
                const float *xp = xn + (int64_t)((id * AH.L_in + ih) * AW.L_in + iw) * P.C_in;
                const float *wp = wg + kidx;
                for (int ci = 0; ci < P.Cig; ++ci)
                    acc = fmaf(xp[ci], wp[(int64_t)ci * P.Cog * P.k_vol], acc);
            }
        }
    }
    const float a = epi_add(EPI) ? add[idx] : 0.0f;
    y[idx] = epilogue<EPI>(acc, bias ? bias[co] : 0.0f, a);
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
    int lds_bytes;                   // dynamic LDS of a workgroup
};
constexpr int kMaxPhaseLds = 32768; // bytes of staged weights per workgroup

template <int CPT, int NPOS, int EPI>
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
            const float a = epi_add(EPI) ? add[idx] : 0.0f;
            y[idx] = epilogue<EPI>(acc[u][j], b, a);
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

// Weight staging shared by the row kernels.  The staged operand is nrows rows
// of 64 floats; row r holds, in lane l, the weight at element offset
// lane_off + src(r).off of w, where src(r).off is uniform (the tap's offset
// plus the row's first input channel times the channel stride) and lane_off
// is the lane's own channel and column.  A lane whose channel lies past the
// group's last (lane_ci + src(r).ci0 >= Cig) gets zero.  Rows are dealt to
// wave r % 4, and each wave issues kStageBatch loads (out of range, so zero,
// where there is no weight) before it writes any of them to LDS, so their
// latencies overlap.
constexpr int kStageBatch = 8;

struct WRow {
    unsigned off; // uniform element offset of the row (tap and channel part)
    int ci0;      // first input channel of the row
};

template <typename Src>
__device__ __forceinline__ void stage_weight_rows(float *wl, rsrc_t rw, unsigned lane_off, int lane_ci, int Cig,
                                                  int nrows, Src &&src) {
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    for (int r0 = wv; r0 < nrows; r0 += 4 * kStageBatch) {
        float v[kStageBatch];
#pragma unroll
        for (int u = 0; u < kStageBatch; ++u) {
            const int r = r0 + 4 * u;
            unsigned o = kOutOfRange;
            if (r < nrows) {
                const WRow q = src(r);
                if (q.ci0 + lane_ci < Cig) o = 4u * (lane_off + q.off);
            }
            v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, o, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < kStageBatch; ++u)
            if (r0 + 4 * u < nrows) wl[(r0 + 4 * u) * 64 + lane] = v[u];
    }
}

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
template <int CPT, int R, int TH, bool FULLCH, int EPI>
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
        const int lane = threadIdx.x & 63;
        {
            // one 64-float row per (tap (d, h, w), 64/CPT channels): lane l
            // holds w[ci = part*64/CPT + l/CPT][co0 + l%CPT] (the group's last
            // channel for columns past it; zero past Cig)
            const rsrc_t rwt = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(w), (short)0,
                                                                 (int)(4 * P.C_in * P.Cog * P.k_vol), kRsrcWord3);
            const int c = min(lane % CPT, ncol - 1);
            const int lane_ci = lane / CPT;
            const unsigned lane_off =
                (unsigned)(((int64_t)g * P.Cig * P.Cog + co0 + (int64_t)lane_ci * P.Cog + c) * P.k_vol);
            const int parts = TS / 64;
            const unsigned ci_stride = (unsigned)(P.Cog * P.k_vol);
            stage_weight_rows(wl, rwt, lane_off, lane_ci, P.Cig, Td * TH * Tw * parts, [&](int r) -> WRow {
                const int part = r % parts, tap = r / parts;
                const int tw = tap % Tw, tdh = tap / Tw;
                const int th = tdh % TH, td = tdh / TH;
                const int kidx = (AD.tap_k[AD.tap_start[rd] + td] * AH.K + AH.tap_k[AH.tap_start[rh] + th]) *
                                     AW.K + AW.tap_k[AW.tap_start[rw] + tw];
                const int ci0 = part * (64 / CPT);
                return WRow{(unsigned)ci0 * ci_stride + (unsigned)kidx, ci0};
            });
        }
        __syncthreads();

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
            const float a = epi_add(EPI) ? add[idx] : 0.0f;
            y[idx] = epilogue<EPI>(acc[r][j / 4][j % 4], b, a);
        }
    }
}

// ------------------------------------------------ 8-channel groups, row pairs
// For groups of 8 output channels a 16-row matrix tile holds two output rows
// along H: row i = dh*8 + co of v_mfma_f32_16x16x4f32 is channel co of output
// row qh0 + dh, its columns are 16 consecutive positions along W of the class,
// and its K is 4 input channels.  With the H taps of every residue at offsets
// 0..TH-1, output row q takes tap j from input row q - j, so input row ih
// feeds row qh0 + dh through tap j = delta + dh with delta = qh0 - ih: one
// B operand (4 channels x 16 positions of input row ih) serves every row pair
// whose window contains ih, each with the A operand of its delta (TH + 1 of
// them per (D tap, W tap, channel quad); the entries with delta + dh outside
// [0, TH) are zero: 2 of the 2(TH + 1) half-tiles).  Lane layouts:
// A[i][k] at lane i + 16k, B[k][j] at lane j + 16k, D[i][j] at lane
// j + 16(i/4), accumulator register i%4.
//
// A wave owns NP row pairs x PB blocks of 16 positions of one (class, qd).
typedef float v4f_p __attribute__((ext_vector_type(4)));

template <int NP, int PB, int TH, int EPI>
__global__ __launch_bounds__(kBlock) void k_generic_pairs(const PhaseParams P,
                                                          const float *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ bias,
                                                          const float *add, float *y) {
    constexpr int ND = TH + 1;          // delta = qh0 - ih in [-1, TH - 1]
    constexpr int NR = 2 * NP + TH - 1; // input rows of a wave's window
    int c = 0;
    while (c + 1 < P.n_cls && (int)blockIdx.x >= P.cls_blk0[c + 1]) ++c;
    const int nqd = P.cls_nq[c][0], nqh = P.cls_nq[c][1], nqw = P.cls_nq[c][2];
    const int nrb = (nqh + 2 * NP - 1) / (2 * NP);
    const int nwb = (nqw + 16 * PB - 1) / (16 * PB);
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int rd = P.cls_r[c][0], rh = P.cls_r[c][1], rw = P.cls_r[c][2];
    const int wave = ((int)blockIdx.x - P.cls_blk0[c]) * (kBlock / 64) + (int)(threadIdx.x >> 6);
    const bool wlive = wave < nqd * nrb * nwb;
    const int iwb = wave % nwb;
    const int t2 = wave / nwb;
    const int irb = t2 % nrb;
    const int iqd = t2 / nrb;
    const int lane = threadIdx.x & 63;
    const int j16 = lane & 15, k4 = lane >> 4;
    const int qd = P.cls_q0[c][0] + iqd;
    const int qh0 = P.cls_q0[c][1] + irb * 2 * NP;
    int iqw[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) iqw[pb] = iwb * 16 * PB + pb * 16 + j16;

    const int g = blockIdx.y / P.co_chunks;
    const int co0 = (blockIdx.y % P.co_chunks) * 8;
    const int n = P.n0 + blockIdx.z;

    v4f_p acc[NP][PB];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) acc[p][pb] = v4f_p{0.0f, 0.0f, 0.0f, 0.0f};

    const int Td = AD.tap_start[rd + 1] - AD.tap_start[rd];
    const int Th = AH.tap_start[rh + 1] - AH.tap_start[rh];
    const int Tw = AW.tap_start[rw + 1] - AW.tap_start[rw];
    if (Td * Th * Tw > 0) {
        // Staged weights as in k_generic_rows with CPT = 8: [class tap (d, h,
        // w)][input channel][8 columns], tap_stride floats per tap.  Th == TH.
        extern __shared__ __attribute__((aligned(16))) float wl[];
        const int NQ = P.Cig / 4;
        const int TS = P.tap_stride;
        {
            const rsrc_t rwt = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(w), (short)0,
                                                                 (int)(4 * P.C_in * P.Cog * P.k_vol), kRsrcWord3);
            const int lane_ci = lane / 8;
            const unsigned lane_off =
                (unsigned)(((int64_t)g * P.Cig * P.Cog + co0 + (int64_t)lane_ci * P.Cog + lane % 8) * P.k_vol);
            const int parts = TS / 64;
            const unsigned ci_stride = (unsigned)(P.Cog * P.k_vol);
            stage_weight_rows(wl, rwt, lane_off, lane_ci, P.Cig, Td * TH * Tw * parts, [&](int r) -> WRow {
                const int part = r % parts, tap = r / parts;
                const int tw = tap % Tw, tdh = tap / Tw;
                const int th = tdh % TH, td = tdh / TH;
                const int kidx = (AD.tap_k[AD.tap_start[rd] + td] * AH.K + AH.tap_k[AH.tap_start[rh] + th]) *
                                     AW.K + AW.tap_k[AW.tap_start[rw] + tw];
                return WRow{(unsigned)(part * 8) * ci_stride + (unsigned)kidx, part * 8};
            });
        }
        __syncthreads();

        const rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig) * P.in_sp), (short)0,
            (int)(4 * P.Cig * P.in_sp), kRsrcWord3);
        const unsigned ch_bytes = 4u * (unsigned)P.in_sp;
        const unsigned lane_ch = (unsigned)k4 * (unsigned)P.in_sp; // this lane's channel in the quad
        const int ih0 = qh0 - (TH - 1);
        const int a_dh = (lane >> 3) & 1;
        const int a_lane = 8 * k4 + (lane & 7);
        for (int td = 0; td < Td; ++td) {
            const int id = qd - AD.tap_c[AD.tap_start[rd] + td];
            const bool okd = wlive && id >= 0 && id < AD.L_in;
            for (int tw = 0; tw < Tw; ++tw) {
                const int cw = AW.tap_c[AW.tap_start[rw] + tw];
                unsigned base[PB];
                bool ok[PB];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    const int iw = P.cls_q0[c][2] + iqw[pb] - cw;
                    ok[pb] = okd && iqw[pb] < nqw && iw >= 0 && iw < AW.L_in;
                    base[pb] = lane_ch + (unsigned)(id * AH.L_in * AW.L_in + iw);
                }
                // the window's row offsets, shared by every channel quad
                unsigned vo[NR][PB];
#pragma unroll
                for (int u = 0; u < NR; ++u) {
                    const int ih = ih0 + u;
                    const bool okh = ih >= 0 && ih < AH.L_in;
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
                        vo[u][pb] = ok[pb] && okh ? 4u * (base[pb] + (unsigned)(ih * AW.L_in)) : kOutOfRange;
                }
                for (int q = 0; q < NQ; ++q) {
                    // A of delta = di - 1: lane i + 16k takes channel 4q + k,
                    // column i%8, H tap di - 1 + i/8 (zero outside [0, TH))
                    float a[ND];
                    const float *wq = wl + (td * TH * Tw + tw) * TS + 32 * q + a_lane;
#pragma unroll
                    for (int di = 0; di < ND; ++di) {
                        const int th = di - 1 + a_dh;
                        const float v = wq[min(max(th, 0), TH - 1) * Tw * TS];
                        a[di] = th >= 0 && th < TH ? v : 0.0f;
                    }
                    const unsigned soff = (unsigned)(4 * q) * ch_bytes;
#pragma unroll
                    for (int u = 0; u < NR; ++u) {
                        float b[PB];
#pragma unroll
                        for (int pb = 0; pb < PB; ++pb)
                            b[pb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vo[u][pb], soff, 0));
#pragma unroll
                        for (int p = 0; p < NP; ++p) {
                            // delta = qh0 + 2p - ih = 2p + TH - 1 - u
                            const int di = 2 * p + TH - u; // delta + 1
                            if (di < 0 || di >= ND) continue;
#pragma unroll
                            for (int pb = 0; pb < PB; ++pb)
                                acc[p][pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[di], b[pb], acc[p][pb], 0, 0, 0);
                        }
                    }
                }
            }
        }
    }

    if (!wlive) return;
    // lane j16 + 16*k4, register v: position j16, output row dh = k4/2,
    // channel 4*(k4%2) + v.  Stores (and add_input loads) through a resource
    // over the sample's output: the lane's byte offset of channel cb, the
    // channel step v*out_sp in the scalar offset; rows and positions past the
    // class's end take an out-of-range offset and are dropped.
    const int dh = k4 >> 1;
    const int cb = g * P.Cog + co0 + 4 * (k4 & 1);
    const int od = qd * AD.s + rd - AD.p;
    const int ybytes = 4 * P.C_out * P.out_sp;
    const rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(y + (int64_t)n * P.C_out * P.out_sp, (short)0, ybytes,
                                                        kRsrcWord3);
    const rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(epi_add(EPI) ? add + (int64_t)n * P.C_out * P.out_sp : y), (short)0, ybytes, kRsrcWord3);
    float bb[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) bb[v] = bias ? bias[cb + v] : 0.0f;
    const unsigned ch_step = 4u * (unsigned)P.out_sp;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int iqh = irb * 2 * NP + 2 * p + dh;
        const int oh = (P.cls_q0[c][1] + iqh) * AH.s + rh - AH.p;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) {
            const int ow = (P.cls_q0[c][2] + iqw[pb]) * AW.s + rw - AW.p;
            const bool in = iqh < nqh && iqw[pb] < nqw;
            const unsigned vo =
                in ? 4u * (unsigned)(cb * P.out_sp + (od * AH.L_out + oh) * AW.L_out + ow) : kOutOfRange;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float aa = epi_add(EPI) ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                       ra, vo, v * ch_step, 0))
                                       : 0.0f;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, epilogue<EPI>(acc[p][pb][v], bb[v], aa)),
                                                      ry, vo, v * ch_step, 0);
            }
        }
    }
}

constexpr int kPairs = 4;      // row pairs per wave in k_generic_pairs
constexpr int kPairBlocks = 1; // 16-position blocks per wave
constexpr int kMaxPairsLds = 65536;

constexpr int kRows = 4;     // H rows per thread in k_generic_rows
constexpr int kRowsMaxTH = 5; // largest H tap count instantiated

// Largest H tap count of the shape if k_generic_rows applies, else 0: 4-channel
// blocks, a group's input, the weights and a sample's output below 2 GiB
// (byte offsets of buffer resources), at least kRows outputs
// along H, and on H every residue's taps at offsets 0, 1, .., T-1.
int rows_th(const convt_plan &Pl) {
    if (pick_cpt(Pl.Cog) < 4) return 0;
    if (4 * Pl.Cig * Pl.in_sp > 0x7fffffff) return 0;           // byte offsets in the buffer
    if (4 * Pl.C_in * Pl.Cog * Pl.k_vol > 0x7fffffff) return 0; // resources over x and w
    if (4 * Pl.C_out * Pl.out_sp > 0x7fffffff) return 0;        // and a sample's output
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
// Launch key of a class for the row kernels: its H tap count, with bias-only
// classes (no tap on some axis) in the 1-tap launch, which skips their
// contraction.
int rows_key(const AxisPlan *A, const int r[kAxes]) {
    int taps = 1;
    for (int a = 0; a < kAxes; ++a) taps *= A[a].tap_start[r[a] + 1] - A[a].tap_start[r[a]];
    return taps == 0 ? 1 : A[1].tap_start[r[1] + 1] - A[1].tap_start[r[1]];
}

// How a launch lays out the positions of a class.
enum class Layout { kFma, kRows, kPairs };

// The class table of a launch: every class with output positions (th_only > 0
// keeps those whose rows_key is th_only), the first workgroup of each, and the
// LDS the staged weights take.  False when the shape has more classes than the
// table holds or the weights do not fit.
bool phase_classes(const convt_plan &Pl, PhaseParams &P, Layout lay, int th_only = 0) {
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
                int64_t units, per_block; // threads (or waves) and units per workgroup
                if (lay == Layout::kPairs) {
                    units = (int64_t)nq[0] * ((nq[1] + 2 * kPairs - 1) / (2 * kPairs)) *
                            ((nq[2] + 16 * kPairBlocks - 1) / (16 * kPairBlocks));
                    per_block = kBlock / 64;
                } else if (lay == Layout::kRows) {
                    units = (int64_t)nq[0] * ((nq[1] + kRows - 1) / kRows) * nq[2];
                    per_block = kBlock;
                } else {
                    units = (int64_t)nq[0] * nq[1] * nq[2];
                    per_block = kBlock * kPhasePos;
                }
                blocks += (int)((units + per_block - 1) / per_block);
            }
    P.cls_blk0[P.n_cls] = blocks;
    // the staged weights of the class with the most taps must fit in LDS
    P.tap_stride = tap_stride(Pl.Cig, lay == Layout::kPairs ? 8 : pick_cpt(Pl.Cog), lay != Layout::kFma);
    int64_t bytes;
    bytes = (int64_t)P.max_taps * P.tap_stride * 4;
    const int64_t limit = lay == Layout::kPairs ? kMaxPairsLds : kMaxPhaseLds;
    if (bytes > limit) return false;
    P.lds_bytes = (int)bytes;
    return true;
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
        launch(dim3(gx, gy, gz), (size_t)P.lds_bytes);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

template <int CPT>
int launch_phase(const convt_plan &Pl, PhaseParams &P, const float *x, const float *w,
                 const float *bias, const float *add, int act, float *y, hipStream_t st) {
    return launch_classes(Pl, P, CPT, [&](dim3 grid, size_t lds) {
        with_epi(add != nullptr, act, [&](auto E) {
            hipLaunchKernelGGL((k_generic_phase<CPT, kPhasePos, decltype(E)::value>),
                               grid, dim3(kBlock), lds, st, P, x, w, bias, add, y);
        });
    });
}

template <int CPT, int TH>
int launch_rows(const convt_plan &Pl, PhaseParams &P, const float *x, const float *w,
                const float *bias, const float *add, int act, float *y, hipStream_t st) {
    constexpr int CH = 64 / CPT;
    const bool full = Pl.Cig % CH == 0;
    return launch_classes(Pl, P, CPT, [&](dim3 grid, size_t lds) {
        if (full) {
            with_epi(add != nullptr, act, [&](auto E) {
                hipLaunchKernelGGL((k_generic_rows<CPT, kRows, TH, true, decltype(E)::value>),
                                   grid, dim3(kBlock), lds, st, P, x, w, bias, add, y);
            });
        } else {
            with_epi(add != nullptr, act, [&](auto E) {
                hipLaunchKernelGGL((k_generic_rows<CPT, kRows, TH, false, decltype(E)::value>),
                                   grid, dim3(kBlock), lds, st, P, x, w, bias, add, y);
            });
        }
    });
}

// One launch per H tap count present (bias-only classes with the first), each
// over the classes with exactly that many H taps.
template <int CPT>
int launch_rows_all(int th_max, const convt_plan &Pl, PhaseParams &Q, const float *x, const float *w,
                    const float *bias, const float *add, int act, float *y, hipStream_t st) {
    static_assert(kRowsMaxTH == 5, "one case per instantiated H tap count");
    for (int th = 1; th <= th_max; ++th) {
        PhaseParams P = Q;
        if (!phase_classes(Pl, P, Layout::kRows, th)) return (int)hipErrorInvalidValue; // checked in rows_plan
        if (P.n_cls == 0) continue;
        int e = 0;
        switch (th) {
        case 1: e = launch_rows<CPT, 1>(Pl, P, x, w, bias, add, act, y, st); break;
        case 2: e = launch_rows<CPT, 2>(Pl, P, x, w, bias, add, act, y, st); break;
        case 3: e = launch_rows<CPT, 3>(Pl, P, x, w, bias, add, act, y, st); break;
        case 4: e = launch_rows<CPT, 4>(Pl, P, x, w, bias, add, act, y, st); break;
        default: e = launch_rows<CPT, 5>(Pl, P, x, w, bias, add, act, y, st); break;
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
        if (!phase_classes(Pl, P, Layout::kRows, t)) return 0;
    }
    return th;
}

// k_generic_pairs applies: groups of a multiple of 8 output channels and of 4
// input channels, the conditions of the rows kernel, and per H tap count a
// class table whose A operands fit in LDS.  Returns the largest H tap count.
int pairs_plan(const convt_plan &Pl) {
    if (Pl.Cog % 8 != 0 || Pl.Cig % 4 != 0) return 0;
    const int th = rows_th(Pl);
    if (th == 0) return 0;
    for (int t = 1; t <= th; ++t) {
        PhaseParams P;
        if (!phase_classes(Pl, P, Layout::kPairs, t)) return 0;
    }
    return th;
}

template <int TH>
int launch_pairs(const convt_plan &Pl, PhaseParams &P, const float *x, const float *w,
                 const float *bias, const float *add, int act, float *y, hipStream_t st) {
    return launch_classes(Pl, P, 8, [&](dim3 grid, size_t lds) {
        with_epi(add != nullptr, act, [&](auto E) {
            hipLaunchKernelGGL((k_generic_pairs<kPairs, kPairBlocks, TH, decltype(E)::value>),
                               grid, dim3(kBlock), lds, st, P, x, w, bias, add, y);
        });
    });
}

int launch_pairs_all(int th_max, const convt_plan &Pl, PhaseParams &Q, const float *x, const float *w,
                     const float *bias, const float *add, int act, float *y, hipStream_t st) {
    static_assert(kRowsMaxTH == 5, "one case per instantiated H tap count");
    for (int th = 1; th <= th_max; ++th) {
        PhaseParams P = Q;
        if (!phase_classes(Pl, P, Layout::kPairs, th)) return (int)hipErrorInvalidValue; // checked in pairs_plan
        if (P.n_cls == 0) continue;
        int e = 0;
        switch (th) {
        case 1: e = launch_pairs<1>(Pl, P, x, w, bias, add, act, y, st); break;
        case 2: e = launch_pairs<2>(Pl, P, x, w, bias, add, act, y, st); break;
        case 3: e = launch_pairs<3>(Pl, P, x, w, bias, add, act, y, st); break;
        case 4: e = launch_pairs<4>(Pl, P, x, w, bias, add, act, y, st); break;
        default: e = launch_pairs<5>(Pl, P, x, w, bias, add, act, y, st); break;
        }
        if (e) return e;
    }
    return 0;
}

template <int CPT>
int launch_cpt(const convt_plan &Pl, const GenericParams &base, const float *x, const float *w,
               const float *bias, const float *add, int act, float *y, hipStream_t st) {
    GenericParams P = base;
    P.co_chunks = (int)((Pl.Cog + CPT - 1) / CPT);
    const unsigned gx = (unsigned)((Pl.out_sp + kBlock - 1) / kBlock);
    const unsigned gy = (unsigned)(Pl.G * P.co_chunks);
    for (int64_t n0 = 0; n0 < Pl.N; n0 += 65535) {
        P.n0 = (int)n0;
        const unsigned gz = (unsigned)(Pl.N - n0 < 65535 ? Pl.N - n0 : 65535);
        dim3 grid(gx, gy, gz);
        with_epi(add != nullptr, act, [&](auto E) {
            hipLaunchKernelGGL((k_generic<CPT, decltype(E)::value>),
                               grid, dim3(kBlock), 0, st, P, x, w, bias, add, y);
        });
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

} // namespace

// The W-pair kernel (wpair.hip) goes first where it applies (CONVT_WPAIR=0
// builds without it).
#ifndef CONVT_WPAIR
#define CONVT_WPAIR 1
#endif

const char *generic_kernel_name(const convt_plan &Pl) {
    if (Pl.layout == CONVT_LAYOUT_CHANNELS_LAST) return "k_generic_nxc";
    if (CONVT_WPAIR && wpair_supports(Pl)) return "k_generic_wpair";
    PhaseParams P;
    if (pairs_plan(Pl) > 0) return "k_generic_pairs";
    if (rows_plan(Pl) > 0) return "k_generic_rows";
    if (phase_classes(Pl, P, Layout::kFma)) return "k_generic_phase";
    return "k_generic";
}

bool generic_supports(const convt_plan &P) {
    // channels last: one thread per output element, a grid of at most 2^31 - 1 blocks
    if (P.layout == CONVT_LAYOUT_CHANNELS_LAST) return (P.N * P.out_sp * P.C_out + kBlock - 1) / kBlock < INT32_MAX;
    const int cpt = pick_cpt(P.Cog);
    return P.G * ((P.Cog + cpt - 1) / cpt) <= 65535;
}

int launch_generic(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                   const float *add, int act, float *y, void *stream) {
    if (Pl.layout == CONVT_LAYOUT_CHANNELS_LAST) {
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
        const int64_t total = Pl.N * Pl.out_sp * Pl.C_out;
        const unsigned grid = (unsigned)((total + kBlock - 1) / kBlock);
        with_epi(add != nullptr, act, [&](auto E) {
            hipLaunchKernelGGL((k_generic_nxc<decltype(E)::value>), dim3(grid), dim3(kBlock), 0, (hipStream_t)stream,
                               P, total, x, w, bias, add, y);
        });
        return (int)hipGetLastError();
    }
    if (CONVT_WPAIR && wpair_supports(Pl)) return launch_wpair(Pl, x, w, bias, add, act, y, stream);
    {
        PhaseParams Q;
        const int thp = pairs_plan(Pl);
        const int th = thp > 0 ? 0 : rows_plan(Pl);
        const bool rows = th > 0;
        if (thp > 0 || rows || phase_classes(Pl, Q, Layout::kFma)) {
            for (int a = 0; a < kAxes; ++a) Q.ax[a] = Pl.ax[a];
            Q.C_in = (int)Pl.C_in;
            Q.C_out = (int)Pl.C_out;
            Q.Cig = (int)Pl.Cig;
            Q.Cog = (int)Pl.Cog;
            Q.k_vol = (int)Pl.k_vol;
            Q.in_sp = (int)Pl.in_sp;
            Q.out_sp = (int)Pl.out_sp;
            hipStream_t st = (hipStream_t)stream;
            if (thp > 0) return launch_pairs_all(thp, Pl, Q, x, w, bias, add, act, y, st);
            if (rows) {
                if (pick_cpt(Pl.Cog) == 8) return launch_rows_all<8>(th, Pl, Q, x, w, bias, add, act, y, st);
                return launch_rows_all<4>(th, Pl, Q, x, w, bias, add, act, y, st);
            }
            switch (pick_cpt(Pl.Cog)) {
            case 8: return launch_phase<8>(Pl, Q, x, w, bias, add, act, y, st);
            case 4: return launch_phase<4>(Pl, Q, x, w, bias, add, act, y, st);
            case 2: return launch_phase<2>(Pl, Q, x, w, bias, add, act, y, st);
            default: return launch_phase<1>(Pl, Q, x, w, bias, add, act, y, st);
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
    case 8: return launch_cpt<8>(Pl, P, x, w, bias, add, act, y, st);
    case 4: return launch_cpt<4>(Pl, P, x, w, bias, add, act, y, st);
    case 2: return launch_cpt<2>(Pl, P, x, w, bias, add, act, y, st);
    default: return launch_cpt<1>(Pl, P, x, w, bias, add, act, y, st);
    }
}

} // namespace convt
