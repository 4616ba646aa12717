// Input gradient of the transposed convolution: the adjoint of the forward's
// linear part (no bias, no epilogue).  The forward adds x[n, ci, i] *
// w[ci, co_l, k] to y[n, g*Cog + co_l, o] at o = i*s - p + k*d per axis, so
//   dx[n, ci, i] = sum_{co_l, k : o in [0, L_out) on every axis}
//                  w[ci, co_l, k] * dy[n, g*Cog + co_l, o].
// "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d, dilation 2): the adjoint
// derivation that defines the transposed convolution as the transpose of the
// strided convolution; "Kimi-K2.6 l2_p26" transcript: the convolution matrix C
// and C^T.  Unlike the forward there are no stride phases here: every input
// position meets every tap, and only taps that leave the output are skipped.
//
// Gather, input-stationary: a thread owns one input position and CPI
// consecutive input channels of one group; consecutive lanes take consecutive
// positions along W, so dx stores coalesce and dy loads step by the W stride.
// The workgroup's weights, [tap][co_l][CPI], are staged in LDS a chunk of
// taps at a time and read as broadcasts, so each dy value loaded feeds CPI
// FMAs.  Every dx element is written once by one thread; no atomics.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "backward.h"

namespace convt {
namespace {

constexpr int kBwdBlock = 256;
constexpr int kBwdMaxLds = 32768; // bytes of staged weights per workgroup

struct BwdParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, k_vol;
    int in_sp, out_sp;
    int ci_chunks;
    int taps_per_chunk; // taps whose weights are staged at once
    int win_pitch;      // floats per staged dy window row (the one-axis matrix kernel)
    int tiles_per_wg;   // position tiles a workgroup of the one-axis matrix kernel walks
    int win_cols;       // columns of that kernel's dy window
    int win_cs;         // output step per window column (s when s divides d, else 1)
    int win_js, win_kd; // window columns per input position (s/cs) and per tap (d/cs)
    int n0;             // first batch index of this launch
};

template <int CPI>
__global__ __launch_bounds__(kBwdBlock) void k_backward_data(const BwdParams P, const float *__restrict__ dy,
                                                             const float *__restrict__ w,
                                                             float *__restrict__ dx) {
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int sp = blockIdx.x * kBwdBlock + threadIdx.x;
    const bool live = sp < P.in_sp;
    const int g = blockIdx.y / P.ci_chunks;
    const int ci0 = (blockIdx.y % P.ci_chunks) * CPI;
    const int n = P.n0 + blockIdx.z;
    const int nci = min(CPI, P.Cig - ci0);

    const int iw = sp % AW.L_in;
    const int t2 = sp / AW.L_in;
    const int ih = t2 % AH.L_in;
    const int id = t2 / AH.L_in;

    float acc[CPI];
#pragma unroll
    for (int j = 0; j < CPI; ++j) acc[j] = 0.0f;

    // ws[(t*Cog + co_l)*CPI + j] = w[g*Cig + ci0 + j][co_l][t0 + t] for the
    // chunk's taps t; channels past the group's last repeat it (their sums are
    // never stored)
    extern __shared__ __attribute__((aligned(16))) float ws[];
    const float *wg = w + (int64_t)(g * P.Cig + ci0) * P.Cog * P.k_vol;
    const float *dyg = dy + ((int64_t)n * P.C_out + (int64_t)g * P.Cog) * P.out_sp;
    for (int t0 = 0; t0 < P.k_vol; t0 += P.taps_per_chunk) {
        const int tc = min(P.taps_per_chunk, P.k_vol - t0);
        if (t0 > 0) __syncthreads(); // the previous chunk is consumed
        // eight loads in flight per thread (indexes past the last element
        // repeat it)
        const int nw = tc * P.Cog * CPI;
        for (int e0 = threadIdx.x; e0 < nw; e0 += 8 * kBwdBlock) {
            float t8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = min(e0 + u * kBwdBlock, nw - 1);
                const int j = e % CPI, t = e / CPI;
                const int co_l = t % P.Cog, tap = t / P.Cog;
                t8[u] = wg[((int64_t)min(j, nci - 1) * P.Cog + co_l) * P.k_vol + t0 + tap];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (e0 + u * kBwdBlock < nw) ws[e0 + u * kBwdBlock] = t8[u];
        }
        __syncthreads();
        for (int t = 0; t < tc; ++t) {
            const int k = t0 + t;
            const int kw = k % AW.K, kdh = k / AW.K;
            const int kh = kdh % AH.K, kd = kdh / AH.K;
            const int od = id * AD.s - AD.p + kd * AD.d;
            const int oh = ih * AH.s - AH.p + kh * AH.d;
            const int ow = iw * AW.s - AW.p + kw * AW.d;
            const bool ok = live && od >= 0 && od < AD.L_out && oh >= 0 && oh < AH.L_out && ow >= 0 &&
                            ow < AW.L_out;
            // lanes whose tap leaves the output read the slab's first element
            // and use 0
            const float *dyo = dyg + (ok ? (od * AH.L_out + oh) * AW.L_out + ow : 0);
            const float *wk = ws + t * P.Cog * CPI;
#pragma unroll 4
            for (int co_l = 0; co_l < P.Cog; ++co_l) {
                const float v0 = dyo[(int64_t)co_l * P.out_sp];
                const float v = ok ? v0 : 0.0f;
                const float *wc = wk + co_l * CPI;
#pragma unroll
                for (int j = 0; j < CPI; ++j) acc[j] = fmaf(v, wc[j], acc[j]);
            }
        }
    }

    if (!live) return;
#pragma unroll
    for (int j = 0; j < CPI; ++j) {
        if (j >= nci) break;
        dx[((int64_t)n * P.C_in + g * P.Cig + ci0 + j) * P.in_sp + sp] = acc[j];
    }
}

// ----------------------------------------------------------- matrix cores
// For groups of 16k input channels and 4k output channels the same sum is an
// implicit GEMM per tap on v_mfma_f32_16x16x4_f32: rows = 16 input channels,
// columns = 16 input positions, K = 4 output channels of the group.  A (lane
// i + 16c) = w[ci0 + i][4q + c][tap], B (lane j + 16c) = dy[4q + c][o(j, tap)],
// D (lane j + 16(i/4), register i%4) = dx[ci0 + i][position j].  A wave owns
// MT row tiles x PB position blocks, so each B it loads feeds MT MFMAs and each
// A feeds PB.  The A operands of a chunk of taps, [tap][q][m][64 lanes], are
// staged in LDS (one 64-float row each, conflict-free lane reads); dy goes
// through a buffer resource over the group's channels of one sample, the
// channel quad in the scalar offset, and a tap that leaves the output gets an
// out-of-range offset (the hardware returns zero).
typedef float bwd_v4f __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t bwd_rsrc_t;
constexpr int kBwdRsrcWord3 = 0x00020000; // raw (untyped) buffer access
constexpr unsigned kBwdOutOfRange = 0x80000000u;
// A-row loads in flight per wave while the matrix kernel stages a chunk of
// taps.  Eight is measured faster with up to 2 row tiles per wave (the
// fused-layer shape, 1.17 -> 1.14 ms) and slower with 4 (the channel-heavy
// shape, 3.52 -> 3.71 ms; 2 and 4 in flight lie between), where one is kept.
template <int MT> constexpr int stage_depth() { return MT >= 4 ? 1 : 8; }
// Four waves per SIMD for the matrix kernel: the 4-row-tile instantiation then
// keeps its accumulators in AGPRs instead of holding 168 VGPRs (three waves);
// channel-heavy shape 3.52 -> 3.36 ms, fused-layer shape unchanged, five no better.
constexpr int kMfmaWavesPerSimd = 4;
// Tuning knob: the LDS-staged variant of the matrix kernel where it applies.
#ifndef CONVT_BWD_STAGE
#define CONVT_BWD_STAGE 1
#endif
constexpr int kRowMaxT = 10; // 64-column steps of the one-axis kernel's dy window (640 columns)
constexpr int kRowMinWgs = 2048;       // the one-axis kernel's grid, at least (8 per CU)
constexpr int kRowMaxTilesPerWg = 8;
constexpr int kRowCh = 4; // output channels per staged window chunk (a multiple of 4, <= 16)

template <int MT, int PB>
__global__ __launch_bounds__(kBwdBlock, kMfmaWavesPerSimd) void k_backward_data_mfma(const BwdParams P,
                                                                                      const float *__restrict__ dy,
                                                                  const float *__restrict__ w,
                                                                  float *__restrict__ dx) {
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j16 = lane & 15, c4 = lane >> 4;
    const int g = blockIdx.y / P.ci_chunks;
    const int ci0 = (blockIdx.y % P.ci_chunks) * 16 * MT; // first input channel of the group
    const int n = P.n0 + blockIdx.z;
    const int NQ = P.Cog / 4;
    constexpr int SD = stage_depth<MT>();

    int id[PB], ih[PB], iw[PB], sp[PB];
    bool live[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
        sp[pb] = (blockIdx.x * 4 + wave) * 16 * PB + pb * 16 + j16;
        live[pb] = sp[pb] < P.in_sp;
        iw[pb] = sp[pb] % AW.L_in;
        const int t2 = sp[pb] / AW.L_in;
        ih[pb] = t2 % AH.L_in;
        id[pb] = t2 / AH.L_in;
    }

    bwd_v4f acc[MT][PB];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) acc[m][pb] = bwd_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const bwd_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + ((int64_t)n * P.C_out + (int64_t)g * P.Cog) * P.out_sp), (short)0,
        (int)(4 * P.Cog * P.out_sp), kBwdRsrcWord3);
    const unsigned quad_bytes = 16u * (unsigned)P.out_sp; // 4 channels
    const unsigned lane_ch = (unsigned)c4 * (unsigned)P.out_sp;

    extern __shared__ __attribute__((aligned(16))) float wa[];
    // lane l of row (t, q, m): w[g*Cig + ci0 + 16m + l%16][4q + l/16][t0 + t]
    const float *wl_ = w + ((int64_t)(g * P.Cig + ci0 + j16) * P.Cog + c4) * P.k_vol;
    for (int t0 = 0; t0 < P.k_vol; t0 += P.taps_per_chunk) {
        const int tc = min(P.taps_per_chunk, P.k_vol - t0);
        if (t0 > 0) __syncthreads(); // the previous chunk is consumed
        // rows dealt to waves, SD loads in flight per wave (indexes past the
        // last row repeat it)
        const int nrows = tc * NQ * MT;
        for (int r0 = wave; r0 < nrows; r0 += 4 * SD) {
            float t8[SD];
#pragma unroll
            for (int u = 0; u < SD; ++u) {
                const int r = min(r0 + 4 * u, nrows - 1);
                const int m = r % MT, t = r / MT;
                const int q = t % NQ, tap = t / NQ;
                t8[u] = wl_[((int64_t)(16 * m) * P.Cog + 4 * q) * P.k_vol + t0 + tap];
            }
#pragma unroll
            for (int u = 0; u < SD; ++u)
                if (r0 + 4 * u < nrows) wa[(r0 + 4 * u) * 64 + lane] = t8[u];
        }
        __syncthreads();
        // Steps (t, q) of the chunk, t-major.  The B operands of the next step
        // are loaded while this step's MFMAs run (two register sets, the loop
        // unrolled by two so they swap roles without copies); past the last
        // step the offsets are out of range (zeros, no traffic) and an odd
        // count ends with a step that adds nothing.  The loads are
        // unconditional, so every path issues the same ones and the waits for
        // a step's operands leave the next step's loads in flight.
        unsigned vo[PB];
        auto tap_offsets = [&](int t) {
            const int k = t0 + min(t, tc - 1);
            const int kw = k % AW.K, kdh = k / AW.K;
            const int kh = kdh % AH.K, kd = kdh / AH.K;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int od = id[pb] * AD.s - AD.p + kd * AD.d;
                const int oh = ih[pb] * AH.s - AH.p + kh * AH.d;
                const int ow = iw[pb] * AW.s - AW.p + kw * AW.d;
                const bool ok = t < tc && live[pb] && od >= 0 && od < AD.L_out && oh >= 0 && oh < AH.L_out &&
                                ow >= 0 && ow < AW.L_out;
                vo[pb] = ok ? 4u * (lane_ch + (unsigned)((od * AH.L_out + oh) * AW.L_out + ow)) : kBwdOutOfRange;
            }
        };
        auto load = [&](float (&b)[PB], int q) {
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
                b[pb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, vo[pb], q * quad_bytes, 0));
        };
        auto contract = [&](const float (&b)[PB], int t, int q) {
            const float *wt = wa + min(t, tc - 1) * NQ * MT * 64 + lane;
            float a[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) a[m] = wt[(q * MT + m) * 64];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int pb = 0; pb < PB; ++pb)
                    acc[m][pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[pb], acc[m][pb], 0, 0, 0);
        };
        const int nsteps = tc * NQ;
        int t = 0, q = 0;
        float b0[PB], b1[PB];
        tap_offsets(0);
        load(b0, 0);
        for (int st = 0; st < nsteps; st += 2) {
            int t1 = t, q1 = q + 1;
            if (q1 == NQ) q1 = 0, ++t1;
            if (q1 == 0) tap_offsets(t1);
            load(b1, q1);
            contract(b0, t, q);
            t = t1, q = q1;
            if (++q1 == NQ) q1 = 0, ++t1;
            if (q1 == 0) tap_offsets(t1);
            load(b0, q1);
            contract(b1, t, q);
            t = t1, q = q1;
        }
    }

    // lane j16 + 16*c4, register v: position j16, input channel 16m + 4*c4 + v
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
        if (!live[pb]) continue;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ci = g * P.Cig + ci0 + 16 * m + 4 * c4 + v;
                dx[((int64_t)n * P.C_in + ci) * P.in_sp + sp[pb]] = acc[m][pb][v];
            }
    }
}

// Along one axis only (1D plans: the leading axes are unit), the dy values
// that a tile of 64*PB consecutive input positions needs for all taps lie in
// one window [p0*s - p, (p0 + 64*PB - 1)*s - p + (K-1)*d] of each output
// channel row.  When d is a multiple of s only every s-th column of it is ever
// read (position j, tap k: column j*s + k*d), so the window keeps those
// columns alone: column e holds output o0 + cs*e with cs = s then, else 1.
// This variant stages the window, kRowCh output channels at a time, into LDS
// with loads along the row and reads the B operands from it, instead of
// gathering 4 channel rows per load instruction.  Every tap's A rows are
// staged once per workgroup, and a workgroup walks tiles_per_wg consecutive
// tiles.  The next (tile, chunk) window is loaded into registers while the
// current one's MFMAs run.  (A second LDS buffer, to save one of the two
// barriers per step, costs a workgroup per CU and is slower.)  Columns
// outside [0, L_out) are zero.
// Five waves per SIMD (at most 102 VGPRs) for up to 2 row tiles per wave: the
// long 1D shape 0.406 -> 0.384 ms; with 4 row tiles the bound would spill.
template <int MT> constexpr int row_waves_per_simd() { return MT >= 4 ? 1 : 5; }

template <int MT, int PB>
__global__ __launch_bounds__(kBwdBlock, row_waves_per_simd<MT>()) void k_backward_data_mfma_row(const BwdParams P,
                                                                      const float *__restrict__ dy,
                                                                      const float *__restrict__ w,
                                                                      float *__restrict__ dx) {
    const AxisPlan &AW = P.ax[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j16 = lane & 15, c4 = lane >> 4;
    const int g = blockIdx.y / P.ci_chunks;
    const int ci0 = (blockIdx.y % P.ci_chunks) * 16 * MT;
    const int n = P.n0 + blockIdx.z;
    const int NQ = P.Cog / 4;
    const int NC = P.Cog / kRowCh; // window chunks per tile
    const int K = P.k_vol;         // taps along W
    const int TP = 64 * PB;        // positions per tile
    const int Wp = P.win_pitch;    // floats per staged row (odd)
    const int Wn = P.win_cols;     // columns of the window
    const int cs = P.win_cs;       // output step per window column
    const int tile0 = blockIdx.x * P.tiles_per_wg;
    const int ntiles = min(P.tiles_per_wg, (P.in_sp + TP - 1) / TP - tile0);
    const int nsteps = ntiles * NC; // (tile, chunk) steps, chunk-minor

    extern __shared__ __attribute__((aligned(16))) float wa[];
    float *bw = wa + K * NQ * MT * 64; // the window, [kRowCh channels][Wp]

    // every tap's A rows, [tap][q][m][64 lanes]; rows dealt to waves, eight
    // loads in flight per wave (indexes past the last row repeat it)
    {
        const float *wl_ = w + ((int64_t)(g * P.Cig + ci0 + j16) * P.Cog + c4) * P.k_vol;
        const int nrows = K * NQ * MT;
        for (int r0 = wave; r0 < nrows; r0 += 32) {
            float t8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int r = min(r0 + 4 * u, nrows - 1);
                const int m = r % MT, t = r / MT;
                const int q = t % NQ, tap = t / NQ;
                t8[u] = wl_[((int64_t)(16 * m) * P.Cog + 4 * q) * P.k_vol + tap];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (r0 + 4 * u < nrows) wa[(r0 + 4 * u) * 64 + lane] = t8[u];
        }
    }

    bwd_v4f acc[MT][PB];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) acc[m][pb] = bwd_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const bwd_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + ((int64_t)n * P.C_out + (int64_t)g * P.Cog) * P.out_sp), (short)0,
        (int)(4 * P.Cog * P.out_sp), kBwdRsrcWord3);
    // this lane's window column for position block pb at tap 0
    int col[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) col[pb] = (wave * 16 * PB + pb * 16 + j16) * P.win_js;
    // wave v stages window rows RW*v .. RW*v + RW-1 of a chunk, lane l the
    // columns l + 64t (t < T <= kRowMaxT); past the last step every load is
    // out of range (zeros, no traffic)
    constexpr int RW = kRowCh / 4;
    const int T = (Wn + 63) >> 6;
    float v[RW][kRowMaxT];
    auto load_window = [&](int st) {
        const int tile = tile0 + st / NC, c0 = (st % NC) * kRowCh;
        const int o0 = tile * TP * AW.s - AW.p;
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const unsigned ch = 4u * (unsigned)((c0 + RW * wave + rr) * P.out_sp);
#pragma unroll
            for (int t = 0; t < kRowMaxT; ++t) {
                if (t >= T) break; // wave-uniform
                const int e = t * 64 + lane;
                const int o = o0 + cs * e;
                const bool ok = st < nsteps && e < Wn && o >= 0 && o < AW.L_out;
                v[rr][t] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rdy, ok ? 4u * (unsigned)o : kBwdOutOfRange, ch, 0));
            }
        }
    };
    load_window(0);
    for (int st = 0; st < nsteps; ++st) {
        __syncthreads(); // the previous window is consumed
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
#pragma unroll
            for (int t = 0; t < kRowMaxT; ++t) {
                const int e = t * 64 + lane;
                if (t < T && e < Wn) bw[(RW * wave + rr) * Wp + e] = v[rr][t];
            }
        __syncthreads();
        load_window(st + 1);
        const int c0 = (st % NC) * kRowCh;
        for (int k = 0; k < K; ++k) {
            const int kd = k * P.win_kd;
            const float *wt = wa + (k * NQ + c0 / 4) * MT * 64 + lane;
#pragma unroll
            for (int qq = 0; qq < kRowCh / 4; ++qq) {
                float a[MT], b[PB];
#pragma unroll
                for (int m = 0; m < MT; ++m) a[m] = wt[(qq * MT + m) * 64];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) b[pb] = bw[(4 * qq + c4) * Wp + col[pb] + kd];
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb)
                        acc[m][pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[pb], acc[m][pb], 0, 0, 0);
            }
        }
        if (st % NC == NC - 1) {
            // the tile is complete: lane j16 + 16*c4, register r holds
            // position j16, input channel 16m + 4*c4 + r
            const int p0 = (tile0 + st / NC) * TP;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                const int sp = p0 + wave * 16 * PB + pb * 16 + j16;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ci = g * P.Cig + ci0 + 16 * m + 4 * c4 + r;
                        if (sp < P.in_sp) dx[((int64_t)n * P.C_in + ci) * P.in_sp + sp] = acc[m][pb][r];
                    }
                    acc[m][pb] = bwd_v4f{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        }
    }
}

// The matrix kernel above reads its B operands from global memory, tap by
// tap; where a workgroup's dy rows do not stay in L2 between taps (the fused
// 3D layer: each dy element is fetched about six times per call), this
// variant stages them in LDS.  A workgroup owns R = 256 / W_in consecutive dx
// rows of one (sample, group, chunk of 16*CT input channels, D position):
// 4*CT waves, wave w holding channel tile w / 4 and 4 blocks of 16 positions
// ((w % 4) * 64 + 16 pb in the rows' row-major order).  It walks sub-steps
// (channel quad q, D tap kd); each stages the dy window of that quad and tap,
// 4 channels x NR rows x NW columns of one dy plane (zero outside the output:
// rows oh0 .. oh0 + NR - 1, columns -p_w .. -p_w + NW - 1), double buffered,
// the next window loaded into registers during the current one's MFMAs.  The
// quad's weights w[ci][4q .. 4q+3][taps] are copied to LDS once per quad
// (loaded during the previous quad).  Per tap, B (lane j + 16c: dy channel
// 4q + c at the position's tap output) and A are read from LDS.
//
// Thread t stages window elements t + 256*CT*u (u < 18/CT) at those LDS
// offsets; the buffer holds 4608 floats, so the writes need no bounds test.
// Each element's byte offset within its plane quad is fixed per workgroup and
// computed once (out of range where it lies outside the output or the
// window: the load reads zero); a sub-step adds the plane's offset as the
// scalar offset, or takes a resource of zero size where its D position lies
// outside the output.  The weights go the same way, 8 per thread (at most 32
// taps).  Above 32 taps (WSUB) the weights are staged per sub-step instead,
// w[ci][4q .. 4q+3][kd's K_h x K_w taps] (at most 16), double buffered with
// the window, and the window buffer holds 5120 floats.
constexpr int kBsWinCap = 4608;  // floats per window buffer
constexpr int kBsWinCap2 = 5120; // the same with weights per sub-step
constexpr int kBsWU = 8;         // weight-slice elements per thread
constexpr int kBsWsub = 2048;    // weight floats per sub-step buffer: 32 x 4 x 16 taps

struct BsParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, kvol;
    int in_sp, out_sp;
    int R, nhb, ccs, NQ;   // rows per workgroup, row blocks, channel chunks, quads
    int NR, NW;            // window rows, columns (the LDS pitch is NW)
    int win_sz;            // window floats: 4 * NR * NW <= kBsWinCap
};

template <int CT, int GEO, bool WSUB>
__global__ __launch_bounds__(256 * CT) __attribute__((amdgpu_waves_per_eu(1, 6))) void k_backward_data_stage(const BsParams P, const float *__restrict__ dy,
                                                                   const float *__restrict__ w,
                                                                   float *__restrict__ dx) {
    constexpr int CAP = WSUB ? kBsWinCap2 : kBsWinCap;
    constexpr int NT = 256 * CT, U = CAP / NT, PB = 4, WSU = kBsWsub / NT;
    static_assert(U * NT == CAP && WSU * NT == kBsWsub, "buffers split evenly over the threads");
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    // H and W geometry as constants, so that every window offset of a tap is
    // an immediate: GEO 1, W_in 16, stride 2, 3 taps and dilation 1 on both
    // (the fused layer's); GEO 2, W_in 32, stride 2, 4 taps and dilation 1
    // (the channel-heavy layer's); GEO 0, the plan's
    constexpr bool FIX = GEO != 0;
    constexpr int FW = GEO == 2 ? 32 : 16, FK = GEO == 2 ? 4 : 3;
    constexpr int FNR = (256 / FW - 1) * 2 + FK, FNW = (FW - 1) * 2 + FK;
    static_assert(GEO != 1 || !WSUB, "the fused geometry stages weights per quad");
    static_assert(GEO != 2 || WSUB, "the channel-heavy geometry stages weights per sub-step");
    const int WIN = FIX ? FW : AW.L_in;
    const int SH = FIX ? 2 : AH.s, SW = FIX ? 2 : AW.s, KH = FIX ? FK : AH.K, KW = FIX ? FK : AW.K;
    const int DH = FIX ? 1 : AH.d, DW = FIX ? 1 : AW.d;
    const int NR = FIX ? FNR : P.NR, NW = FIX ? FNW : P.NW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = wave >> 2, wq4 = wave & 3;
    const int j16 = lane & 15, c4 = lane >> 4;
    int64_t b = blockIdx.x;
    const int hb = (int)(b % P.nhb);
    b /= P.nhb;
    const int id = (int)(b % AD.L_in);
    b /= AD.L_in;
    const int cc = (int)(b % P.ccs);
    b /= P.ccs;
    const int g = (int)(b % (P.C_in / P.Cig));
    const int n = (int)(b / (P.C_in / P.Cig));
    const int ih0 = hb * P.R;
    const int ci0 = g * P.Cig + cc * 16 * CT;
    const int od0 = id * AD.s - AD.p, oh0 = ih0 * SH - AH.p, ow0 = -AW.p;
    const int KHW = KH * KW, nsub = P.NQ * AD.K;

    extern __shared__ __attribute__((aligned(16))) float lds_bs[];
    float *win0 = lds_bs, *win1 = lds_bs + CAP, *wq = lds_bs + 2 * CAP, *wq1 = wq + kBsWsub;

    // window element e = tid + NT*u: channel c, row rr, column col; its byte
    // offset from the plane quad's start, or out of range
    unsigned voff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = tid + u * NT;
        const int c = e / (NR * NW), rem = e - c * (NR * NW);
        const int rr = rem / NW, col = rem - rr * NW;
        const int oh = oh0 + rr, ow = ow0 + col;
        const bool ok = e < 4 * NR * NW && oh >= 0 && oh < AH.L_out && ow >= 0 && ow < AW.L_out;
        voff[u] = ok ? 4u * (unsigned)(c * P.out_sp + oh * AW.L_out + ow) : kBwdOutOfRange;
    }
    const int dy_bytes = 4 * P.C_out * P.out_sp;
    float *dyn = const_cast<float *>(dy + (int64_t)n * P.C_out * P.out_sp);
    const bwd_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(dyn, (short)0, dy_bytes, kBwdRsrcWord3);
    const bwd_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc(dyn, (short)0, 0, kBwdRsrcWord3);
    // window of sub-step ss = (q, kd) into registers (zeros outside the output)
    auto fetch = [&](float (&pf)[U], int ss) __attribute__((always_inline)) {
        const int q = ss / AD.K, kd = ss - q * AD.K;
        const int od = od0 + kd * AD.d;
        const bool odok = ss < nsub && od >= 0 && od < AD.L_out;
        const bwd_rsrc_t r = odok ? rdy : rnone;
        const int soff = odok ? 4 * ((g * P.Cog + 4 * q) * P.out_sp + od * AH.L_out * AW.L_out) : 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            pf[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff[u], soff, 0));
    };
    auto stage = [&](float *wb, const float (&pf)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) wb[tid + u * NT] = pf[u];
    };
    // weight element e = tid + NT*u: input channel cil, [c][k] index rem of
    // w[ci0 + cil][4q + c][k] (per sub-step: k = kd*KHW + t); byte offset
    // from w[ci0][4q][0] (out of range past the slice)
    constexpr int WN = WSUB ? WSU : kBsWU;
    const int wsl = WSUB ? KHW : P.kvol; // taps per channel in a slice
    unsigned woff[WN];
#pragma unroll
    for (int u = 0; u < WN; ++u) {
        const int e = tid + u * NT;
        const int cil = e / (4 * wsl), rem = e - cil * (4 * wsl);
        const int c = rem / wsl, t = rem - c * wsl;
        woff[u] = e < 16 * CT * 4 * wsl ? 4u * (unsigned)(cil * P.Cog * P.kvol + c * P.kvol + t) : kBwdOutOfRange;
    }
    const bwd_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(w + (int64_t)ci0 * P.Cog * P.kvol), (short)0, 4 * 16 * CT * P.Cog * P.kvol, kBwdRsrcWord3);
    float wpf[WN];
    // weights of quad q (per quad) or of sub-step q = (quad, kd) (per sub-step)
    auto fetch_w = [&](int q) __attribute__((always_inline)) {
        int soff;
        if constexpr (WSUB) {
            const int qq = min(q, nsub - 1), quad = qq / AD.K, kd = qq - quad * AD.K;
            soff = 16 * quad * P.kvol + 4 * kd * KHW;
        } else {
            soff = 16 * min(q, P.NQ - 1) * P.kvol;
        }
#pragma unroll
        for (int u = 0; u < WN; ++u)
            wpf[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, woff[u], soff, 0));
    };
    auto stage_w = [&](float *wqb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < WN; ++u) wqb[tid + u * NT] = wpf[u];
    };

    // per block pb of this wave: row r and first column, so the B address is
    // bpos[pb] + (kh*dh)*NW + kw*dw within the channel's window
    int bpos[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
        const int blk = wq4 * PB + pb;
        const int r = (blk * 16) / WIN, col0 = (blk * 16) - r * WIN;
        bpos[pb] = (c4 * NR + r * SH) * NW + (col0 + j16) * SW;
    }
    const int abase = ((16 * m + j16) * 4 + c4) * (WSUB ? KHW : P.kvol);
    bwd_v4f acc[PB];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) acc[pb] = bwd_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    float pf[U];
    fetch_w(0);
    fetch(pf, 0);
    stage_w(wq);
    stage(win0, pf);
    fetch(pf, 1);
    fetch_w(1);
    __syncthreads();
    for (int ss = 0; ss < nsub; ++ss) {
        const int kd = ss % AD.K;
        const float *wb = (ss & 1) ? win1 : win0;
        // the A operands: this sub-step's buffer, or the quad's slice at kd
        const float *wqa = WSUB ? ((ss & 1) ? wq1 : wq) : wq + kd * KHW;
        // taps (kd, kh, kw) in order, two operand sets: the reads of tap t + 1
        // are in flight during tap t's products.  (k, kw, toff) walk the taps
        // with scalar steps.  With an even tap count the last reads are of
        // the tap after the last (row K_h, column 0; weight index k = kvol at
        // the last kd), never used: they stay within d_h * NW floats past the
        // window buffer and one past the weight slice, which the allocation
        // pads.
        auto mma = [&](const float a, const float (&bb)[PB]) __attribute__((always_inline)) {
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
                acc[pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb[pb], acc[pb], 0, 0, 0);
        };
        if constexpr (FIX) {
            // FK x FK taps unrolled (window offsets are constants past
            // bpos[pb]), the operands of tap t + 1 read before tap t's products
            constexpr int NTAP = FK * FK;
            float a[NTAP], bb[2][PB];
#pragma unroll
            for (int t = 0; t < NTAP; ++t) a[t] = wqa[abase + t];
#pragma unroll
            for (int t = 0; t < NTAP; ++t) {
                if (t == 0) {
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) bb[0][pb] = wb[bpos[pb]];
                }
                if (t + 1 < NTAP) {
                    const int kh = (t + 1) / FK, kw = (t + 1) - FK * ((t + 1) / FK);
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) bb[(t + 1) & 1][pb] = wb[bpos[pb] + kh * NW + kw];
                }
                mma(a[t], bb[t & 1]);
            }
            // issue order: the A reads and tap 0's B reads, then per tap the
            // two B reads of the next tap before its four products (the A
            // reads pair up: 5 instructions for 9, 8 for 16)
            __builtin_amdgcn_sched_group_barrier(0x100, (NTAP + 1) / 2 + 2, 0);
#pragma unroll
            for (int t = 0; t < NTAP - 1; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        } else {
            int k = 0, kw = 0, toff = 0;
            auto next = [&]() __attribute__((always_inline)) {
                const bool row_end = kw == KW - 1;
                toff += row_end ? DH * NW - (KW - 1) * DW : DW;
                kw = row_end ? 0 : kw + 1;
                ++k;
            };
            auto rd = [&](float &a, float (&bb)[PB]) __attribute__((always_inline)) {
                a = wqa[abase + k];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) bb[pb] = wb[bpos[pb] + toff];
            };
            float a0, b0[PB], a1, b1[PB];
            rd(a0, b0);
            int t = 0;
            for (; t + 2 <= KHW; t += 2) {
                next();
                rd(a1, b1);
                mma(a0, b0);
                next();
                rd(a0, b0);
                mma(a1, b1);
            }
            if (t < KHW) mma(a0, b0);
        }
        if constexpr (WSUB) {
            // the next window and weights into the other buffers (read last
            // in sub-step ss - 1)
            stage((ss & 1) ? win0 : win1, pf);
            stage_w((ss & 1) ? wq : wq1);
            fetch_w(ss + 2);
        } else {
            const bool quad_end = kd == AD.K - 1;
            if (quad_end) __syncthreads(); // every wave is done with this quad's weights
            // the next window into the other buffer (read last in sub-step ss - 1)
            stage((ss & 1) ? win0 : win1, pf);
            if (quad_end) {
                stage_w(wq);
                fetch_w(ss / AD.K + 2);
            }
        }
        fetch(pf, ss + 2);
        __syncthreads();
    }

    // lane j16 + 16*c4, register v: position j16 of block pb, input channel
    // 16m + 4*c4 + v
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
        const int blk = wq4 * PB + pb;
        const int r = (blk * 16) / WIN, col0 = (blk * 16) - r * WIN;
        if (ih0 + r >= AH.L_in) continue;
        const int sp = (id * AH.L_in + ih0 + r) * WIN + col0 + j16;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            dx[((int64_t)n * P.C_in + ci0 + 16 * m + 4 * c4 + v) * P.in_sp + sp] = acc[pb][v];
    }
}

// LDS floats of one workgroup: two window buffers, the weight slice (NT *
// kBsWU) or the two per-sub-step weight buffers, and the pad past them that
// the last tap's unused reads may touch.
inline size_t stage_lds_floats(int ct, bool wsub, int dh, int NW) {
    return wsub ? 2 * (size_t)kBsWinCap2 + 2 * (size_t)kBsWsub + (size_t)dh * NW + 1
                : 2 * (size_t)kBsWinCap + (size_t)256 * ct * kBsWU + (size_t)dh * NW + 1;
}

// The staged variant applies: 2D or 3D plans with groups of 32k input and 4k
// output channels (two channel tiles per workgroup; with one, each dy window
// would be staged once per 16 channels and the matrix kernel is faster),
// W_in of 16, 32 or 64, and the buffers within 64 KB of LDS; up to 32 taps
// with the quad's weights staged once (a window of at most kBsWinCap floats),
// up to 64 with at most 16 per D tap staged per sub-step (kBsWinCap2).
// Returns 1 (weights per quad), 2 (per sub-step) or 0 when it does not apply;
// fills the window fields of P.
int stage_mode(const convt_plan &Pl, BsParams &P) {
    const AxisPlan &AH = Pl.ax[1], &AW = Pl.ax[2];
    if (Pl.ndim < 2 || Pl.Cig % 32 != 0 || Pl.Cog % 4 != 0 || Pl.k_vol > 64) return 0;
    const bool wsub = Pl.k_vol > 32;
    if (wsub && AH.K * AW.K > 16) return 0;
    if (AW.L_in != 16 && AW.L_in != 32 && AW.L_in != 64) return 0;
    if (4 * Pl.C_out * Pl.out_sp > 0x7fffffff || Pl.N * Pl.C_in * Pl.in_sp > ((int64_t)1 << 40)) return 0;
    if (4 * 32 * Pl.Cog * Pl.k_vol > 0x7fffffff) return 0; // a chunk's weights in one buffer resource
    P.R = 256 / AW.L_in;
    P.NR = (P.R - 1) * AH.s + (AH.K - 1) * AH.d + 1;
    P.NW = (AW.L_in - 1) * AW.s + (AW.K - 1) * AW.d + 1;
    P.win_sz = 4 * P.NR * P.NW;
    if (P.win_sz > (wsub ? kBsWinCap2 : kBsWinCap)) return 0;
    if (4 * stage_lds_floats(2, wsub, AH.d, P.NW) > 65536) return 0;
    return wsub ? 2 : 1;
}

template <int CT>
int launch_stage(const convt_plan &Pl, BsParams &P, bool wsub, const float *dy, const float *w, float *dx,
                 hipStream_t st) {
    const AxisPlan &AH = Pl.ax[1], &AW = Pl.ax[2];
    const bool fix = AW.L_in == 16 && AH.s == 2 && AW.s == 2 && AH.K == 3 && AW.K == 3 && AH.d == 1 && AW.d == 1;
    const bool fix2 = AW.L_in == 32 && AH.s == 2 && AW.s == 2 && AH.K == 4 && AW.K == 4 && AH.d == 1 && AW.d == 1;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.Cig = (int)Pl.Cig;
    P.Cog = (int)Pl.Cog;
    P.kvol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    P.nhb = (Pl.ax[1].L_in + P.R - 1) / P.R;
    P.ccs = (int)(Pl.Cig / (16 * CT));
    P.NQ = (int)(Pl.Cog / 4);
    const int64_t blocks = Pl.N * Pl.G * (int64_t)P.ccs * Pl.ax[0].L_in * P.nhb;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    const size_t lds = 4 * stage_lds_floats(CT, wsub, P.ax[1].d, P.NW);
    const dim3 grid((unsigned)blocks), blk(256 * CT);
    if (wsub) {
        if (fix2)
            hipLaunchKernelGGL((k_backward_data_stage<CT, 2, true>), grid, blk, lds, st, P, dy, w, dx);
        else
            hipLaunchKernelGGL((k_backward_data_stage<CT, 0, true>), grid, blk, lds, st, P, dy, w, dx);
    } else {
        if (fix)
            hipLaunchKernelGGL((k_backward_data_stage<CT, 1, false>), grid, blk, lds, st, P, dy, w, dx);
        else
            hipLaunchKernelGGL((k_backward_data_stage<CT, 0, false>), grid, blk, lds, st, P, dy, w, dx);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

// Groups of 8 input and 8 output channels with stride 2 and dilation 1 along
// W and stride 1, dilation 1 along H (the grouped 3D layer), where the matrix
// kernel above does not apply and the gather runs on the vector ALUs.  The two
// W phases of each pair of input positions share one tile, as in the forward
// W-pair kernel: rows (sigma, ci) hold dx at W position 2j + sigma, columns
// are 16 pairs j.  Position 2j + sigma meets tap kw at output 4j + 2 sigma -
// p + kw, so for a dy shift c the B operand dy[co][4j + c] serves row sigma
// with tap kw = c + p - 2 sigma (zero where that tap does not exist), and
// c over [-p, K_w - p + 2) covers every tap of both phases.  A wave owns kBpRows
// consecutive dx rows along H: dy row oh feeds row ih through tap
// kh = oh - ih + p_h, so each B operand it loads serves up to kBpRows MFMAs.
// The group's weights are copied to LDS once per workgroup (coalesced) and
// the A operands read from there.  Steps (kd, c, channel quad) run with the
// next step's operands loaded during the current step's MFMAs (two register
// sets, every load issued; out-of-range offsets read zero).  dx is stored
// once per element, 32 consecutive floats per store instruction.
constexpr int kBpRows = 4;
constexpr int kBpMaxKvol = 192; // KD*KH*KW whose group weights fit the LDS copy
constexpr int kBpWPer = 8 * 8 * kBpMaxKvol / 4 / kBwdBlock; // weight float4 per thread at most

struct BpParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, G, kvol;
    int in_sp, out_sp;
    int nwt, nhb;      // W tiles of 32 positions, H blocks of kBpRows rows
    int per_ng;        // wave units per (sample, group): D_in * nhb * nwt
    int blocks_per_ng; // workgroups per (sample, group)
};

template <int KH>
__global__ __launch_bounds__(kBwdBlock) void k_backward_data_wpair(const BpParams P, const float *__restrict__ dy,
                                                                   const float *__restrict__ w,
                                                                   float *__restrict__ dx) {
    constexpr int NR = KH + kBpRows - 1; // dy rows a wave's dx rows reach
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    __shared__ __attribute__((aligned(16))) float wl[8 * 8 * kBpMaxKvol];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ng = blockIdx.x / P.blocks_per_ng;
    const int g = ng % P.G, n = ng / P.G;

    // the group's weights [ci][co][kd][kh][kw], contiguous
    {
        const int n4 = 8 * 8 * P.kvol / 4;
        const bwd_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(w + (int64_t)g * 64 * P.kvol),
                                                                (short)0, 4 * 64 * P.kvol, kBwdRsrcWord3);
        bwd_v4f tw[kBpWPer]; // every load in flight before the first write
#pragma unroll
        for (int u = 0; u < kBpWPer; ++u) {
            const int i = tid + u * kBwdBlock;
            tw[u] = __builtin_bit_cast(bwd_v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rw, i < n4 ? 16u * (unsigned)i : kBwdOutOfRange, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < kBpWPer; ++u) {
            const int i = tid + u * kBwdBlock;
            if (i < n4) *reinterpret_cast<bwd_v4f *>(wl + 4 * i) = tw[u];
        }
    }
    __syncthreads();
    const int unit = (blockIdx.x - ng * P.blocks_per_ng) * 4 + wave;
    if (unit >= P.per_ng) return; // no barrier after this point
    const int jt = unit % P.nwt;
    const int hb = (unit / P.nwt) % P.nhb;
    const int id = unit / (P.nwt * P.nhb);
    const int ih0 = hb * kBpRows;

    const int j = lane & 15, c4 = lane >> 4;
    const int sig = j >> 3, ci = j & 7; // A row (sigma, ci) of this lane: row index j
    const bwd_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + ((int64_t)n * P.C_out + (int64_t)g * 8) * P.out_sp), (short)0, 4 * 8 * P.out_sp,
        kBwdRsrcWord3);
    const int NC = AW.K + 2;
    const int nsteps = AD.K * NC * 2;
    const int KW = AW.K;

    // operands of step st = (kd, c, q): A[kh] and B[r]
    auto load = [&](int st, bool live, float (&a)[KH], float (&b)[NR]) __attribute__((always_inline)) {
        const int q = st & 1, t = st >> 1;
        const int kd = t / NC, c = t - kd * NC - AW.p;
        // A: w[ci][4q + c4][kd][kh][kw], kw = c + p - 2 sigma
        const int kw = c + AW.p - 2 * sig;
        const bool aok = live & (kw >= 0) & (kw < KW);
        const int abase = ((ci * 8 + 4 * q + c4) * AD.K + kd) * KH * KW + (aok ? kw : 0);
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
            const float v = wl[abase + kh * KW];
            a[kh] = aok ? v : 0.0f;
        }
        // B: dy[4q + c4][od][ih0 - p_h + r][4(16 jt + j) + c]
        const int od = id * AD.s - AD.p + kd * AD.d;
        const int ow = 4 * (16 * jt + j) + c;
        const bool cok = (od >= 0) & (od < AD.L_out) & (ow >= 0) & (ow < AW.L_out);
        const int cbase = (4 * q + c4) * P.out_sp + od * AH.L_out * AW.L_out + ow;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int oh = ih0 - AH.p + r;
            const bool ok = cok & (oh >= 0) & (oh < AH.L_out);
            const unsigned off = ok ? 4u * (unsigned)(cbase + oh * AW.L_out) : kBwdOutOfRange;
            b[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, off, 0, 0));
        }
    };
    bwd_v4f acc[kBpRows];
#pragma unroll
    for (int h = 0; h < kBpRows; ++h) acc[h] = bwd_v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const float (&a)[KH], const float (&b)[NR]) __attribute__((always_inline)) {
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
            for (int h = 0; h < kBpRows; ++h)
                acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kh], b[h + kh], acc[h], 0, 0, 0);
    };
    // two register sets in turn; a step past the last loads the last again
    // with A = 0
    float a0[KH], a1[KH], b0[NR], b1[NR];
    load(0, true, a0, b0);
    for (int st = 0; st < nsteps; st += 2) {
        load(min(st + 1, nsteps - 1), st + 1 < nsteps, a1, b1);
        compute(a0, b0);
        load(min(st + 2, nsteps - 1), st + 2 < nsteps, a0, b0);
        compute(a1, b1);
    }

    // lane j + 16 c4, register v: row i = 4 c4 + v = (sigma, ci): dx[ci][ih][2(16 jt + j) + sigma]
    const bwd_rsrc_t rdx = __builtin_amdgcn_make_buffer_rsrc(dx + ((int64_t)n * P.C_in + (int64_t)g * 8) * P.in_sp,
                                                             (short)0, 4 * 8 * P.in_sp, kBwdRsrcWord3);
    const int iw = 2 * (16 * jt + j) + (c4 >> 1);
#pragma unroll
    for (int h = 0; h < kBpRows; ++h) {
        const int ih = ih0 + h;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int cio = 4 * (c4 & 1) + v;
            const bool ok = (ih < AH.L_in) & (iw < AW.L_in);
            const unsigned off = ok ? 4u * (unsigned)(cio * P.in_sp + (id * AH.L_in + ih) * AW.L_in + iw)
                                    : kBwdOutOfRange;
            // (through a VGPR: passed straight from the accumulator registers,
            // this compiler stored component 0 for every v)
            float val = acc[h][v];
            asm volatile("" : "+v"(val));
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, val), rdx, off, 0, 0);
        }
    }
}

// The W-pair kernel applies: groups of 8 and 8 channels, stride 2 and dilation
// 1 along W, stride 1 and dilation 1 along H, at most 7 H taps, the group's
// weights within the LDS copy, and a group's x and dy below 2 GiB.
bool bwd_wpair_applies(const convt_plan &P) {
    const AxisPlan &AH = P.ax[1], &AW = P.ax[2];
    return P.Cig == 8 && P.Cog == 8 && AW.s == 2 && AW.d == 1 && AH.s == 1 && AH.d == 1 && AH.K <= 7 &&
           P.k_vol <= kBpMaxKvol && 4 * 8 * P.in_sp <= 0x7fffffff && 4 * 8 * P.out_sp <= 0x7fffffff;
}

int launch_bwd_wpair(const convt_plan &Pl, const float *dy, const float *w, float *dx, hipStream_t st) {
    BpParams P;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.G = (int)Pl.G;
    P.kvol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    P.nwt = (Pl.ax[2].L_in + 31) / 32;
    P.nhb = (Pl.ax[1].L_in + kBpRows - 1) / kBpRows;
    P.per_ng = Pl.ax[0].L_in * P.nhb * P.nwt;
    P.blocks_per_ng = (P.per_ng + 3) / 4;
    const int64_t blocks = Pl.N * Pl.G * (int64_t)P.blocks_per_ng;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    auto go = [&](auto khc) {
        hipLaunchKernelGGL((k_backward_data_wpair<decltype(khc)::value>), dim3((unsigned)blocks), dim3(kBwdBlock), 0,
                           st, P, dy, w, dx);
    };
    switch (Pl.ax[1].K) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    default: go(std::integral_constant<int, 7>{}); break;
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

constexpr int kBwdPB = 4; // 16-position blocks per wave

// Row tiles per wave for the matrix kernel (0: it does not apply).  Needs
// groups of 16k input and 4k output channels, one tap's A rows within the
// staging budget, and a group's dy below 2 GiB (buffer offsets).
int pick_mt(const convt_plan &P) {
    if (P.Cig % 16 != 0 || P.Cog % 4 != 0) return 0;
    if (4 * P.Cog * P.out_sp > 0x7fffffff) return 0;
    for (int mt = 4; mt >= 1; mt /= 2)
        if ((P.Cig / 16) % mt == 0 && (int64_t)(P.Cog / 4) * mt * 64 * 4 <= kBwdMaxLds) return mt;
    return 0;
}

// Input channels per thread: as many as the group has, up to 16, while one
// tap's weights for them (C_out/G x CPI floats) fit in LDS.
int pick_cpi(const convt_plan &P) {
    for (int c = 16; c >= 1; c /= 2)
        if ((c <= P.Cig || c == 1) && (int64_t)P.Cog * c * 4 <= kBwdMaxLds) return c;
    return 0;
}

template <int CPI>
int launch(const convt_plan &Pl, BwdParams &P, const float *dy, const float *w, float *dx, hipStream_t st) {
    P.ci_chunks = (int)((Pl.Cig + CPI - 1) / CPI);
    const int64_t per_tap = Pl.Cog * CPI * (int64_t)sizeof(float);
    P.taps_per_chunk = (int)(kBwdMaxLds / per_tap < Pl.k_vol ? kBwdMaxLds / per_tap : Pl.k_vol);
    const unsigned gx = (unsigned)((Pl.in_sp + kBwdBlock - 1) / kBwdBlock);
    const unsigned gy = (unsigned)(Pl.G * P.ci_chunks);
    const size_t lds = (size_t)(P.taps_per_chunk * per_tap);
    for (int64_t n0 = 0; n0 < Pl.N; n0 += 65535) {
        P.n0 = (int)n0;
        const unsigned gz = (unsigned)(Pl.N - n0 < 65535 ? Pl.N - n0 : 65535);
        hipLaunchKernelGGL((k_backward_data<CPI>), dim3(gx, gy, gz), dim3(kBwdBlock), lds, st, P, dy, w, dx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

template <int MT>
int launch_mfma(const convt_plan &Pl, BwdParams &P, const float *dy, const float *w, float *dx, hipStream_t st) {
    P.ci_chunks = (int)(Pl.Cig / (16 * MT));
    const int64_t per_tap = (Pl.Cog / 4) * MT * 64 * (int64_t)sizeof(float);
    P.taps_per_chunk = (int)(kBwdMaxLds / per_tap < Pl.k_vol ? kBwdMaxLds / per_tap : Pl.k_vol);
    const unsigned gx = (unsigned)((Pl.in_sp + 64 * kBwdPB - 1) / (64 * kBwdPB));
    const unsigned gy = (unsigned)(Pl.G * P.ci_chunks);
    const size_t lds = (size_t)(P.taps_per_chunk * per_tap);
    for (int64_t n0 = 0; n0 < Pl.N; n0 += 65535) {
        P.n0 = (int)n0;
        const unsigned gz = (unsigned)(Pl.N - n0 < 65535 ? Pl.N - n0 : 65535);
        hipLaunchKernelGGL((k_backward_data_mfma<MT, kBwdPB>), dim3(gx, gy, gz), dim3(kBwdBlock), lds, st, P, dy,
                           w, dx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

// The one-axis window variant applies: a 1D plan (unit leading axes), the
// matrix kernel's channel counts, output channels in whole window chunks, and
// every tap's A rows plus a kRowCh-row window within 64 KB of LDS.  Fills
// the window fields of P and returns true when it applies.  The row pitch is
// odd, so the rows one MFMA operand reads start on different banks.
bool row_window(const convt_plan &Pl, int mt, BwdParams &P) {
    if (mt == 0 || Pl.Cog % kRowCh != 0) return false;
    // A leading axis must be a unit axis whose one tap lands on its one output
    // (p = 0 and L_out = 1): the window kernels index only the last axis.
    for (int a = 0; a < 2; ++a)
        if (Pl.ax[a].L_in != 1 || Pl.ax[a].K != 1 || Pl.ax[a].p != 0 || Pl.ax[a].L_out != 1) return false;
    const AxisPlan &A = Pl.ax[2];
    const int cs = A.d % A.s == 0 ? A.s : 1;
    const int64_t wn = (int64_t)(64 * kBwdPB - 1) * (A.s / cs) + (int64_t)(A.K - 1) * (A.d / cs) + 1;
    if (wn > 64 * kRowMaxT) return false;
    const int64_t wp = wn | 1;
    const int64_t a_bytes = (int64_t)Pl.k_vol * (Pl.Cog / 4) * mt * 64 * 4;
    if (a_bytes > kBwdMaxLds || a_bytes + kRowCh * wp * 4 > 65536) return false;
    P.win_pitch = (int)wp;
    P.win_cols = (int)wn;
    P.win_cs = cs;
    P.win_js = A.s / cs;
    P.win_kd = A.d / cs;
    return true;
}

template <int MT>
int launch_mfma_row(const convt_plan &Pl, BwdParams &P, const float *dy, const float *w, float *dx,
                    hipStream_t st) {
    P.ci_chunks = (int)(Pl.Cig / (16 * MT));
    // enough tiles per workgroup to amortise staging the A rows, while the
    // grid keeps at least kRowMinWgs workgroups
    const int64_t ntiles = (Pl.in_sp + 64 * kBwdPB - 1) / (64 * kBwdPB);
    const int64_t per_tile = Pl.N * Pl.G * P.ci_chunks;
    int64_t tpw = ntiles * per_tile / kRowMinWgs;
    P.tiles_per_wg = (int)(tpw < 1 ? 1 : tpw > kRowMaxTilesPerWg ? kRowMaxTilesPerWg : tpw);
    const unsigned gx = (unsigned)((ntiles + P.tiles_per_wg - 1) / P.tiles_per_wg);
    const unsigned gy = (unsigned)(Pl.G * P.ci_chunks);
    const size_t lds = (size_t)(Pl.k_vol * (Pl.Cog / 4) * MT * 64 + kRowCh * P.win_pitch) * sizeof(float);
    for (int64_t n0 = 0; n0 < Pl.N; n0 += 65535) {
        P.n0 = (int)n0;
        const unsigned gz = (unsigned)(Pl.N - n0 < 65535 ? Pl.N - n0 : 65535);
        hipLaunchKernelGGL((k_backward_data_mfma_row<MT, kBwdPB>), dim3(gx, gy, gz), dim3(kBwdBlock), lds, st, P,
                           dy, w, dx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

} // namespace

const char *backward_data_kernel_name(const convt_plan &P) {
    const int mt = pick_mt(P);
    BwdParams W;
    if (row_window(P, mt, W)) return "k_backward_data_mfma_row";
    if (mt == 0 && bwd_wpair_applies(P)) return "k_backward_data_wpair";
    BsParams S;
    if (CONVT_BWD_STAGE && mt > 0 && stage_mode(P, S) > 0) return "k_backward_data_stage";
    return mt > 0 ? "k_backward_data_mfma" : "k_backward_data";
}

bool backward_data_supports(const convt_plan &P) {
    const int c = pick_cpi(P);
    return c > 0 && P.G * ((P.Cig + c - 1) / c) <= 65535;
}

int launch_backward_data(const convt_plan &Pl, const float *dy, const float *w, float *dx, void *stream) {
    BwdParams P;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.Cig = (int)Pl.Cig;
    P.Cog = (int)Pl.Cog;
    P.k_vol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    hipStream_t st = (hipStream_t)stream;
    const int mt = pick_mt(Pl);
    if (row_window(Pl, mt, P)) {
        switch (mt) {
        case 4: return launch_mfma_row<4>(Pl, P, dy, w, dx, st);
        case 2: return launch_mfma_row<2>(Pl, P, dy, w, dx, st);
        default: return launch_mfma_row<1>(Pl, P, dy, w, dx, st);
        }
    }
    BsParams S;
    if (CONVT_BWD_STAGE && mt > 0) {
        const int mode = stage_mode(Pl, S);
        if (mode > 0) return launch_stage<2>(Pl, S, mode == 2, dy, w, dx, st);
    }
    switch (mt) {
    case 4: return launch_mfma<4>(Pl, P, dy, w, dx, st);
    case 2: return launch_mfma<2>(Pl, P, dy, w, dx, st);
    case 1: return launch_mfma<1>(Pl, P, dy, w, dx, st);
    default: break;
    }
    if (bwd_wpair_applies(Pl)) return launch_bwd_wpair(Pl, dy, w, dx, st);
    switch (pick_cpi(Pl)) {
    case 16: return launch<16>(Pl, P, dy, w, dx, st);
    case 8: return launch<8>(Pl, P, dy, w, dx, st);
    case 4: return launch<4>(Pl, P, dy, w, dx, st);
    case 2: return launch<2>(Pl, P, dy, w, dx, st);
    default: return launch<1>(Pl, P, dy, w, dx, st);
    }
}

} // namespace convt
