// Weight and bias gradients of the transposed convolution.  The forward is
// linear in w: x[n, ci, i] * w[ci, co_l, k] lands on y[n, g*Cog + co_l, o]
// with o = i*s - p + k*d per axis, so for an output gradient dy
//   dw[ci, co_l, k] = sum over n and the inputs i whose o lies in [0, L_out)
//                     of x[n, ci, i] * dy[n, g*Cog + co_l, o]
//   db[co]          = sum over n and every output position of dy[n, co, o].
// Same sources as the forward ("Kimi-K2.6 l1_p79" transcript, the scatter
// definition; "Kimi-K2.6 l1_p72" transcript, the per-group loop with bias).
//
// Per tap k the weight gradient is a GEMM over positions: dW_k = X * DY_k^T
// with X (C_in/G x positions) and DY_k[p][co] = dy[co][o(p, k)].  It runs on
// v_mfma_f32_16x16x4_f32 with K = 4 input positions: A (lane i + 16c) =
// x[ci0 + i][p_c], B (lane j + 16c) = dy[co0 + j][o(p_c, k)], D (lane
// j + 16(i/4), register i%4) = the partial dW_k[ci0 + i][co0 + j].  A wave
// owns CTW input-channel tiles x OTW output-channel tiles x up to TK taps over
// one range of positions of one batch sample; each lane walks its own
// position four at a time, so the tap offsets need no division.  Tiles past
// the group's channels load zeros and are not stored, so any channel counts
// run.  The partial sums of all ranges are added into dw with fp32 atomics
// (dw is cleared first, in the same call): the result is the sum in some order,
// so it varies in the last bits from run to run.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "wgrad.h"

namespace convt {
namespace {

typedef float wg_v4f __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t wg_rsrc_t;
constexpr int kWgRsrcWord3 = 0x00020000; // raw (untyped) buffer access
constexpr unsigned kWgOutOfRange = 0x80000000u;
constexpr int kWgBlock = 256;  // four waves, each its own unit
constexpr int kWgRange = 1024; // input positions per wave (256 steps of 4)
// Tuning knob: the LDS-staged weight kernel where it applies.
#ifndef CONVT_WT_STAGE
#define CONVT_WT_STAGE 1
#endif

struct WgradParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, k_vol;
    int in_sp, out_sp;
    int CT, OT;        // 16-channel tiles of the group (input, output)
    int kchunks;       // chunks of TK taps
    int nranges;       // position ranges per sample
    int64_t units;     // waves of work
};

template <int CTW, int OTW, int TK>
__global__ __launch_bounds__(kWgBlock) void k_backward_weight(const WgradParams P, const float *__restrict__ x,
                                                              const float *__restrict__ dy, float *dw) {
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * (kWgBlock / 64) + (threadIdx.x >> 6);
    if (unit >= P.units) return; // no barrier in this kernel: a wave may leave early
    int64_t t = unit;
    const int range = (int)(t % P.nranges);
    t /= P.nranges;
    const int kc = (int)(t % P.kchunks);
    t /= P.kchunks;
    const int otw = (int)(t % (P.OT / OTW));
    t /= P.OT / OTW;
    const int ctw = (int)(t % (P.CT / CTW));
    t /= P.CT / CTW;
    const int g = (int)(t % (P.C_in / P.Cig));
    const int n = (int)(t / (P.C_in / P.Cig));
    const int ci0 = ctw * CTW * 16, co0 = otw * OTW * 16;
    const int k0 = kc * TK, tk = min(TK, P.k_vol - k0);

    const int i16 = lane & 15, c4 = lane >> 4;
    // this lane's A rows (input channel ci0 + 16m + i16) and B columns
    // (output channel co0 + 16o + i16); c4 is its position within the step
    const wg_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig) * P.in_sp), (short)0,
        (int)(4 * P.Cig * P.in_sp), kWgRsrcWord3);
    const wg_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + ((int64_t)n * P.C_out + (int64_t)g * P.Cog) * P.out_sp), (short)0,
        (int)(4 * P.Cog * P.out_sp), kWgRsrcWord3);
    bool a_ok[CTW], b_ok[OTW];
    unsigned a_ch[CTW], b_ch[OTW];
#pragma unroll
    for (int m = 0; m < CTW; ++m) {
        a_ok[m] = ci0 + 16 * m + i16 < P.Cig;
        a_ch[m] = (unsigned)(ci0 + 16 * m + i16) * (unsigned)P.in_sp;
    }
#pragma unroll
    for (int o = 0; o < OTW; ++o) {
        b_ok[o] = co0 + 16 * o + i16 < P.Cog;
        b_ch[o] = (unsigned)(co0 + 16 * o + i16) * (unsigned)P.out_sp;
    }
    // the taps of this chunk: output offset and per-axis tap shifts
    int tkd[TK], tkh[TK], tkw[TK];
#pragma unroll
    for (int u = 0; u < TK; ++u) {
        const int k = k0 + min(u, tk - 1);
        const int kw = k % AW.K, kdh = k / AW.K;
        tkw[u] = kw * AW.d;
        tkh[u] = (kdh % AH.K) * AH.d;
        tkd[u] = (kdh / AH.K) * AD.d;
    }

    wg_v4f acc[TK][CTW][OTW];
#pragma unroll
    for (int u = 0; u < TK; ++u)
#pragma unroll
        for (int m = 0; m < CTW; ++m)
#pragma unroll
            for (int o = 0; o < OTW; ++o) acc[u][m][o] = wg_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // this lane's position: p = range*kWgRange + 4*step + c4
    const int p_begin = range * kWgRange;
    const int p_end = min(p_begin + kWgRange, P.in_sp);
    int p = p_begin + c4;
    int iw = p % AW.L_in, ih = (p / AW.L_in) % AH.L_in, id = p / (AW.L_in * AH.L_in);
    for (int step = p_begin; step < p_end; step += 4) {
        const bool live = p < p_end;
        // A: x[ci][p]
        float a[CTW];
#pragma unroll
        for (int m = 0; m < CTW; ++m) {
            const unsigned vo = live && a_ok[m] ? 4u * (a_ch[m] + (unsigned)p) : kWgOutOfRange;
            a[m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, vo, 0, 0));
        }
        const int bd = id * AD.s - AD.p, bh = ih * AH.s - AH.p, bw = iw * AW.s - AW.p;
#pragma unroll
        for (int u = 0; u < TK; ++u) {
            if (u >= tk) break;
            const int od = bd + tkd[u], oh = bh + tkh[u], ow = bw + tkw[u];
            const bool ok = live && od >= 0 && od < AD.L_out && oh >= 0 && oh < AH.L_out && ow >= 0 &&
                            ow < AW.L_out;
            const unsigned o_sp = (unsigned)((od * AH.L_out + oh) * AW.L_out + ow);
            float b[OTW];
#pragma unroll
            for (int o = 0; o < OTW; ++o) {
                const unsigned vo = ok && b_ok[o] ? 4u * (b_ch[o] + o_sp) : kWgOutOfRange;
                b[o] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, vo, 0, 0));
            }
#pragma unroll
            for (int m = 0; m < CTW; ++m)
#pragma unroll
                for (int o = 0; o < OTW; ++o)
                    acc[u][m][o] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[o], acc[u][m][o], 0, 0, 0);
        }
        // next position, four along
        p += 4;
        iw += 4;
        while (iw >= AW.L_in) {
            iw -= AW.L_in;
            if (++ih == AH.L_in) {
                ih = 0;
                ++id;
            }
        }
    }

    // lane j + 16*c4, register v: dW_k[ci0 + 16m + 4*c4 + v][co0 + 16o + j]
#pragma unroll
    for (int u = 0; u < TK; ++u) {
        if (u >= tk) break;
#pragma unroll
        for (int m = 0; m < CTW; ++m)
#pragma unroll
            for (int o = 0; o < OTW; ++o) {
                const int co = co0 + 16 * o + i16;
                if (co >= P.Cog) continue;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int ci = ci0 + 16 * m + 4 * c4 + v;
                    if (ci >= P.Cig) continue;
                    atomicAdd(dw + ((int64_t)(g * P.Cig + ci) * P.Cog + co) * P.k_vol + k0 + u, acc[u][m][o][v]);
                }
            }
    }
}

// Groups of 8 input and 8 output channels with stride 2 and dilation 1 along
// W (the grouped 3D layer), where the kernel above would mask three quarters
// of every 16 x 16 tile.  Here a tile's rows are (sigma, ci), sigma = 0, 1,
// with A = x[ci][iw + sigma], and its columns (tau, co), tau = 0, 1, with
// B = dy[co][2 iw - p + T + tau].  With i = iw + sigma, entry ((sigma, ci),
// (tau, co)) sums x[ci][i] * dy[co][2 i - p + kw] over i for the W tap
// kw = T + tau - 2 sigma, so with T = 2, 6, 10, ... each W tap lies in exactly
// one entry of one tile (taps 4t .. 4t+3 in tile t), and a tile is useful work
// but for taps past K.  The positions iw run over [-1, W_in) four at a time
// (the MFMA's K), with x zero outside its row.  A wave walks a range of x rows
// (id, ih) of one (sample, group) for up to kWsTiles (D tap, H tap, T) tiles,
// skipping a tile whose dy row lies outside the output, then adds its tiles
// into dw with atomics (so the result varies in the last bits from run to run,
// as above).
// Tuning knob: (D tap, H tap, T) tiles per wave.
#ifndef CONVT_WS_TILES
#define CONVT_WS_TILES 4
#endif
constexpr int kWsTiles = CONVT_WS_TILES;

struct WsParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, G, k_vol;
    int in_sp, out_sp;
    int nT;            // W tap blocks: taps T-2 .. T+1 for T = 2 + 4t
    int ntiles;        // KD * KH * nT
    int tchunks;       // chunks of kWsTiles tiles
    int rows;          // x rows (id, ih) per sample
    int rows_per_wave;
    int rchunks;       // row ranges per (sample, group, chunk)
    int64_t units;     // waves of work
    int wsplit;        // row-sharing kernel: the 4 waves split one unit's W steps
};

__global__ __launch_bounds__(kWgBlock) void k_backward_weight_shift(const WsParams P, const float *__restrict__ x,
                                                                    const float *__restrict__ dy, float *dw) {
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int lane = threadIdx.x & 63;
    const int64_t unit =
        (int64_t)blockIdx.x * (kWgBlock / 64) + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (unit >= P.units) return; // no barrier in this kernel: a wave may leave early
    int64_t t = unit;
    const int rc = (int)(t % P.rchunks);
    t /= P.rchunks;
    const int tc = (int)(t % P.tchunks);
    t /= P.tchunks;
    const int g = (int)(t % P.G);
    const int n = (int)(t / P.G);
    const int tile0 = tc * kWsTiles, ntl = min(kWsTiles, P.ntiles - tile0);
    const int r_begin = rc * P.rows_per_wave, r_end = min(r_begin + P.rows_per_wave, P.rows);

    const int i16 = lane & 15, c4 = lane >> 4;
    const int sig = i16 >> 3, ci = i16 & 7;  // A row
    const int tau = i16 >> 3, co = i16 & 7;  // B column
    const wg_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + ((int64_t)n * P.C_in + (int64_t)g * 8) * P.in_sp), (short)0, (int)(4 * 8 * P.in_sp),
        kWgRsrcWord3);
    const wg_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + ((int64_t)n * P.C_out + (int64_t)g * 8) * P.out_sp), (short)0,
        (int)(4 * 8 * P.out_sp), kWgRsrcWord3);
    const int xch = ci * P.in_sp, ych = co * P.out_sp;

    // the chunk's tiles (uniform): D tap, H tap, W tap base T
    int tkd[kWsTiles], tkh[kWsTiles], tT[kWsTiles];
#pragma unroll
    for (int u = 0; u < kWsTiles; ++u) {
        const int tile = tile0 + min(u, ntl - 1);
        tT[u] = 2 + 4 * (tile % P.nT);
        const int kdh = tile / P.nT;
        tkh[u] = kdh % AH.K;
        tkd[u] = kdh / AH.K;
    }
    wg_v4f acc[kWsTiles];
#pragma unroll
    for (int u = 0; u < kWsTiles; ++u) acc[u] = wg_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Steps k = (row, iw0) flattened, iw0 = -1, 3, 7, ... per row; the operands
    // of step k + 1 are loaded while step k's MFMAs run.  The loop has no
    // branch: every load is issued (one outside x's row or the output returns
    // zero), and every tile's MFMA runs (a dy row outside the output adds
    // zeros; tiles past the chunk's last repeat it and are not stored), so
    // the loads stay in flight across the MFMAs.
    const int spr = (AW.L_in + 4) / 4; // steps per row: iw0 + 3 >= W_in - 1 at the last
    const int nsteps = (r_end - r_begin) * spr;
    auto load = [&](int k, float &a, float (&b)[kWsTiles]) __attribute__((always_inline)) {
        const int rr = k / spr;
        const int r = r_begin + rr, iw = -1 + 4 * (k - rr * spr) + c4;
        const int id = r / AH.L_in, ih = r - id * AH.L_in;
        const int xrow = (id * AH.L_in + ih) * AW.L_in;
        const int xi = iw + sig;
        // (& rather than &&: no branch around the loads)
        const unsigned xo = ((xi >= 0) & (xi < AW.L_in)) ? 4u * (unsigned)(xch + xrow + xi) : kWgOutOfRange;
        a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, xo, 0, 0));
        const int ow0 = 2 * iw - AW.p + tau;
#pragma unroll
        for (int u = 0; u < kWsTiles; ++u) {
            const int od = id * AD.s - AD.p + tkd[u] * AD.d, oh = ih * AH.s - AH.p + tkh[u] * AH.d;
            const int ow = ow0 + tT[u];
            const bool ok = (od >= 0) & (od < AD.L_out) & (oh >= 0) & (oh < AH.L_out) & (ow >= 0) & (ow < AW.L_out);
            const unsigned yo = ok ? 4u * (unsigned)(ych + (od * AH.L_out + oh) * AW.L_out + ow) : kWgOutOfRange;
            b[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, yo, 0, 0));
        }
    };
    auto compute = [&](const float a, const float (&b)[kWsTiles]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kWsTiles; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[u], acc[u], 0, 0, 0);
    };
    // Two register sets in turn (a copy from one to the other would wait for
    // the loads in flight); a load past the last step fetches the last again,
    // unused, and an odd last step runs its second half with A = 0.
    float a0 = 0.0f, a1, b0[kWsTiles], b1[kWsTiles];
    if (nsteps > 0) load(0, a0, b0);
    for (int k = 0; k < nsteps; k += 2) {
        load(min(k + 1, nsteps - 1), a1, b1);
        compute(a0, b0);
        load(min(k + 2, nsteps - 1), a0, b0);
        compute(k + 1 < nsteps ? a1 : 0.0f, b1);
    }

    // lane j + 16*c4, register v: row i = 4*c4 + v = (sigma, ci), column j = (tau, co)
#pragma unroll
    for (int u = 0; u < kWsTiles; ++u) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 4 * c4 + v;
            const int kw = tT[u] + tau - 2 * (i >> 3);
            if (u < ntl && kw >= 0 && kw < AW.K)
                atomicAdd(dw + ((int64_t)(g * 8 + (i & 7)) * 8 + co) * P.k_vol + (tkd[u] * AH.K + tkh[u]) * AW.K +
                              kw,
                          acc[u][v]);
        }
    }
}

// The same tiles where H has stride 1 and dilation 1 (the grouped 3D layer),
// with dy rows shared across x rows: x row ih meets dy row ih - p_h + kh
// through H tap kh, so the dy row that x row ih + 1 needs for tap kh - 1 is
// the one row ih used for tap kh.  A wave owns one (sample, group, D tap,
// D position) and a range of consecutive x rows, with a tile for each (H tap,
// T) pair; per W step it walks its rows holding the dy rows in KH + 1 slots,
// each new row loading one dy row per T instead of KH (the slot names rotate
// with the row, compile-time in a loop unrolled by KH + 1).  The next row's
// operands are loaded while the current row's MFMAs run.  Rows past the range
// read x as zero.  The four waves of a workgroup share (sample, group, D tap)
// and take different (x plane, row range) units; they sum their tiles in LDS
// and add a quarter of the atomic updates each.
template <int KH, int NTW>
__global__ __launch_bounds__(kWgBlock) void k_backward_weight_shift_rows(const WsParams P,
                                                                         const float *__restrict__ x,
                                                                         const float *__restrict__ dy, float *dw) {
    constexpr int NSL = KH + 1;                       // dy row slots
    constexpr int U = NSL % 2 == 0 ? NSL : 2 * NSL;   // rows per unrolled trip (x alternates two registers)
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // workgroup: (sample, group, D tap) and four of its (x plane, row range)
    // units, or with wsplit one unit whose W steps the four waves split (they
    // then read the same x and dy lines at about the same time); a wave past
    // the last unit, or whose D tap reaches no output from its plane, has no
    // work but joins the reduction
    const int per = AD.L_in * P.rchunks;
    const int bpg = P.wsplit ? per : (per + 3) / 4;
    const int64_t ngk = (int64_t)blockIdx.x / bpg;
    const int sub = P.wsplit ? (int)((int64_t)blockIdx.x - ngk * bpg)
                             : (int)((int64_t)blockIdx.x - ngk * bpg) * 4 + wave;
    const int kd = (int)(ngk % AD.K);
    const int g = (int)((ngk / AD.K) % P.G);
    const int n = (int)(ngk / AD.K / P.G);
    const int rri = sub % P.rchunks;
    const int id = min(sub / P.rchunks, AD.L_in - 1);
    const int od = id * AD.s - AD.p + kd * AD.d;
    const bool work = sub < per && od >= 0 && od < AD.L_out; // uniform over the wave
    const int ih_b = rri * P.rows_per_wave;
    const int nrows = min(P.rows_per_wave, AH.L_in - ih_b);
    const int npad = (nrows + U - 1) / U * U;

    const int i16 = lane & 15, c4 = lane >> 4;
    const int sig = i16 >> 3, ci = i16 & 7;  // A row
    const int tau = i16 >> 3, co = i16 & 7;  // B column
    const wg_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + ((int64_t)n * P.C_in + (int64_t)g * 8) * P.in_sp), (short)0, (int)(4 * 8 * P.in_sp),
        kWgRsrcWord3);
    const wg_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + ((int64_t)n * P.C_out + (int64_t)g * 8) * P.out_sp), (short)0,
        (int)(4 * 8 * P.out_sp), kWgRsrcWord3);
    const int xbase = ci * P.in_sp + (id * AH.L_in + ih_b) * AW.L_in;             // x row ih_b, channel ci
    const int ybase = co * P.out_sp + (od * AH.L_out + ih_b - AH.p) * AW.L_out;   // dy row R = 0, channel co

    wg_v4f acc[KH][NTW];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) acc[kh][tt] = wg_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int spr = work ? (AW.L_in + 4) / 4 : 0; // W steps: iw = -1 + 4 st + c4
    // dy relative row R (oh = ih_b - p_h + R) at W step st, every T; zero
    // outside the output
    auto load_b = [&](int R, int st, float (&b)[NTW]) __attribute__((always_inline)) {
        const int oh = ih_b - AH.p + R;
        const bool rok = (oh >= 0) & (oh < AH.L_out);
        const int ow0 = 2 * (4 * st + c4 - 1) - AW.p + 2 + tau;
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt) {
            const int ow = ow0 + 4 * tt;
            const unsigned off = (rok & (ow >= 0) & (ow < AW.L_out)) ? 4u * (unsigned)(ybase + R * AW.L_out + ow)
                                                                   : kWgOutOfRange;
            b[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, off, 0, 0));
        }
    };
    // x row ih_b + rr at W step st, zero past the wave's rows or the row's ends
    auto load_x = [&](int rr, int st) __attribute__((always_inline)) {
        const int xi = 4 * st + c4 - 1 + sig;
        const unsigned off = ((rr < nrows) & (xi >= 0) & (xi < AW.L_in)) ? 4u * (unsigned)(xbase + rr * AW.L_in + xi)
                                                                      : kWgOutOfRange;
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
    };
    const int st0 = P.wsplit ? wave : 0, dst = P.wsplit ? 4 : 1;
    for (int st = st0; st < spr; st += dst) {
        float sl[NSL][NTW];
        float xa[2];
#pragma unroll
        for (int R = 0; R < KH; ++R) load_b(R, st, sl[R]);
        xa[0] = load_x(0, st);
        for (int rr0 = 0; rr0 < npad; rr0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int rr = rr0 + u;
                // the next row's new dy row (its tap KH - 1) and x row
                load_b(rr + KH, st, sl[(u + KH) % NSL]);
                xa[(u + 1) & 1] = load_x(rr + 1, st);
#pragma unroll
                for (int kh = 0; kh < KH; ++kh)
#pragma unroll
                    for (int tt = 0; tt < NTW; ++tt)
                        acc[kh][tt] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(xa[u & 1], sl[(u + kh) % NSL][tt], acc[kh][tt], 0, 0, 0);
            }
        }
    }

    // The four waves' tiles meet in LDS ([value e][wave][lane], e = (kh, tt,
    // v)); wave w then adds values e = w, w + 4, ... of the sum into dw.
    // Lane j + 16*c4, register v: row i = 4*c4 + v = (sigma, ci), column j =
    // (tau, co).
    constexpr int NE = KH * NTW * 4;
    __shared__ float red[NE * 4 * 64];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(((kh * NTW + tt) * 4 + v) * 4 + wave) * 64 + lane] = acc[kh][tt][v];
    __syncthreads();
    for (int e = wave; e < NE; e += 4) {
        const float sum = (red[(e * 4 + 0) * 64 + lane] + red[(e * 4 + 1) * 64 + lane]) +
                          (red[(e * 4 + 2) * 64 + lane] + red[(e * 4 + 3) * 64 + lane]);
        const int v = e & 3, tt = (e >> 2) % NTW, kh = (e >> 2) / NTW;
        const int i = 4 * c4 + v;
        const int kw = 2 + 4 * tt + tau - 2 * (i >> 3);
        if (kw >= 0 && kw < AW.K)
            atomicAdd(dw + ((int64_t)(g * 8 + (i & 7)) * 8 + co) * P.k_vol + (kd * KH + kh) * AW.K + kw, sum);
    }
}

// The shift-pair kernel applies: groups of 8 input and 8 output channels,
// stride 2 and dilation 1 along W, a group's x and dy below 2 GiB.
bool weight_shift_applies(const convt_plan &Pl) {
    return Pl.Cig == 8 && Pl.Cog == 8 && Pl.ax[2].s == 2 && Pl.ax[2].d == 1 && 4 * 8 * Pl.in_sp <= 0x7fffffff &&
           4 * 8 * Pl.out_sp <= 0x7fffffff;
}

// Tuning knob: waves the shift-pair kernel's grid aims for (more waves, more
// atomic adds).
#ifndef CONVT_WS_WAVES
#define CONVT_WS_WAVES 4096
#endif

// Tuning knob: waves the row-sharing kernel's grid aims for (fewer waves walk
// longer row ranges: less warm-up and padding per row, fewer partial sums).
#ifndef CONVT_WSR_WAVES
#define CONVT_WSR_WAVES 1024
#endif
// Tuning knob: the row-sharing kernel's four waves split one unit's W steps.
#ifndef CONVT_WSR_WSPLIT
#define CONVT_WSR_WSPLIT 1
#endif

// The row-sharing variant applies as well: H stride 1 and dilation 1, at most
// 7 H taps and 8 W taps (two T blocks).
bool weight_shift_rows_applies(const convt_plan &Pl) {
    return weight_shift_applies(Pl) && Pl.ax[1].s == 1 && Pl.ax[1].d == 1 && Pl.ax[1].K <= 7 && Pl.ax[2].K <= 8;
}

int launch_weight_shift_rows(const convt_plan &Pl, const float *x, const float *dy, float *dw, hipStream_t st) {
    WsParams P;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.G = (int)Pl.G;
    P.k_vol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    const int KH = Pl.ax[1].K, NTW = (Pl.ax[2].K + 3) / 4;
    const int U = (KH + 1) % 2 == 0 ? KH + 1 : 2 * (KH + 1);
    const int H = Pl.ax[1].L_in;
    // row ranges: about CONVT_WSR_WAVES waves (at least one range per x
    // plane), each range a multiple of the unrolled trip (its padding rows add
    // zeros)
    const int64_t base = Pl.N * Pl.G * (int64_t)Pl.ax[0].K * Pl.ax[0].L_in;
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>(H, (CONVT_WSR_WAVES + base - 1) / base));
    int rpw = (int)((H + want - 1) / want);
    rpw = (rpw + U - 1) / U * U;
    P.rows_per_wave = rpw;
    P.rchunks = (H + rpw - 1) / rpw;
    P.units = base * P.rchunks;
    // workgroups: per (sample, group, D tap), four (x plane, row range) units
    // each, or one with its W steps split over the waves
    P.wsplit = CONVT_WSR_WSPLIT;
    const int64_t per = Pl.ax[0].L_in * (int64_t)P.rchunks;
    const int64_t blocks = Pl.N * Pl.G * (int64_t)Pl.ax[0].K * (P.wsplit ? per : (per + 3) / 4);
    if (blocks > 0x7fffffff || Pl.ax[0].L_in * (int64_t)P.rchunks > 0x7fffffff) return (int)hipErrorInvalidValue;
    auto go = [&](auto khc, auto ntc) {
        hipLaunchKernelGGL((k_backward_weight_shift_rows<decltype(khc)::value, decltype(ntc)::value>),
                           dim3((unsigned)blocks), dim3(kWgBlock), 0, st, P, x, dy, dw);
    };
    auto by_nt = [&](auto khc) {
        if (NTW == 1) go(khc, std::integral_constant<int, 1>{});
        else go(khc, std::integral_constant<int, 2>{});
    };
    switch (KH) {
    case 1: by_nt(std::integral_constant<int, 1>{}); break;
    case 2: by_nt(std::integral_constant<int, 2>{}); break;
    case 3: by_nt(std::integral_constant<int, 3>{}); break;
    case 4: by_nt(std::integral_constant<int, 4>{}); break;
    case 5: by_nt(std::integral_constant<int, 5>{}); break;
    case 6: by_nt(std::integral_constant<int, 6>{}); break;
    default: by_nt(std::integral_constant<int, 7>{}); break;
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

int launch_weight_shift(const convt_plan &Pl, const float *x, const float *dy, float *dw, hipStream_t st) {
    WsParams P;
    P.wsplit = 0;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.G = (int)Pl.G;
    P.k_vol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    P.nT = (Pl.ax[2].K + 3) / 4;
    P.ntiles = Pl.ax[0].K * Pl.ax[1].K * P.nT;
    P.tchunks = (P.ntiles + kWsTiles - 1) / kWsTiles;
    P.rows = Pl.ax[0].L_in * Pl.ax[1].L_in;
    const int64_t lanes = Pl.N * Pl.G * (int64_t)P.tchunks;
    const int64_t want = (lanes * P.rows + CONVT_WS_WAVES - 1) / CONVT_WS_WAVES;
    P.rows_per_wave = (int)std::max<int64_t>(1, std::min<int64_t>(want, P.rows));
    P.rchunks = (P.rows + P.rows_per_wave - 1) / P.rows_per_wave;
    P.units = lanes * P.rchunks;
    const int64_t blocks = (P.units + kWgBlock / 64 - 1) / (kWgBlock / 64);
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_backward_weight_shift, dim3((unsigned)blocks), dim3(kWgBlock), 0, st, P, x, dy, dw);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

// Channel-rich groups (32k input, 64k output channels): the same GEMM with
// both operands staged through LDS, so that global loads run along positions
// (coalesced) instead of gathering 16 channel rows per instruction.  A
// workgroup owns 32 input x 64 output channels x up to kWlTaps taps over a
// range of positions of one sample; per tile of 64 positions it stages x as
// [position][ci] once and, per tap, dy at o(p, k) as [position][co] (rows
// padded by one float: the transposed writes do not collide on a bank); wave
// w then runs the 16 K-steps of its output-channel tile for both input-channel
// tiles.  Partial sums go to dw with atomics as above.
constexpr int kWlTaps = 4;      // taps per workgroup
constexpr int kWlTile = 64;     // positions per staged tile
constexpr int kWlRange = 2048;  // positions per workgroup
constexpr int kWlApitch = 33;   // floats per staged x position row (32 channels + 1)
constexpr int kWlBpitch = 65;   // floats per staged dy position row (64 channels + 1)

struct WlParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, k_vol;
    int in_sp, out_sp;
    int cib, cob;      // 32- and 64-channel blocks of the group
    int kchunks;       // chunks of kWlTaps taps
    int nranges;       // position ranges per sample
};

__global__ __launch_bounds__(kWgBlock) void k_backward_weight_lds(const WlParams P, const float *__restrict__ x,
                                                                  const float *__restrict__ dy, float *dw) {
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t t = blockIdx.x;
    const int range = (int)(t % P.nranges);
    t /= P.nranges;
    const int kc = (int)(t % P.kchunks);
    t /= P.kchunks;
    const int cb = (int)(t % P.cob);
    t /= P.cob;
    const int ib = (int)(t % P.cib);
    t /= P.cib;
    const int g = (int)(t % (P.C_in / P.Cig));
    const int n = (int)(t / (P.C_in / P.Cig));
    const int ci0 = 32 * ib, co0 = 64 * cb;
    const int k0 = kc * kWlTaps, tk = min(kWlTaps, P.k_vol - k0);

    __shared__ float As[kWlTile * kWlApitch];
    __shared__ float Bs[kWlTile * kWlBpitch];

    const float *xg = x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig + ci0) * P.in_sp;
    const float *dyg = dy + ((int64_t)n * P.C_out + (int64_t)g * P.Cog + co0) * P.out_sp;

    wg_v4f acc[kWlTaps][2];
#pragma unroll
    for (int u = 0; u < kWlTaps; ++u) acc[u][0] = acc[u][1] = wg_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int i16 = lane & 15, c4 = lane >> 4;
    const int p_begin = range * kWlRange;
    const int p_end = min(p_begin + kWlRange, P.in_sp);
    for (int p0 = p_begin; p0 < p_end; p0 += kWlTile) {
        // this lane's position of the tile
        const int p = p0 + lane;
        const bool live = p < p_end;
        const int iw = p % AW.L_in, ih = (p / AW.L_in) % AH.L_in, id = p / (AW.L_in * AH.L_in);
        __syncthreads(); // the previous tile's operands are consumed
        {
            // unconditional loads (positions past the range read its last one
            // and store zero), so all eight are in flight at once
            const int pc = min(p, p_end - 1);
            float xv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) xv[r] = xg[(int64_t)(wave + 4 * r) * P.in_sp + pc];
#pragma unroll
            for (int r = 0; r < 8; ++r) As[lane * kWlApitch + wave + 4 * r] = live ? xv[r] : 0.0f;
        }
        for (int u = 0; u < tk; ++u) {
            const int k = k0 + u;
            const int kw = k % AW.K, kdh = k / AW.K;
            const int od = id * AD.s - AD.p + (kdh / AH.K) * AD.d;
            const int oh = ih * AH.s - AH.p + (kdh % AH.K) * AH.d;
            const int ow = iw * AW.s - AW.p + kw * AW.d;
            const bool ok = live && od >= 0 && od < AD.L_out && oh >= 0 && oh < AH.L_out && ow >= 0 &&
                            ow < AW.L_out;
            const int o = ok ? (od * AH.L_out + oh) * AW.L_out + ow : 0;
            if (u > 0) __syncthreads(); // the previous tap's dy tile is consumed
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = wave + 4 * r;
                const float v = dyg[(int64_t)co * P.out_sp + o];
                Bs[lane * kWlBpitch + co] = ok ? v : 0.0f;
            }
            __syncthreads();
            // wave: output-channel tile `wave`, both input-channel tiles
#pragma unroll
            for (int q = 0; q < kWlTile / 4; ++q) {
                const int pp = 4 * q + c4;
                const float b = Bs[pp * kWlBpitch + 16 * wave + i16];
                const float a0 = As[pp * kWlApitch + i16];
                const float a1 = As[pp * kWlApitch + 16 + i16];
#pragma unroll
                for (int uu = 0; uu < kWlTaps; ++uu) {
                    if (uu != u) continue;
                    acc[uu][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b, acc[uu][0], 0, 0, 0);
                    acc[uu][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b, acc[uu][1], 0, 0, 0);
                }
            }
        }
    }

    // lane j + 16*c4, register v: dW_k[ci0 + 16m + 4*c4 + v][co0 + 16*wave + j]
    const int co = co0 + 16 * wave + i16;
#pragma unroll
    for (int u = 0; u < kWlTaps; ++u) {
        if (u >= tk) break;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ci = ci0 + 16 * m + 4 * c4 + v;
                atomicAdd(dw + ((int64_t)(g * P.Cig + ci) * P.Cog + co) * P.k_vol + k0 + u, acc[u][m][v]);
            }
    }
}

// One-axis plans (unit leading axes) with the same channel blocks: for a tile
// of 64 consecutive positions the dy values of every tap of the chunk lie in
// one window of each output-channel row, columns e <-> o = p0*s - p + k0*d +
// cs*e, where cs = s when s divides d (then only every s-th column is read:
// position pp, tap u at column pp*js + u*kd with js = s/cs, kd = d/cs), else
// 1.  The window is staged once per tile for all taps, transposed to
// [column][co] (pitch 65), with loads along the row, so the tile takes two
// barriers instead of one per tap, and each A read from LDS feeds every tap.
// Partial sums go to dw with atomics as above.
struct WrParams {
    WlParams L;
    int win_cols;            // columns of the staged window
    int win_cs, win_js, win_kd;
    float inv_cols;          // 1 / win_cols (exact quotients for the staged index range)
};

__global__ __launch_bounds__(kWgBlock) void k_backward_weight_row(const WrParams R, const float *__restrict__ x,
                                                                  const float *__restrict__ dy, float *dw) {
    const WlParams &P = R.L;
    const AxisPlan &AW = P.ax[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t t = blockIdx.x;
    const int range = (int)(t % P.nranges);
    t /= P.nranges;
    const int kc = (int)(t % P.kchunks);
    t /= P.kchunks;
    const int cb = (int)(t % P.cob);
    t /= P.cob;
    const int ib = (int)(t % P.cib);
    t /= P.cib;
    const int g = (int)(t % (P.C_in / P.Cig));
    const int n = (int)(t / (P.C_in / P.Cig));
    const int ci0 = 32 * ib, co0 = 64 * cb;
    const int k0 = kc * kWlTaps, tk = min(kWlTaps, P.k_vol - k0);
    const int Wn = R.win_cols, cs = R.win_cs;

    extern __shared__ __attribute__((aligned(16))) float wr_lds[];
    float *As = wr_lds;                     // [position][ci], pitch kWlApitch
    float *Bw = wr_lds + kWlTile * kWlApitch; // [column][co], pitch kWlBpitch

    const float *xg = x + ((int64_t)n * P.C_in + (int64_t)g * P.Cig + ci0) * P.in_sp;
    const float *dyg = dy + ((int64_t)n * P.C_out + (int64_t)g * P.Cog + co0) * P.out_sp;

    wg_v4f acc[kWlTaps][2];
#pragma unroll
    for (int u = 0; u < kWlTaps; ++u) acc[u][0] = acc[u][1] = wg_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int i16 = lane & 15, c4 = lane >> 4;
    const int p_begin = range * kWlRange;
    const int p_end = min(p_begin + kWlRange, P.in_sp);
    const int nwin = Wn * 64;
    for (int p0 = p_begin; p0 < p_end; p0 += kWlTile) {
        const int p = p0 + lane;
        const bool live = p < p_end;
        const int obase = p0 * AW.s - AW.p + k0 * AW.d;
        __syncthreads(); // the previous tile's operands are consumed
        // x tile, [position][ci]; positions past the range are zero, so the
        // window's columns for them add nothing
        {
            // unconditional loads (positions past the range read its last one
            // and store zero), so all eight are in flight at once
            const int pc = min(p, p_end - 1);
            float xv[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) xv[r] = xg[(int64_t)(wave + 4 * r) * P.in_sp + pc];
#pragma unroll
            for (int r = 0; r < 8; ++r) As[lane * kWlApitch + wave + 4 * r] = live ? xv[r] : 0.0f;
        }
        // dy window: element idx = co*Wn + e, consecutive threads along e
        for (int i0 = 0; i0 < nwin; i0 += 8 * kWgBlock) {
            float v[8];
            int slot[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int idx = i0 + u * kWgBlock + threadIdx.x;
                const int co = (int)(((float)idx + 0.5f) * R.inv_cols);
                const int e = idx - co * Wn;
                const int o = obase + cs * e;
                const bool ok = idx < nwin && o >= 0 && o < AW.L_out;
                v[u] = ok ? dyg[(int64_t)co * P.out_sp + o] : 0.0f;
                slot[u] = idx < nwin ? e * kWlBpitch + co : -1;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (slot[u] >= 0) Bw[slot[u]] = v[u];
        }
        __syncthreads();
        // wave: output-channel tile `wave`, both input-channel tiles, every tap
#pragma unroll
        for (int q = 0; q < kWlTile / 4; ++q) {
            const int pp = 4 * q + c4;
            const float a0 = As[pp * kWlApitch + i16];
            const float a1 = As[pp * kWlApitch + 16 + i16];
            const float *bcol = Bw + pp * R.win_js * kWlBpitch + 16 * wave + i16;
#pragma unroll
            for (int u = 0; u < kWlTaps; ++u) {
                if (u >= tk) break;
                const float b = bcol[u * R.win_kd * kWlBpitch];
                acc[u][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b, acc[u][0], 0, 0, 0);
                acc[u][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b, acc[u][1], 0, 0, 0);
            }
        }
    }

    // lane j + 16*c4, register v: dW_k[ci0 + 16m + 4*c4 + v][co0 + 16*wave + j]
    const int co = co0 + 16 * wave + i16;
#pragma unroll
    for (int u = 0; u < kWlTaps; ++u) {
        if (u >= tk) break;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int ci = ci0 + 16 * m + 4 * c4 + v;
                atomicAdd(dw + ((int64_t)(g * P.Cig + ci) * P.Cog + co) * P.k_vol + k0 + u, acc[u][m][v]);
            }
    }
}

// The one-axis window kernel applies: unit leading axes, the LDS kernel's
// channel blocks, and the x tile plus the window within 64 KB.  Fills the
// window fields of R and returns true when it applies.
bool weight_row_window(const convt_plan &Pl, WrParams &R) {
    if (Pl.Cig % 32 != 0 || Pl.Cog % 64 != 0) return false;
    // A leading axis must be a unit axis whose one tap lands on its one output
    // (p = 0 and L_out = 1): the window kernels index only the last axis.
    for (int a = 0; a < 2; ++a)
        if (Pl.ax[a].L_in != 1 || Pl.ax[a].K != 1 || Pl.ax[a].p != 0 || Pl.ax[a].L_out != 1) return false;
    const AxisPlan &A = Pl.ax[2];
    const int cs = A.d % A.s == 0 ? A.s : 1;
    const int tk = Pl.k_vol < kWlTaps ? (int)Pl.k_vol : kWlTaps;
    const int64_t wn = (int64_t)(kWlTile - 1) * (A.s / cs) + (int64_t)(tk - 1) * (A.d / cs) + 1;
    if ((kWlTile * kWlApitch + wn * kWlBpitch) * 4 > 65536) return false;
    R.win_cols = (int)wn;
    R.win_cs = cs;
    R.win_js = A.s / cs;
    R.win_kd = A.d / cs;
    R.inv_cols = 1.0f / (float)wn;
    return true;
}

// Groups of 32k input and 4k output channels with W_in of 16, 32 or 64 and at
// most 32 taps (the fused 3D layer): both operands staged in LDS per block of
// 128 input positions, as in the staged input gradient.  A workgroup owns the
// tile dw[32 input channels][output-channel quad q][all taps] of one (sample,
// group) and walks the sample's blocks (D position, R = 128 / W_in rows).
// Per block it stages the x tile [ci][position] and, for each D tap, the dy
// window of the quad: 4 channels x NR rows x NW columns of one dy plane (zero
// outside the output).  With K = 4 positions of one row, the MFMA's 16
// columns are (tap t = 4*tg + j/4, channel c = j%4): B (lane j + 16k) is the
// window value of channel c at position k's tap-t output, A (lane i + 16k)
// is x[ci0 + 16m + i] at position k.  Wave w owns tap group (w - workgroup)
// mod 8 (so the waves without a group, when there are fewer than 8, move
// over the SIMDs from workgroup to workgroup) for both input-channel tiles,
// and adds its tiles into dw with atomics at the end.  The next block's
// operands are loaded into registers during the current block's products.
// Each thread's window elements keep their offset from the block's origin
// with an index kd*NR + rr (63: never valid) into a per-block mask of the
// (D tap, row) pairs inside the output.
constexpr int kWtPos = 128;                       // positions per block
constexpr int kWtNT = 512;                        // 8 waves
constexpr int kWtXP = kWtPos + 4;                 // x tile pitch
constexpr int kWtWinCap = 7168;                   // window floats, all D taps (one tap group per wave)
constexpr int kWtWinCap2 = 10752;                 // the same with two tap groups per wave (33 to 64 taps)
constexpr int kWtXU = 32 * kWtPos / 4 / kWtNT;    // x float4s per thread

struct WtParams {
    AxisPlan ax[kAxes];
    int C_in, C_out, Cig, Cog, kvol;
    int in_sp, out_sp;
    int R, nhb, ccs, NQ, NR, NW, TG;
};

// Tuning knob: waves per SIMD the fused-geometry instance must allow (6: three
// workgroups per CU, 80 registers).
#ifndef CONVT_WT_WAVES
#define CONVT_WT_WAVES 6
#endif
template <int TGW, int GEO>
__global__ __launch_bounds__(kWtNT) __attribute__((amdgpu_waves_per_eu(GEO == 1 ? CONVT_WT_WAVES : 1)))
void k_backward_weight_stage(const WtParams P, const float *__restrict__ x,
                                                                 const float *__restrict__ dy,
                                                                 float *__restrict__ dw) {
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    // GEO 1: the fused layer's geometry (W_in 16, 3 x 3 x 3 taps, H and W
    // stride 2 and dilation 1), GEO 2: the channel-heavy layer's (W_in 32,
    // 4 x 4 x 4 taps, the same strides), as constants; GEO 0: the plan's
    constexpr bool FIX = GEO != 0;
    constexpr int FW = GEO == 2 ? 32 : 16, FK = GEO == 2 ? 4 : 3, FR = 128 / FW;
    constexpr int FNR = (FR - 1) * 2 + FK, FNW = (FW - 1) * 2 + FK;
    const int WIN = FIX ? FW : AW.L_in;
    const int SH = FIX ? 2 : AH.s, SW = FIX ? 2 : AW.s, DH = FIX ? 1 : AH.d, DW = FIX ? 1 : AW.d;
    const int KD = FIX ? FK : AD.K, KH = FIX ? FK : AH.K, KW = FIX ? FK : AW.K;
    const int R = FIX ? FR : P.R, NR = FIX ? FNR : P.NR, NW = FIX ? FNW : P.NW;
    const int TG = FIX ? (FK * FK * FK + 3) / 4 : P.TG;
    static_assert(!FIX || TGW == (FK * FK * FK > 32 ? 2 : 1), "tap groups per wave of the fixed geometry");
    constexpr int CAP = TGW == 2 ? kWtWinCap2 : kWtWinCap, WU = CAP / kWtNT;
    static_assert(WU * kWtNT == CAP, "window buffer split evenly over the threads");
    const int win_sz = 4 * NR * NW, kvol = KD * KH * KW, wins = KD * win_sz;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int64_t b = blockIdx.x;
    const int q = (int)(b % P.NQ);
    b /= P.NQ;
    const int cc = (int)(b % P.ccs);
    b /= P.ccs;
    const int G = P.C_in / P.Cig;
    const int g = (int)(b % G);
    const int n = (int)(b / G);
    const int ci0 = g * P.Cig + cc * 32;
    // tap groups tg and tg + 8 (TGW = 2)
    const int tg = (wave + 8 - (int)(blockIdx.x & 7)) & 7;
    const int HWo = AH.L_out * AW.L_out;

    extern __shared__ __attribute__((aligned(16))) float lds_wt[];
    float *wl = lds_wt, *xl = lds_wt + CAP;

    // window elements: offset (bits 0-25) from the block's origin and (D tap,
    // row) index (bits 26-31)
    unsigned winfo[WU];
#pragma unroll
    for (int u = 0; u < WU; ++u) {
        const int e = tid + u * kWtNT;
        const int kd = e / win_sz, r1 = e - kd * win_sz;
        const int c = r1 / (NR * NW), r2 = r1 - c * (NR * NW);
        const int rr = r2 / NW, col = r2 - rr * NW;
        const int ow = col - AW.p;
        const bool ok = e < wins && ow >= 0 && ow < AW.L_out;
        const unsigned off = (unsigned)(c * P.out_sp + kd * AD.d * HWo + rr * AW.L_out + col);
        winfo[u] = off | ((unsigned)(ok ? kd * NR + rr : 63) << 26);
    }
    // x float4s: channel ci, position 4*p4 of the block
    unsigned xoff[kWtXU];
    int xlo[kWtXU], xp[kWtXU];
#pragma unroll
    for (int u = 0; u < kWtXU; ++u) {
        const int f = tid + u * kWtNT;
        const int ci = f >> 5, p4 = f & 31;
        xoff[u] = 4u * (unsigned)(ci * P.in_sp + 4 * p4);
        xlo[u] = ci * kWtXP + 4 * p4;
        xp[u] = 4 * p4;
    }
    const wg_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(dy + (int64_t)n * P.C_out * P.out_sp), (short)0, 4 * P.C_out * P.out_sp, kWgRsrcWord3);
    const wg_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + (int64_t)n * P.C_in * P.in_sp), (short)0, 4 * P.C_in * P.in_sp, kWgRsrcWord3);
    const int soff_q = 4 * (g * P.Cog + 4 * q) * P.out_sp;
    const int nblk = AD.L_in * P.nhb;

    float pf[WU];
    wg_v4f xpf[kWtXU];
    // block blk = (id, hb) into registers; past the last block everything
    // reads zero
    auto fetch = [&](int blk) __attribute__((always_inline)) {
        const int id = blk / P.nhb, hb = blk - id * P.nhb;
        const int ih0 = hb * R;
        const bool live = blk < nblk;
        const int od0 = id * AD.s - AD.p, oh0 = ih0 * SH - AH.p;
        const int base = od0 * HWo + oh0 * AW.L_out - AW.p;
        // rows of the window inside the output: [lo, hi)
        const int lo = max(0, -oh0), hi = min(NR, AH.L_out - oh0);
        const uint64_t rows = hi > lo ? (((uint64_t)1 << hi) - 1) & ~(((uint64_t)1 << lo) - 1) : 0;
        uint64_t mask = 0;
        for (int kd = 0; kd < KD; ++kd) {
            const int od = od0 + kd * AD.d;
            if (live && od >= 0 && od < AD.L_out) mask |= rows << (kd * NR);
        }
#pragma unroll
        for (int u = 0; u < WU; ++u) {
            // the shift stays in the loop (a 64-bit 1 << idx per element
            // hoisted out of it would hold two registers each)
            unsigned idx = winfo[u] >> 26;
            asm volatile("" : "+v"(idx));
            const bool ok = ((mask >> idx) & 1u) != 0;
            const unsigned vo = ok ? 4u * (unsigned)((int)(winfo[u] & 0x3ffffffu) + base) : kWgOutOfRange;
            pf[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdy, vo, soff_q, 0));
        }
        const int vlen = live ? min(kWtPos, (AH.L_in - ih0) * WIN) : 0;
        const int soff_x = live ? 4 * (ci0 * P.in_sp + (id * AH.L_in + ih0) * WIN) : 0;
#pragma unroll
        for (int u = 0; u < kWtXU; ++u) {
            const unsigned vo = xp[u] < vlen ? xoff[u] : kWgOutOfRange;
            xpf[u] = __builtin_bit_cast(wg_v4f, __builtin_amdgcn_raw_buffer_load_b128(rx, vo, soff_x, 0));
        }
    };

    // this lane's B base: tap t of its column (the last tap for padding
    // columns, which are not stored) and position k of the K-step
    const int j16 = lane & 15, k4 = lane >> 4;
    int bbase[TGW];
#pragma unroll
    for (int h = 0; h < TGW; ++h) {
        const int t_l = min(4 * (tg + 8 * h) + (j16 >> 2), kvol - 1);
        const int kd_l = t_l / (KH * KW), kh_l = (t_l / KW) % KH, kw_l = t_l % KW;
        bbase[h] = kd_l * win_sz + (j16 & 3) * NR * NW + kh_l * DH * NW + kw_l * DW + k4 * SW;
    }
    const int abase = j16 * kWtXP + k4;
    wg_v4f acc[TGW][2];
#pragma unroll
    for (int h = 0; h < TGW; ++h) acc[h][0] = acc[h][1] = wg_v4f{0.0f, 0.0f, 0.0f, 0.0f};

    fetch(0);
    for (int blk = 0; blk < nblk; ++blk) {
        __syncthreads(); // every wave is done with the previous block
#pragma unroll
        for (int u = 0; u < WU; ++u) wl[tid + u * kWtNT] = pf[u];
#pragma unroll
        for (int u = 0; u < kWtXU; ++u) *reinterpret_cast<wg_v4f *>(xl + xlo[u]) = xpf[u];
        __syncthreads();
        fetch(blk + 1);
        if (tg < TG) {
            // K-step s: positions 4s .. 4s+3 of row 4s / W_in
            auto kstep = [&](int s) __attribute__((always_inline)) {
                const int r = (4 * s) / WIN, col0 = 4 * s - r * WIN;
                float bv[TGW];
#pragma unroll
                for (int h = 0; h < TGW; ++h) bv[h] = wl[bbase[h] + r * SH * NW + col0 * SW];
                const float a0 = xl[abase + 4 * s], a1 = xl[abase + 16 * kWtXP + 4 * s];
#pragma unroll
                for (int h = 0; h < TGW; ++h) {
                    acc[h][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, bv[h], acc[h][0], 0, 0, 0);
                    acc[h][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bv[h], acc[h][1], 0, 0, 0);
                }
            };
            if constexpr (GEO == 2) {
#pragma unroll
                for (int s = 0; s < kWtPos / 4; ++s) kstep(s);
            } else if constexpr (GEO == 1) {
#pragma unroll
                for (int s = 0; s < kWtPos / 4; ++s) kstep(s);
                // issue order: the reads of K-steps 0-3, then per pair of
                // K-steps its four products and the reads two pairs ahead
                __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
                for (int i = 0; i < kWtPos / 8 - 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            } else {
                for (int s = 0; s < kWtPos / 4; ++s) kstep(s);
            }
        }
    }

    // lane j16 + 16*k4, register v: input channel 16m + 4*k4 + v, column j16
#pragma unroll
    for (int h = 0; h < TGW; ++h) {
        const int t_s = 4 * (tg + 8 * h) + (j16 >> 2);
        if (tg < TG && t_s < kvol) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    atomicAdd(dw + ((int64_t)(ci0 + 16 * m + 4 * k4 + v) * P.Cog + 4 * q + (j16 & 3)) * kvol + t_s,
                              acc[h][m][v]);
        }
    }
}

// The staged weight kernel applies: 2D or 3D plans with groups of 32k input
// and 4k output channels, W_in of 16, 32 or 64, at most 64 taps (one tap group
// per wave up to 32, two above), the D taps' windows within kWtWinCap floats
// (kWtWinCap2 with two groups per wave) and their (D tap, row) pairs within 63
// mask bits, window offsets within 26 bits, per-sample x and dy below 2 GiB.
bool weight_stage_applies(const convt_plan &Pl, WtParams &P) {
    const AxisPlan &AD = Pl.ax[0], &AH = Pl.ax[1], &AW = Pl.ax[2];
    if (Pl.ndim < 2 || Pl.Cig % 32 != 0 || Pl.Cog % 4 != 0 || Pl.k_vol > 64) return false;
    if (AW.L_in != 16 && AW.L_in != 32 && AW.L_in != 64) return false;
    if (4 * Pl.C_out * Pl.out_sp > 0x7fffffff || 4 * Pl.C_in * Pl.in_sp > 0x7fffffff) return false;
    if (4 * Pl.out_sp + (int64_t)AD.K * AD.d * AH.L_out * AW.L_out >= ((int64_t)1 << 26)) return false;
    P.R = kWtPos / AW.L_in;
    P.NR = (P.R - 1) * AH.s + (AH.K - 1) * AH.d + 1;
    P.NW = (AW.L_in - 1) * AW.s + (AW.K - 1) * AW.d + 1;
    const int cap = Pl.k_vol > 32 ? kWtWinCap2 : kWtWinCap;
    if (AD.K * P.NR > 63 || AD.K * 4 * P.NR * P.NW > cap) return false;
    return true;
}

int launch_weight_stage(const convt_plan &Pl, const float *x, const float *dy, float *dw, hipStream_t st) {
    WtParams P;
    if (!weight_stage_applies(Pl, P)) return (int)hipErrorInvalidValue;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.Cig = (int)Pl.Cig;
    P.Cog = (int)Pl.Cog;
    P.kvol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    P.nhb = (Pl.ax[1].L_in + P.R - 1) / P.R;
    P.ccs = (int)(Pl.Cig / 32);
    P.NQ = (int)(Pl.Cog / 4);
    P.TG = (int)((Pl.k_vol + 3) / 4);
    const int64_t blocks = Pl.N * Pl.G * (int64_t)P.ccs * P.NQ;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    const AxisPlan &AD = Pl.ax[0], &AH = Pl.ax[1], &AW = Pl.ax[2];
    const bool fix = AW.L_in == 16 && AD.K == 3 && AH.K == 3 && AW.K == 3 && AH.s == 2 && AW.s == 2 && AH.d == 1 &&
                     AW.d == 1;
    const bool fix2 = AW.L_in == 32 && AD.K == 4 && AH.K == 4 && AW.K == 4 && AH.s == 2 && AW.s == 2 && AH.d == 1 &&
                      AW.d == 1;
    const bool two = P.TG > 8;
    const size_t lds = sizeof(float) * ((two ? kWtWinCap2 : kWtWinCap) + 32 * kWtXP);
    if (fix)
        hipLaunchKernelGGL((k_backward_weight_stage<1, 1>), dim3((unsigned)blocks), dim3(kWtNT), lds, st, P, x, dy, dw);
    else if (fix2)
        hipLaunchKernelGGL((k_backward_weight_stage<2, 2>), dim3((unsigned)blocks), dim3(kWtNT), lds, st, P, x, dy, dw);
    else if (two)
        hipLaunchKernelGGL((k_backward_weight_stage<2, 0>), dim3((unsigned)blocks), dim3(kWtNT), lds, st, P, x, dy, dw);
    else
        hipLaunchKernelGGL((k_backward_weight_stage<1, 0>), dim3((unsigned)blocks), dim3(kWtNT), lds, st, P, x, dy, dw);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

// db[co] += the sum of dy[n, co, e] over one chunk of kBiasChunk positions e
// per workgroup, grid (co, chunk, n).  Each thread keeps kBiasDepth partial
// sums, so that many loads are in flight; a pairwise tree, a wave tree and an
// atomic add finish the chunk.
constexpr int kBiasChunk = 16384;
constexpr int kBiasDepth = 16;
__global__ __launch_bounds__(kWgBlock) void k_backward_bias(const float *__restrict__ dy, float *db, int C_out,
                                                            int out_sp) {
    const int co = blockIdx.x, n = blockIdx.z;
    const float *row = dy + ((int64_t)n * C_out + co) * out_sp;
    const int e0 = blockIdx.y * kBiasChunk;
    const int e1 = min(e0 + kBiasChunk, out_sp);
    float sp[kBiasDepth];
#pragma unroll
    for (int u = 0; u < kBiasDepth; ++u) sp[u] = 0.0f;
    for (int e = e0 + threadIdx.x; e < e1; e += kBiasDepth * kWgBlock) {
#pragma unroll
        for (int u = 0; u < kBiasDepth; ++u) {
            // unconditional loads (a clamped index; past the chunk the value
            // is dropped), so all of them are in flight at once
            const int i = e + u * kWgBlock;
            const float v = row[min(i, e1 - 1)];
            sp[u] += i < e1 ? v : 0.0f;
        }
    }
#pragma unroll
    for (int h = kBiasDepth / 2; h >= 1; h /= 2)
#pragma unroll
        for (int u = 0; u < h; ++u) sp[u] += sp[u + h];
    float s = sp[0];
    __shared__ float part[kWgBlock / 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(db + co, (part[0] + part[1]) + (part[2] + part[3]));
}

__global__ void k_fill_zero(float *p, int64_t n) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
        p[e] = 0.0f;
}

constexpr int kWgTaps = 2; // taps per wave

template <int CTW, int OTW>
int launch_w(const convt_plan &Pl, WgradParams &P, const float *x, const float *dy, float *dw, hipStream_t st) {
    P.kchunks = (int)((Pl.k_vol + kWgTaps - 1) / kWgTaps);
    P.units = Pl.N * Pl.G * (int64_t)(P.CT / CTW) * (P.OT / OTW) * P.kchunks * P.nranges;
    const int64_t blocks = (P.units + kWgBlock / 64 - 1) / (kWgBlock / 64);
    hipLaunchKernelGGL((k_backward_weight<CTW, OTW, kWgTaps>), dim3((unsigned)blocks), dim3(kWgBlock), 0, st, P, x,
                       dy, dw);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

} // namespace

const char *backward_weight_kernel_name(const convt_plan &P) {
    WrParams R;
    if (weight_row_window(P, R)) return "k_backward_weight_row";
    WtParams T;
    if (CONVT_WT_STAGE && weight_stage_applies(P, T)) return "k_backward_weight_stage";
    if (weight_shift_rows_applies(P)) return "k_backward_weight_shift_rows";
    if (weight_shift_applies(P)) return "k_backward_weight_shift";
    return P.Cig % 32 == 0 && P.Cog % 64 == 0 ? "k_backward_weight_lds" : "k_backward_weight";
}

bool backward_weight_supports(const convt_plan &P) {
    if (4 * P.Cig * P.in_sp > 0x7fffffff || 4 * P.Cog * P.out_sp > 0x7fffffff) return false;
    const int64_t CT = (P.Cig + 15) / 16, OT = (P.Cog + 15) / 16;
    const int64_t units = P.N * P.G * CT * OT * ((P.k_vol + kWgTaps - 1) / kWgTaps) *
                          ((P.in_sp + kWgRange - 1) / kWgRange);
    return units / (kWgBlock / 64) < 0x7fffffff && P.N <= 65535 && P.C_out <= 0x7fffffff;
}

int launch_backward_weight(const convt_plan &Pl, const float *x, const float *dy, float *dw, float *db,
                           void *stream) {
    hipStream_t st = (hipStream_t)stream;
    const int64_t nw = Pl.C_in * Pl.Cog * Pl.k_vol;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((nw + 255) / 256 < 4096 ? (nw + 255) / 256 : 4096)), dim3(256), 0,
                       st, dw, nw);
    if (db) hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(256), 0, st, db, Pl.C_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;

    WgradParams P;
    for (int a = 0; a < kAxes; ++a) P.ax[a] = Pl.ax[a];
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.Cig = (int)Pl.Cig;
    P.Cog = (int)Pl.Cog;
    P.k_vol = (int)Pl.k_vol;
    P.in_sp = (int)Pl.in_sp;
    P.out_sp = (int)Pl.out_sp;
    P.CT = (int)((Pl.Cig + 15) / 16);
    P.OT = (int)((Pl.Cog + 15) / 16);
    P.nranges = (int)((Pl.in_sp + kWgRange - 1) / kWgRange);
    int rc;
    WtParams T;
    WrParams R0;
    if (CONVT_WT_STAGE && !weight_row_window(Pl, R0) && weight_stage_applies(Pl, T)) {
        rc = launch_weight_stage(Pl, x, dy, dw, st);
    } else if (Pl.Cig % 32 == 0 && Pl.Cog % 64 == 0) {
        WlParams L;
        for (int a = 0; a < kAxes; ++a) L.ax[a] = Pl.ax[a];
        L.C_in = P.C_in, L.C_out = P.C_out, L.Cig = P.Cig, L.Cog = P.Cog, L.k_vol = P.k_vol;
        L.in_sp = P.in_sp, L.out_sp = P.out_sp;
        L.cib = (int)(Pl.Cig / 32);
        L.cob = (int)(Pl.Cog / 64);
        L.kchunks = (int)((Pl.k_vol + kWlTaps - 1) / kWlTaps);
        L.nranges = (int)((Pl.in_sp + kWlRange - 1) / kWlRange);
        const int64_t blocks = Pl.N * Pl.G * (int64_t)L.cib * L.cob * L.kchunks * L.nranges;
        WrParams R;
        if (weight_row_window(Pl, R)) {
            R.L = L;
            const size_t lds = (size_t)(kWlTile * kWlApitch + R.win_cols * kWlBpitch) * sizeof(float);
            hipLaunchKernelGGL(k_backward_weight_row, dim3((unsigned)blocks), dim3(kWgBlock), lds, st, R, x, dy, dw);
        } else {
            hipLaunchKernelGGL(k_backward_weight_lds, dim3((unsigned)blocks), dim3(kWgBlock), 0, st, L, x, dy, dw);
        }
        e = hipGetLastError();
        rc = e == hipSuccess ? 0 : (int)e;
    } else if (weight_shift_rows_applies(Pl)) {
        rc = launch_weight_shift_rows(Pl, x, dy, dw, st);
    } else if (weight_shift_applies(Pl)) {
        rc = launch_weight_shift(Pl, x, dy, dw, st);
    } else {
        rc = (P.CT % 2 == 0 && P.OT % 4 == 0) ? launch_w<2, 4>(Pl, P, x, dy, dw, st)
                                              : launch_w<1, 1>(Pl, P, x, dy, dw, st);
    }
    if (rc || !db) return rc;
    const unsigned chunks = (unsigned)((Pl.out_sp + kBiasChunk - 1) / kBiasChunk);
    hipLaunchKernelGGL(k_backward_bias, dim3((unsigned)Pl.C_out, chunks, (unsigned)Pl.N), dim3(kWgBlock), 0, st, dy,
                       db, (int)Pl.C_out, (int)Pl.out_sp);
    e = hipGetLastError();
    return e == hipSuccess ? 0 : (int)e;
}

} // namespace convt
