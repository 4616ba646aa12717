// 3D path: per-phase implicit GEMM on fp32 MFMA (v_mfma_f32_16x16x4_f32).
//
// Method.  On each axis the residue r of o + p mod s selects a dense tap set
// T_r with input offsets c (convt_internal.h).  An output row (n, od, oh) has
// one D phase and one H phase; together they form its class, whose taps
// T_d x T_h are the same for every row of the class.  Along W the S_W phases
// interleave inside the row.  Per class the work is a GEMM
//   Y[co, (n, qd, qh, qw)] = sum_{ci, kd in T_d, kh in T_h, kw in T_w(rw)}
//        W[ci, co, kd, kh, kw] * X[ci, qd - c_kd, qh - c_kh, qw - c_kw]
// with M = C_out, N = positions, K = C_in * taps.
// "Kimi-K2.6 l1_p72" transcript (ConvTranspose3d, groups 4): the parity-class
// blocking (a block never mixes classes, so trip counts stay uniform) and the
// reuse of one input value across all output channels of a position;
// "Kimi-K2.6 l2_p26" transcript (ConvTranspose3d + add + HardSwish): outputs
// with one or two taps per axis, and the fused epilogue.
//
// Mapping.  A workgroup holds one class and walks a run of its output rows.
// Wave w owns output channels 16w .. 16w+15; the class's weights for those
// channels stay in VGPRs (A operand, W^T: 16 co x 4 ci).  The input rows
// x[n, :, qd - c_kd, qh - c_kh, :] of all D/H taps of the next output row are
// fetched into registers during the current row's contraction, then written
// to LDS (double buffer); B operands (4 ci x 16 positions) are read from
// there, zero outside the input.  For W phase rw the first position
// qw0(rw) = max(0, ceil((p_w - rw)/S_W)) gives output sigma(rw) =
// qw0*S_W + rw - p_w in [0, S_W), so lane j of W-block t holds the outputs
// ow = S_W*(16t + j) + sigma(rw): S_W consecutive outputs of one row per lane,
// one vector store per channel.  Atomic-free: every output is stored once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <type_traits>
#include <utility>

#include "convt_internal.h"
#include "epilogue.hpp"

namespace convt {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ f4 load4u(const float *p) {
    f4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// Tuning knobs: workgroups aimed for per CU when sizing the rows per block,
// and the most rows one block walks.
#ifndef CONVT_IG_BLOCKS_PER_CU
#define CONVT_IG_BLOCKS_PER_CU 4
#endif
#ifndef CONVT_IG_MAX_ROWS
#define CONVT_IG_MAX_ROWS 256
#endif

// Tuning knob: each XCD walks a contiguous range of a class's row chunks.
#ifndef CONVT_IG_XCD_ORDER
#define CONVT_IG_XCD_ORDER 1
#endif

// Tuning knob: classes with one or two D x H taps take 4 or 2 rows per step.
#ifndef CONVT_IG_MULTIROW
#define CONVT_IG_MULTIROW 1
#endif

// Tuning knob: minimum waves per SIMD the register allocation must allow.
#ifndef CONVT_IG_WAVES_PER_EU
#define CONVT_IG_WAVES_PER_EU 3
#endif

constexpr int kMaxClasses = 16;
constexpr int kXcds = 8; // accelerator complex dies (each with its own L2) per device
constexpr int kTapMax = 4; // per-axis taps per class the table holds
constexpr int kMaxSW = 8;

template <int K, int S, int D> struct WPhases {
    static constexpr int r_of(int k) { return (k * D) % S; }
    static constexpr int c_of(int k) { return (k * D) / S; }
    static constexpr bool nonempty(int r) {
        for (int k = 0; k < K; ++k)
            if (r_of(k) == r) return true;
        return false;
    }
    static constexpr int slot(int r) {
        int n = 0;
        for (int q = 0; q < r; ++q) n += nonempty(q) ? 1 : 0;
        return n;
    }
    static constexpr int count() {
        int n = 0;
        for (int r = 0; r < S; ++r) n += nonempty(r) ? 1 : 0;
        return n;
    }
    static constexpr int cmax() {
        int m = 0;
        for (int k = 0; k < K; ++k) m = c_of(k) > m ? c_of(k) : m;
        return m;
    }
    static constexpr int first_k(int r) { // first tap of phase r
        for (int k = 0; k < K; ++k)
            if (r_of(k) == r) return k;
        return -1;
    }
};

struct Igemm3dParams {
    int C_in, C_out;
    int D_in, H_in, W_in, D_out, H_out, W_out;
    int KD, KH;          // kernel extents along D and H (W is a template constant)
    int s_d, s_h;
    int n_class;
    int rows_per_block;
    int iw_lo;           // input position held at LDS offset 0 (multiple of 4, <= 0)
    int nwb;             // W-blocks of 16*S_W outputs per row (equals the template's NWBM)
    int qw0[kMaxSW], sigma[kMaxSW];
    int cls_block0[kMaxClasses + 1]; // classes ordered heaviest first
    int cls_chunks[kMaxClasses];     // row chunks (rows_per_block rows each) per class
    int xcd_order;                   // 1: each XCD walks a contiguous range of a class's chunks
    int x_bytes;                     // bytes of x (wide variant: one buffer resource over it)
    int wseg;                        // wide variant: W segments of 16*NWB input positions per row
    int G, Cig, Cog;                 // wide variant: groups and channels per group
    int wnf;                         // wide variant: float4s staged per input row and segment
    int cls_rows[kMaxClasses];
    int cls_rstep[kMaxClasses]; // output rows per step: 1, or 4 / taps for classes of 1 or 2 D x H taps
    int cls_td[kMaxClasses], cls_th[kMaxClasses];
    int cls_kd[kMaxClasses][kTapMax], cls_cd[kMaxClasses][kTapMax];
    int cls_kh[kMaxClasses][kTapMax], cls_ch[kMaxClasses][kTapMax];
    int cls_od0[kMaxClasses], cls_qd0[kMaxClasses], cls_nqd[kMaxClasses];
    int cls_oh0[kMaxClasses], cls_qh0[kMaxClasses], cls_nqh[kMaxClasses];
};

struct RowPos {
    int n, qd, qh, od, oh;
};

__device__ __forceinline__ RowPos decode_row(const Igemm3dParams &P, int cls, int r) {
    const int nqh = P.cls_nqh[cls], nqd = P.cls_nqd[cls];
    const int iqh = r % nqh;
    const int t = r / nqh;
    const int iqd = t % nqd;
    RowPos R;
    R.n = t / nqd;
    R.qd = P.cls_qd0[cls] + iqd;
    R.qh = P.cls_qh0[cls] + iqh;
    R.od = P.cls_od0[cls] + iqd * P.s_d;
    R.oh = P.cls_oh0[cls] + iqh * P.s_h;
    return R;
}

// A row of a class as (sample, D and H input positions relative to the
// class's first), advanced row by row without dividing.
struct RowCur {
    int n, iqd, iqh;
};
__device__ __forceinline__ RowCur cursor_at(const Igemm3dParams &P, int cls, int r) {
    const int nqh = P.cls_nqh[cls], nqd = P.cls_nqd[cls];
    const int t = r / nqh;
    return RowCur{t / nqd, t % nqd, r % nqh};
}
__device__ __forceinline__ void cursor_next(const Igemm3dParams &P, int cls, RowCur &c) {
    if (++c.iqh == P.cls_nqh[cls]) {
        c.iqh = 0;
        if (++c.iqd == P.cls_nqd[cls]) {
            c.iqd = 0;
            ++c.n;
        }
    }
}
__device__ __forceinline__ RowPos row_at(const Igemm3dParams &P, int cls, const RowCur &c) {
    RowPos R;
    R.n = c.n;
    R.qd = P.cls_qd0[cls] + c.iqd;
    R.qh = P.cls_qh0[cls] + c.iqh;
    R.od = P.cls_od0[cls] + c.iqd * P.s_d;
    R.oh = P.cls_oh0[cls] + c.iqh * P.s_h;
    return R;
}

// Buffer resources: a load past num_records returns zeros and a store past it
// is dropped, so input rows outside the input need no select, and lanes past
// a row end read harmlessly.  One resource per sample keeps every byte offset
// within 31 bits (checked on the host).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000; // raw (untyped) buffer access
constexpr unsigned kOutOfRange = 0x80000000u;
// Cache policy nt (non-temporal) for the output stores, as y is written once
// and not read back here (fused layer 0.673 -> 0.666 ms), and for the
// add_input loads below.
constexpr int kNonTemporal = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ f4 buf_load4(rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// add_input loads (buf_load1/2) are non-temporal as well: each element is
// read once, and keeping it out of the caches leaves them to the input rows
// that other classes read again (fused layer 0.678 -> 0.667 ms warm, cold
// cache 0.72 -> 0.70 ms).
__device__ __forceinline__ float buf_load1(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal));
}
typedef float fl2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ fl2 buf_load2(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(fl2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNonTemporal));
}
__device__ __forceinline__ void buf_store1(float v, rsrc_t r, unsigned voff, unsigned soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, voff, soff, kNonTemporal);
}
typedef int i2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void buf_store2(float a, float b, rsrc_t r, unsigned voff, unsigned soff) {
    __builtin_amdgcn_raw_buffer_store_b64(i2{__float_as_int(a), __float_as_int(b)}, r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ f4 buf_load4nt(rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kNonTemporal));
}
__device__ __forceinline__ void buf_store4(f4 v, rsrc_t r, unsigned voff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, v), r, voff,
                                           0, kNonTemporal);
}

template <int CIG, int COG, int KW, int SW, int DW, int TDM, int THM, int NWBM, int PWM, int PER,
          int EPI, bool FULLW, bool SWAP, bool LAST>
__global__ __launch_bounds__(COG * 4)
__attribute__((amdgpu_waves_per_eu(CONVT_IG_WAVES_PER_EU))) void k_igemm3d(const Igemm3dParams P,
                                                     const float *__restrict__ x,
                                                     const float *__restrict__ w,
                                                     const float *__restrict__ bias,
                                                     const float *add, float *y) {
    using Ph = WPhases<KW, SW, DW>;
    constexpr bool FUSED = epi_add(EPI); // add_input is read
    constexpr int NCIG = CIG / 4;
    constexpr int NT = COG * 4;
    constexpr int SLOTS = TDM * THM;
    constexpr int NPH = Ph::count() > 0 ? Ph::count() : 1;
    static_assert(CIG % 8 == 0 && COG % 16 == 0, "tile shape");
    static_assert(SW <= kMaxSW, "W stride");
    // Staged input rows.  Channels first: [slot][ci][w] with a pitch of PWM
    // floats per channel row.  Channels last (LAST): [slot][w][ci] with a
    // pitch of CIG + 4 floats per position (the 16 positions x 4 channels of
    // one B read then fall on distinct banks, and an input float4 of 4
    // channels is one aligned LDS store), PWN positions per slot.
    constexpr int PCL = CIG + 4;
    constexpr int PWN = 16 * NWBM + 8;
    constexpr int SLOT_SZ = LAST ? PWN * PCL : CIG * PWM;
    __shared__ __attribute__((aligned(16))) float lds[2][SLOTS * SLOT_SZ];
    // Channels last: the output row's 16*SW*NWBM positions x COG channels,
    // staged across the waves so that one store instruction writes 1 KB of
    // whole lines; float4 column c4 of position row p sits at c4 ^ key(p),
    // key(p) = (p / SW) mod (COG/4), so the accumulator writes (16 lanes j of
    // one g4: rows SW*j + const) and the row reads hit distinct banks.
    constexpr int OPOS = 16 * SW * NWBM;
    constexpr int OC4 = COG / 4;
    constexpr int NSO = LAST ? OPOS * OC4 / NT : 1; // staged float4 each thread stores
    static_assert(!LAST || (OPOS * OC4) % NT == 0, "output staging split");
    __shared__ __attribute__((aligned(16))) float ost[LAST ? OPOS * COG : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ct = tid >> 6;
    const int j = lane & 15;
    const int g4 = lane >> 4;

    int cls = 0;
    while (cls + 1 < P.n_class && (int)blockIdx.x >= P.cls_block0[cls + 1]) ++cls;
    int chunk = (int)blockIdx.x - P.cls_block0[cls];
    if (P.xcd_order) {
        // Blocks go to the XCDs round robin, so block k of the class runs on XCD
        // (k mod 8) up to a fixed rotation; give each XCD a contiguous range of
        // chunks, walked in order, so blocks running together on one L2 share
        // the input rows at their chunk boundaries.
        const int per = (P.cls_chunks[cls] + kXcds - 1) / kXcds;
        chunk = (chunk % kXcds) * per + chunk / kXcds;
    }
    const int r_begin = chunk * P.rows_per_block;
    const int r_end = min(r_begin + P.rows_per_block, P.cls_rows[cls]);
    if (r_begin >= r_end) return;
    const int td = P.cls_td[cls], th = P.cls_th[cls];
    // Rows per step.  A class with one or two D x H taps (set by the host when
    // its H run length allows) takes 4 or 2 consecutive rows along H per step,
    // so that its steps issue as many MFMAs as those of a four-tap class and
    // the per-step costs (row set-up, barrier, waits) are shared.  Its LDS
    // slot s then holds tap t = s mod taps of row s / taps, and its weights
    // sit in tap order (tap t at flat slot t, whether the taps lie along D
    // or H).
    const int ntaps = td * th;
    const bool flat = P.cls_rstep[cls] > 1;
    // flat slot t of a one- or two-tap class -> its (D tap, H tap)
    auto flat_tap = [&](int t, int &ajd, int &ajh) {
        ajd = th == 1 ? t : 0;
        ajh = th == 1 ? 0 : t;
    };

    // zero both buffers once: halo columns and unused slots stay zero
    for (int i = tid; i < 2 * SLOTS * SLOT_SZ; i += NT) (&lds[0][0])[i] = 0.0f;

    // the class's weights for this wave's channels: W[4cig + g4][16ct + j][kd][kh][kw]
    // The class's weights for this wave's channels, W[4cig + g4][16ct + j][kd]
    // [kh][kw], into flat tap slots 0 .. NW-1 (each step mode loads its own
    // set, so that the register allocator sees one set per mode).
    auto load_weights = [&](float (&wr)[TDM][THM][KW][NCIG], auto nwc) {
        constexpr int NW = decltype(nwc)::value;
#pragma unroll
        for (int jd = 0; jd < TDM; ++jd)
#pragma unroll
            for (int jh = 0; jh < THM; ++jh) {
                if (jd * THM + jh >= NW) continue;
                bool used = jd < td && jh < th;
                int ajd = jd, ajh = jh;
                if (flat) {
                    used = jd * THM + jh < ntaps;
                    flat_tap(jd * THM + jh, ajd, ajh);
                }
                const int kd = used ? P.cls_kd[cls][ajd] : 0;
                const int kh = used ? P.cls_kh[cls][ajh] : 0;
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int cig = 0; cig < NCIG; ++cig) {
                        const int64_t idx =
                            ((((int64_t)(4 * cig + g4) * COG + 16 * ct + j) * P.KD + kd) * P.KH + kh) *
                                KW + kw;
                        const float v = w[idx];
                        wr[jd][jh][kw][cig] = used ? v : 0.0f;
                    }
            }
        // wait for these here, not inside the row loop (vmcnt is in order)
#pragma unroll
        for (int jd = 0; jd < TDM; ++jd)
#pragma unroll
            for (int jh = 0; jh < THM; ++jh)
#pragma unroll
                for (int kw = 0; kw < KW; ++kw)
#pragma unroll
                    for (int cig = 0; cig < NCIG; ++cig)
                        if (jd * THM + jh < NW) asm volatile("" : "+v"(wr[jd][jh][kw][cig]));
    };
    float bo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bo[e] = bias ? bias[16 * ct + 4 * g4 + e] : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(bo[e]));

    static_assert(TDM <= 2 && THM <= 2, "tap offsets are selected from two registers");
    const int cd0 = P.cls_cd[cls][0], cd1 = P.cls_cd[cls][1];
    const int ch0 = P.cls_ch[cls][0], ch1 = P.cls_ch[cls][1];
    const int dhw = P.D_in * P.H_in * P.W_in;
    const int64_t dhw_out = (int64_t)P.D_out * P.H_out * P.W_out;

    // Input rows of one output row: SLOTS x CIG rows of W_in floats.  Thread
    // tid stages float4 number f = tid + u*NT, whose meaning does not depend on
    // the row: tap slot (jd, jh), channel ci, float4 c4.  Its byte offset in
    // the sample is 4*((qd*H_in + qh)*W_in) + xo4, valid when the slot's tap
    // exists in the class and its input row lies inside the input (one bit per
    // slot, the same for the whole workgroup).
    // The float4s are numbered H tap slot first (jh, then jd, channel, float4),
    // so that when they split evenly the second half of a thread's float4s are
    // all of the second H tap (see the sliding rows below).
    int xo4[PER], lo[PER], tb[PER];
    if constexpr (LAST) {
        // channels last: float4 f is 4 channels (CIG/4 of them per position,
        // fastest) of one input position of one tap slot's row
        constexpr int CQ = CIG / 4;
        const int nf = SLOTS * CQ * P.W_in;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int f = tid + u * NT;
            const int sq = f / (CQ * P.W_in); // jh * TDM + jd
            const int rem = f - sq * (CQ * P.W_in);
            const int iw = rem / CQ, cq = rem - iw * CQ;
            const int jh = sq / TDM, jd = sq % TDM;
            const int slot = jd * THM + jh;
            const int cd = jd == 0 ? cd0 : cd1, ch = jh == 0 ? ch0 : ch1;
            xo4[u] = 4 * ((iw - (cd * P.H_in + ch) * P.W_in) * CIG + 4 * cq);
            lo[u] = f < nf ? slot * SLOT_SZ + (iw - P.iw_lo) * PCL + 4 * cq : -1;
            tb[u] = f < nf ? slot : 31;
        }
    } else {
        const int W4 = P.W_in >> 2;
        const int nf = SLOTS * CIG * W4;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int f = tid + u * NT;
            const int sq = f / (CIG * W4); // jh * TDM + jd
            const int rem = f - sq * (CIG * W4);
            const int ci = rem / W4, c4 = rem - ci * W4;
            const int jh = sq / TDM, jd = sq % TDM;
            const int slot = jd * THM + jh;
            int cd = jd == 0 ? cd0 : cd1, ch = jh == 0 ? ch0 : ch1, q = 0;
            if (flat) { // tap slot % taps of row slot / taps
                q = ntaps == 1 ? slot : slot >> 1;
                int ajd, ajh;
                flat_tap(slot - q * ntaps, ajd, ajh);
                cd = ajd == 0 ? cd0 : cd1;
                ch = ajh == 0 ? ch0 : ch1;
            }
            xo4[u] = 4 * (ci * dhw + 4 * c4 - (cd * P.H_in + ch - q) * P.W_in);
            lo[u] = f < nf ? (slot * CIG + ci) * PWM + 4 * c4 - P.iw_lo : -1;
            tb[u] = f < nf ? slot : 31;
        }
    }
    const int xbytes = 4 * P.C_in * dhw;
    // Sliding rows: when the class has two H taps at offsets c and c+1 and
    // the float4s split evenly by H tap, a row that follows the previous row
    // of its chunk along H (same sample and D position, qh one higher) needs
    // as its second H tap's input rows the first H tap's rows of that
    // previous row, which are still in the other LDS buffer when the row is
    // staged: they are copied from there, and their loads are issued out of
    // range (no traffic; the number of loads per row stays fixed, which keeps
    // the compiler's wait counts exact).
    const bool slide_ok = !flat && THM == 2 && PER % 2 == 0 && th == 2 && ch1 == ch0 + 1 &&
                          SLOTS * (CIG / 4) * P.W_in == PER * NT;
    // Per LDS slot s = jd*THM + jh: the input row it holds, relative to the
    // step's (first) row, at D offset sdd[s] and H offset sdh[s]; bit s of
    // sused is set when the class uses the slot.
    int sdd[SLOTS], sdh[SLOTS];
    unsigned sused = 0;
#pragma unroll
    for (int jd = 0; jd < TDM; ++jd)
#pragma unroll
        for (int jh = 0; jh < THM; ++jh) {
            const int sl = jd * THM + jh;
            int ajd = jd, ajh = jh, q = 0;
            bool used = jd < td && jh < th;
            if (flat) {
                q = ntaps == 1 ? sl : sl >> 1;
                flat_tap(sl - q * ntaps, ajd, ajh);
                used = true;
            }
            sdd[sl] = -(ajd == 0 ? cd0 : cd1);
            sdh[sl] = q - (ajh == 0 ? ch0 : ch1);
            sused |= (unsigned)used << sl;
        }
    // row k (at cursor c) slides unless it starts its chunk or an H run
    auto slide_of = [&](int k, const RowCur &c) { return slide_ok && k > r_begin && c.iqh != 0; };
    auto fetch_rows = [&](f4 (&rv)[PER], const RowPos &Q, bool slide) {
        unsigned bad = 0xffffffffu; // bit slot clear: the slot's input row exists
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            const int id = Q.qd + sdd[sl], ih = Q.qh + sdh[sl];
            // bitwise, not short-circuit: no branch per condition
            const bool ok = ((sused >> sl) & 1u) & ((unsigned)id < (unsigned)P.D_in) &
                            ((unsigned)ih < (unsigned)P.H_in) & !(slide & (sl % THM == 1));
            bad &= ~((unsigned)ok << sl);
        }
        const rsrc_t rx = make_rsrc(x + (int64_t)Q.n * P.C_in * dhw, xbytes);
        const int rowx4 = 4 * (Q.qd * P.H_in + Q.qh) * P.W_in * (LAST ? CIG : 1);
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            // an invalid slot gets bit 31 set: past num_records, the load returns zeros
            const unsigned off = ((bad >> tb[u]) << 31) | (unsigned)(rowx4 + xo4[u]);
            rv[u] = buf_load4(rx, off);
        }
    };
    auto store_rows = [&](float *lbuf, const f4 (&rv)[PER], bool slide, const float *lprev) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            f4 v = rv[u];
            if (u >= PER / 2 && slide && lo[u] >= 0) // second H tap: the previous row's first (one slot back)
                v = *reinterpret_cast<const f4 *>(lprev + lo[u] - SLOT_SZ);
            if (lo[u] >= 0) *reinterpret_cast<f4 *>(lbuf + lo[u]) = v;
        }
    };

    // Outputs of lane (g4, j): channel 16ct + 4g4 + e (scalar offset e*dhw_out),
    // W position SW*(16t + j) + rr (immediate offset), at the row's offset
    // (od*H_out + oh)*W_out.  Lanes past the row end read the next row or
    // nothing and store nothing.
    const int ybytes = (int)(4 * P.C_out * dhw_out);
    const unsigned lane4 = 4u * (unsigned)((16 * ct + 4 * g4) * dhw_out + SW * j);
    const unsigned e4 = 4u * (unsigned)dhw_out;
    auto row_off4 = [&](const RowPos &Q) {
        return 4u * (unsigned)((Q.od * P.H_out + Q.oh) * P.W_out * (LAST ? COG : 1));
    };
    // Channels last: the staged float4 f = NT*u + tid of an output row is
    // position f / OC4, channels 4*(f % OC4) .. +3; its byte offset in the row,
    // or past the resource for positions beyond the row end.
    unsigned lst[NSO];
    if constexpr (LAST) {
#pragma unroll
        for (int u = 0; u < NSO; ++u) {
            const int f = NT * u + tid, pp = f / OC4, c4 = f % OC4;
            lst[u] = pp < P.W_out ? 4u * (unsigned)(pp * COG + 4 * c4) : kOutOfRange;
        }
    }
    // add_input registers of one output row; the multi-row modes hold up to 4
    using AddRegs = std::conditional_t<LAST, f4[NSO], float[NWBM][4][SW]>;
    constexpr bool MULTI = !LAST && SLOTS == 4 && NWBM == 1; // multi-row steps compiled in
    constexpr int RMAX = MULTI ? 4 : 1;
    // byte offset of the next output row along H (rows of a multi-row step)
    const unsigned dhy4 = 4u * (unsigned)(P.s_h * P.W_out * (LAST ? COG : 1));
    auto fetch_add = [&](AddRegs &a, const RowPos &Q, unsigned dq) {
        const rsrc_t ra = make_rsrc(add + (int64_t)Q.n * P.C_out * dhw_out, ybytes);
        if constexpr (LAST) {
#pragma unroll
            for (int u = 0; u < NSO; ++u) a[u] = buf_load4nt(ra, row_off4(Q) + dq + lst[u]);
            return;
        } else {
        const unsigned vo = lane4 + row_off4(Q) + dq;
#pragma unroll
        for (int t = 0; t < NWBM; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (SW == 2) { // the lane's two outputs are adjacent: one 8-byte load
                    const fl2 v = buf_load2(ra, vo + 4 * SW * 16 * t, e * e4);
                    a[t][e][0] = v.x;
                    a[t][e][1] = v.y;
                } else {
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr)
                        a[t][e][rr] = buf_load1(ra, vo + 4 * (SW * 16 * t + rr), e * e4);
                }
            }
        }
    };

    const f4 bias4 = f4{bo[0], bo[1], bo[2], bo[3]};
    static_assert(!SWAP || SW == 2, "the phase swap is for two W phases");

    // Epilogue of one output row (its accumulators ac, add_input a, byte
    // offset dq past row R): lane (g4, j) owns co = 16ct + 4g4 + e,
    // ow = SW*(16t + j) + rr.  W phase 0 on the odd outputs (swapped) is
    // fixed for the launch, so a template flag (as a runtime flag the
    // compiler turns the two orders into per-element selects).
    auto epi_row = [&](const RowPos &R, const f4 (&ac)[NPH][NWBM], const AddRegs &a, unsigned dq, auto swapped) {
        const rsrc_t ry = make_rsrc(y + (int64_t)R.n * P.C_out * dhw_out, ybytes);
        const unsigned vo_row = row_off4(R) + dq;
        const unsigned vo = lane4 + vo_row;
#pragma unroll
        for (int t = 0; t < NWBM; ++t) {
            const int ow0 = SW * (16 * t + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v[SW];
                if constexpr (SW == 2 && NPH == 2) {
                    v[0] = ac[decltype(swapped)::value ? 1 : 0][t][e];
                    v[1] = ac[decltype(swapped)::value ? 0 : 1][t][e];
                } else {
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr) v[rr] = bo[e];
#pragma unroll
                    for (int rw = 0; rw < SW; ++rw) {
                        if constexpr (Ph::count() > 0) {
                            if (Ph::nonempty(rw)) {
                                const float av = ac[Ph::slot(rw)][t][e];
#pragma unroll
                                for (int rr = 0; rr < SW; ++rr)
                                    if (P.sigma[rw] == rr) v[rr] = av;
                            }
                        }
                    }
                }
                if constexpr (LAST) { // staged as they are; the epilogue follows the read back
                    const int c4 = (4 * ct + g4) ^ ((16 * t + j) & (OC4 - 1));
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr) ost[(ow0 + rr) * COG + 4 * c4 + e] = v[rr];
                    continue;
                } else {
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr) v[rr] = finish<EPI>(v[rr], FUSED ? a[t][e][rr] : 0.0f);
                }
                const unsigned o = vo + 4 * SW * 16 * t;
                if (FULLW || ow0 + SW <= P.W_out) {
                    if constexpr (SW == 2) {
                        buf_store2(v[0], v[1], ry, o, e * e4);
                    } else {
#pragma unroll
                        for (int rr = 0; rr < SW; ++rr) buf_store1(v[rr], ry, o + 4 * rr, e * e4);
                    }
                } else {
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr)
                        if (ow0 + rr < P.W_out) buf_store1(v[rr], ry, o + 4 * rr, e * e4);
                }
            }
        }
        if constexpr (LAST) {
            __syncthreads();
#pragma unroll
            for (int u = 0; u < NSO; ++u) {
                const int f = NT * u + tid, pp = f / OC4, c4 = f % OC4;
                f4 v = *reinterpret_cast<const f4 *>(&ost[pp * COG + 4 * (c4 ^ ((pp / SW) & (OC4 - 1)))]);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = finish<EPI>(v[e], FUSED ? a[u][e] : 0.0f);
                buf_store4(v, ry, vo_row + lst[u]);
            }
        }
    };

    // Steps of RS rows (template MODE: 0 one row, any taps; 1 or 2 taps per
    // row, 4 / MODE rows along H).  Input rows are fetched two steps ahead,
    // before the current step's stores: the vector-memory counter retires in
    // issue order, so the wait for them then covers only stores issued two
    // steps earlier.  (With rows that every lane fills, FULLW, each path
    // issues the same stores and the compiler's wait counts stay exact.)  Past
    // the block's last step the last step is fetched again, never used.
    auto run = [&](auto modec) {
        constexpr int MODE = decltype(modec)::value;
        constexpr int RS = MODE == 0 ? 1 : 4 / MODE;
        float wr[TDM][THM][KW][NCIG];
        load_weights(wr, std::integral_constant<int, MODE == 0 ? TDM * THM : MODE>{});
        f4 pre0[PER], pre1[PER];
        AddRegs av[RS], avn[RS];
        RowPos R = decode_row(P, cls, r_begin);
        // cursors of the first rows of steps r+RS and r+2RS (clamped to the
        // last step), with their slide flags
        RowCur c1 = cursor_at(P, cls, min(r_begin + RS, r_end - RS));
        RowCur c2 = cursor_at(P, cls, min(r_begin + 2 * RS, r_end - RS));
        bool sl1 = slide_of(min(r_begin + 1, r_end - 1), c1);
        bool sl2 = slide_of(min(r_begin + 2, r_end - 1), c2);
        __syncthreads(); // LDS zeroed before the first row lands
        fetch_rows(pre0, R, false);
        store_rows(lds[0], pre0, false, lds[1]);
        fetch_rows(pre0, row_at(P, cls, c1), sl1);
        if constexpr (FUSED && MODE == 0) fetch_add(av[0], R, 0);
        __syncthreads();

        // One step; the loop below runs it twice per trip with the two
        // add_input register sets swapped, so the prefetched set needs no
        // copy, and with the LDS buffer as a compile-time index (steps
        // alternate between the two buffers), so buffer addresses are
        // immediate offsets.
        auto step = [&](const int r, auto &avc, auto &avp, auto &pre, auto &pre2, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            // Single rows: x rows of row r+2 (into pre2), then add_input of
            // row r+1 (a row ahead).  Multi-row steps: add_input of this
            // step's rows first (their registers would not fit twice; the
            // step's MFMAs cover the latency), then x rows of step r+2RS.  pre
            // holds the x rows of step r+RS, fetched a step earlier.
            const RowPos Rn = row_at(P, cls, c1);
            if constexpr (FUSED && MODE > 0) {
#pragma unroll
                for (int q = 0; q < RS; ++q) fetch_add(avc[q], R, q * dhy4);
            }
            fetch_rows(pre2, row_at(P, cls, c2), sl2);
            if constexpr (FUSED && MODE == 0) fetch_add(avp[0], Rn, 0);

            // The bias enters as the accumulators' start value: the first MFMA
            // of each W phase takes it as its accumulator input.  Rows of a
            // class without taps keep the bias.
            f4 acc[RS][NPH][NWBM];
            if (Ph::count() == 0 || td == 0 || th == 0) {
#pragma unroll
                for (int q = 0; q < RS; ++q)
#pragma unroll
                    for (int s = 0; s < NPH; ++s)
#pragma unroll
                        for (int t = 0; t < NWBM; ++t) acc[q][s][t] = bias4;
            } else if constexpr (Ph::count() > 0) {
                // one base per (W phase, tap shift): the reads below are then the
                // base plus multiples of 64 floats (channel and slot pitches), which
                // paired LDS reads reach without address arithmetic
                // (the empty asm hides how the bases relate, or the compiler would pair
                // reads one float apart and rebuild a base for every pair)
                typedef const __attribute__((address_space(3))) float *lds_ptr;
                constexpr int CM = Ph::cmax() + 1;
                lds_ptr bcol[SW][CM];
#pragma unroll
                for (int rw = 0; rw < SW; ++rw)
#pragma unroll
                    for (int c = 0; c < CM; ++c) {
                        bcol[rw][c] = LAST ? (lds_ptr)(lds[buf] + (j + P.qw0[rw] - c - P.iw_lo) * PCL + g4)
                                           : (lds_ptr)(lds[buf] + g4 * PWM - P.iw_lo + j + P.qw0[rw] - c);
                        asm volatile("" : "+v"(bcol[rw][c]));
                    }
                auto bread = [&](int rw, int c, int slot, int cig, int t) {
                    return LAST ? bcol[rw][c][slot * SLOT_SZ + 4 * cig + 16 * t * PCL]
                                : bcol[rw][c][(slot * CIG + 4 * cig) * PWM + 16 * t];
                };
                if constexpr (MODE == 0) {
#pragma unroll
                    for (int jd = 0; jd < TDM; ++jd) {
                        if (jd > 0 && jd >= td) break;
#pragma unroll
                        for (int jh = 0; jh < THM; ++jh) {
                            if (jh > 0 && jh >= th) break;
                            const int slot = jd * THM + jh;
#pragma unroll
                            for (int cig = 0; cig < NCIG; ++cig) {
#pragma unroll
                                for (int kw = 0; kw < KW; ++kw) {
                                    const int rw = Ph::r_of(kw);
                                    const int sl = Ph::slot(rw);
                                    const int c = Ph::c_of(kw);
#pragma unroll
                                    for (int t = 0; t < NWBM; ++t) {
                                        const bool first = jd == 0 && jh == 0 && cig == 0 && kw == Ph::first_k(rw);
                                        acc[0][sl][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                            wr[jd][jh][kw][cig], bread(rw, c, slot, cig, t),
                                            first ? bias4 : acc[0][sl][t], 0, 0, 0);
                                    }
                                }
                            }
                        }
                    }
                } else {
                    // tap t of row q in slot q*MODE + t; the rows' accumulators
                    // interleave (innermost), so consecutive MFMAs are independent
#pragma unroll
                    for (int tp = 0; tp < MODE; ++tp)
#pragma unroll
                        for (int cig = 0; cig < NCIG; ++cig)
#pragma unroll
                            for (int kw = 0; kw < KW; ++kw) {
                                const int rw = Ph::r_of(kw);
                                const int sl = Ph::slot(rw);
                                const int c = Ph::c_of(kw);
                                const bool first = tp == 0 && cig == 0 && kw == Ph::first_k(rw);
#pragma unroll
                                for (int q = 0; q < RS; ++q)
#pragma unroll
                                    for (int t = 0; t < NWBM; ++t)
                                        acc[q][sl][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                            wr[tp / THM][tp % THM][kw][cig], bread(rw, c, q * MODE + tp, cig, t),
                                            first ? bias4 : acc[q][sl][t], 0, 0, 0);
                            }
                }
            }

            // The next step's inputs go to the other LDS buffer (free since the
            // last barrier) before this step's stores: the vector-memory counter
            // retires in issue order, so the wait for them must not follow the
            // stores.  Unconditional, so that no path leaves them pending into
            // the next step's fetch.
#pragma unroll
            for (int u = 0; u < PER; ++u) asm volatile("" : "+v"(pre[u]));
            store_rows(lds[buf ^ 1], pre, sl1, lds[buf]);

#pragma unroll
            for (int q = 0; q < RS; ++q) epi_row(R, acc[q], avc[q], q * dhy4, std::integral_constant<bool, SWAP>{});

            __syncthreads();
            R = Rn;
            c1 = c2;
            sl1 = sl2;
            if (r + 3 * RS <= r_end - RS) {
                if constexpr (RS == 1) {
                    cursor_next(P, cls, c2);
                } else { // a multi-row class's H runs hold whole steps
                    c2.iqh += RS;
                    if (c2.iqh == P.cls_nqh[cls]) {
                        c2.iqh = 0;
                        if (++c2.iqd == P.cls_nqd[cls]) {
                            c2.iqd = 0;
                            ++c2.n;
                        }
                    }
                }
                sl2 = slide_of(r + 3, c2);
            }
        };
        for (int r = r_begin; r < r_end; r += 2 * RS) {
            step(r, av, avn, pre0, pre1, std::integral_constant<int, 0>{});
            if (r + RS < r_end) step(r + RS, avn, av, pre1, pre0, std::integral_constant<int, 1>{});
        }
    };
    if constexpr (MULTI) {
        if (flat) {
            if (ntaps == 1) run(std::integral_constant<int, 1>{});
            else run(std::integral_constant<int, 2>{});
            return;
        }
    }
    run(std::integral_constant<int, 0>{});
}

// ---------------------------------------------------------------- wide variant
// Channel-heavy layers: the class's weights (C_in x C_out x taps) do not fit in
// VGPRs, so they stream through LDS.  A workgroup of 4 waves owns 4 output
// rows of one class and one block of COB = 16*MT output channels of one group
// (wave w: row w, the block's channels x NWB W-blocks, MT*NWB accumulator
// tiles per W phase); blocks of one row run side by side (channel block
// fastest), so the rows' inputs are read from L2 after the first.  The contraction runs over
// stages (D/H tap slot x chunk of CC input channels, C_in/CC chunks); each
// stage stages the weight chunk and the 4 rows' input rows, double-buffered.
// The weights are staged as [kw][ci][j][m] for channel co = 16m + j of the
// block, so one 8- or 16-byte read gives a lane its MT A operands (W^T: 16 co
// x 4 ci for m < MT); the K_W taps of one (ci, co, kd, kh) are contiguous in
// the weight tensor and come in one 12- or 16-byte load.  Per (ci quad, kw):
// 1 A read and NWB B reads feed MT*NWB MFMAs.  Channels last (NDHWC, CL): a
// staged input row is [position][channel] with a pitch of CC + 4 floats (one
// 16-byte LDS store per 4-channel load; the 16 positions x 4 channels of a B
// read fall on distinct banks), and a lane stores its 4 consecutive output
// channels of a position as one float4.  Rows longer than 16*NWB input
// positions split into W segments (a block each): a segment stages its input
// positions plus the halo its taps reach; positions outside the row are never
// staged and keep the zeros written at the start.  Staging offsets are fixed per thread for the
// block; per stage only a uniform offset changes, and input rows outside the
// input load as zeros through the buffer resource's range check.
// Two workgroups fit a CU's LDS, so two waves per SIMD: the register budget
// that target allows keeps the accumulators in place across stages.
#ifndef CONVT_IGW_WAVES_PER_EU
#define CONVT_IGW_WAVES_PER_EU 2
#endif

// A operands of a lane: MT floats, read from LDS in one access.
template <int MT> struct AVec {
    typedef float t __attribute__((ext_vector_type(MT)));
};
template <> struct AVec<1> {
    typedef float t;
};
template <typename V> __device__ __forceinline__ float aget(const V &a, int m) { return a[m]; }
__device__ __forceinline__ float aget(float a, int) { return a; }

// Row q (0..3) of four held in separate variables, by selects (an array
// indexed with a per-lane value would live in scratch memory).
__device__ __forceinline__ int sel4(int q, int a, int b, int c, int d) {
    return q == 0 ? a : q == 1 ? b : q == 2 ? c : d;
}
__device__ __forceinline__ RowPos pick_row(int q, const RowPos &A, const RowPos &B, const RowPos &C,
                                           const RowPos &D) {
    RowPos o;
    o.n = sel4(q, A.n, B.n, C.n, D.n);
    o.qd = sel4(q, A.qd, B.qd, C.qd, D.qd);
    o.qh = sel4(q, A.qh, B.qh, C.qh, D.qh);
    o.od = sel4(q, A.od, B.od, C.od, D.od);
    o.oh = sel4(q, A.oh, B.oh, C.oh, D.oh);
    return o;
}

template <int KW, int SW, int DW, int NWB, int MT, int CC, int PWX, int EPI, bool CL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CONVT_IGW_WAVES_PER_EU)))
void k_igemm3d_wide(const Igemm3dParams P,
                                                      const float *__restrict__ x,
                                                      const float *__restrict__ w,
                                                      const float *__restrict__ bias,
                                                      const float *add, float *y) {
    using Ph = WPhases<KW, SW, DW>;
    constexpr int COB = 16 * MT;           // output channels of a block
    constexpr int NT = 256;
    constexpr int NPH = Ph::count() > 0 ? Ph::count() : 1;
    constexpr int WPAIRS = CC * COB;       // (ci, co) pairs of a weight chunk
    constexpr int WPER = WPAIRS / NT;      // per thread
    constexpr int XPER = (4 * CC * (PWX / 4) + NT - 1) / NT; // input rows: 4 rows x CC x NF float4s
    static_assert(CC % 4 == 0 && WPAIRS % NT == 0, "chunking");
    static_assert(MT == 1 || MT == 2 || MT == 4, "one 4-, 8- or 16-byte LDS read gives the A operands");
    static_assert(KW == 3 || KW == 4, "one 12- or 16-byte weight load covers the W taps");
    typedef typename AVec<MT>::t amt;
    constexpr int XCP = CC + 4;                      // CL: floats per staged position
    constexpr int XRS = CL ? PWX * XCP : CC * PWX;   // floats per staged row
    constexpr int XCI = CL ? 4 : 4 * PWX;            // LDS step of 4 input channels
    constexpr int XT = CL ? 16 * XCP : 16;           // LDS step of 16 positions
    constexpr int XG = CL ? 1 : PWX;                 // LDS step of one input channel
    constexpr int XP = CL ? XCP : 1;                 // LDS step of one position

    __shared__ __attribute__((aligned(16))) float Wl[2][KW][CC][COB];
    __shared__ __attribute__((aligned(16))) float Xl[2][4][XRS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6; // wave = row of the block
    const int j = lane & 15;
    const int g4 = lane >> 4;

    // channel block fastest, then W segment (C_out/G is a multiple of COB, C_in/G
    // of CC: checked on the host)
    const int cpg = P.Cog / COB; // channel blocks per group
    const int ncb = P.G * cpg;
    const int rsb = (int)blockIdx.x / ncb;
    const int cb = (int)blockIdx.x - rsb * ncb;
    const int grp = cb / cpg, cbg = cb - grp * cpg;
    const int rblk = rsb / P.wseg;
    const int seg = rsb - rblk * P.wseg;
    int cls = 0;
    while (cls + 1 < P.n_class && rblk >= P.cls_block0[cls + 1]) ++cls;
    const int r0 = (rblk - P.cls_block0[cls]) * 4;
    const int nrows = min(4, P.cls_rows[cls] - r0);
    if (nrows <= 0) return;
    const int td = P.cls_td[cls], th = P.cls_th[cls];
    const int nslots = td * th;
    const int nch = P.Cig / CC; // input-channel chunks of the group
    const int nstages = nslots * nch;
    const int pos0 = seg * 16 * NWB + P.iw_lo;     // input position at LDS offset 0
    // staged positions: the segment's P.wnf float4s (<= PWX/4, host) inside the row
    const int lo = max(pos0, 0), hi = min(pos0 + 4 * P.wnf, P.W_in);
    const int nfs = max(hi - lo, 0) >> 2;
    const int fdiv = max(nfs, 1);
    const int xused = (4 * CC * nfs + NT - 1) / NT; // staging slots in use (uniform)

    for (int i = tid; i < 2 * 4 * XRS; i += NT) (&Xl[0][0][0])[i] = 0.0f;

    const RowPos R0 = decode_row(P, cls, r0);
    const RowPos R1 = decode_row(P, cls, r0 + min(1, nrows - 1));
    const RowPos R2 = decode_row(P, cls, r0 + min(2, nrows - 1));
    const RowPos R3 = decode_row(P, cls, r0 + min(3, nrows - 1));

    // Per-thread staging offsets, fixed for the block.
    const int KDHW = P.KD * P.KH * KW;
    const int dhw = P.D_in * P.H_in * P.W_in;
    unsigned wo4[WPER]; // weight byte offset of (ci in chunk, co in block), tap part excluded
    int wlo[WPER];      // its LDS index in a [kw] plane: ci*COB + MT*(co mod 16) + co/16
#pragma unroll
    for (int u = 0; u < WPER; ++u) {
        const int pr = tid + u * NT;
        const int cil = pr / COB, co = pr - cil * COB;
        wo4[u] = 4u * (unsigned)(((grp * P.Cig + cil) * P.Cog + cbg * COB + co) * KDHW);
        wlo[u] = cil * COB + MT * (co & 15) + (co >> 4);
    }
    // Each float4 holds 4 positions of one channel (channels first) or 4
    // channels of one position (channels last); 4*CC*nfs of them per stage.
    int xo[XPER];  // input element offset of the float4 at the row's (qd, qh), chunk 0
    int xlo[XPER]; // its LDS index, -1 past the staged float4s
    int xrw[XPER]; // its row; 31 past the staged float4s or outside the input row (loads zeros)
#pragma unroll
    for (int u = 0; u < XPER; ++u) {
        const int f = tid + u * NT;
        const bool in = f < 4 * CC * nfs;
        const int rr = in ? f / (CC * fdiv) : 3;
        const int rem = in ? f - rr * (CC * nfs) : 0;
        const RowPos R = pick_row(rr, R0, R1, R2, R3);
        if constexpr (CL) {
            const int pi = rem / (CC / 4), q = rem - pi * (CC / 4); // position, channel quad
            const int pos = lo + pi;
            xo[u] = (((R.n * P.D_in + R.qd) * P.H_in + R.qh) * P.W_in + pos) * P.C_in + grp * P.Cig + 4 * q;
            xlo[u] = in ? rr * XRS + (pos - pos0) * XCP + 4 * q : -1;
        } else {
            const int cil = rem / fdiv, c4 = rem - cil * nfs;
            const int pos = lo + 4 * c4;
            xo[u] = (((R.n * P.C_in + grp * P.Cig + cil) * P.D_in + R.qd) * P.H_in + R.qh) * P.W_in + pos;
            xlo[u] = in ? rr * XRS + cil * PWX + pos - pos0 : -1;
        }
        xrw[u] = in ? rr : 31;
    }
    const rsrc_t rw_ = make_rsrc(w, 4 * P.C_in * P.Cog * KDHW);
    const rsrc_t rx = make_rsrc(x, P.x_bytes);

    f4 wpre[WPER];
    f4 xpre[XPER];

    auto fetch = [&](int sidx) {
        const int slot = sidx / nch, ch = sidx - slot * nch;
        const int jd = slot / th, jh = slot - jd * th;
        const int kd = P.cls_kd[cls][jd], kh = P.cls_kh[cls][jh];
        const int cd = P.cls_cd[cls][jd], chh = P.cls_ch[cls][jh];
        const unsigned wst = 4u * (unsigned)(ch * CC * P.Cog * KDHW + (kd * P.KH + kh) * KW);
#pragma unroll
        for (int u = 0; u < WPER; ++u) {
            if constexpr (KW == 4) {
                wpre[u] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rw_, wo4[u], wst, 0));
            } else {
                const f3 v = __builtin_bit_cast(f3, __builtin_amdgcn_raw_buffer_load_b96(rw_, wo4[u], wst, 0));
                wpre[u] = f4{v.x, v.y, v.z, 0.0f};
            }
        }
        // rows whose input row (qd - cd, qh - ch) lies inside the input: one bit each
        unsigned bad = 0xffffffffu;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const RowPos &R = q == 0 ? R0 : q == 1 ? R1 : q == 2 ? R2 : R3;
            const int id = R.qd - cd, ih = R.qh - chh;
            if (q < nrows && id >= 0 && id < P.D_in && ih >= 0 && ih < P.H_in) bad &= ~(1u << q);
        }
        const int xst = CL ? ch * CC - (cd * P.H_in + chh) * P.W_in * P.C_in
                           : ch * CC * dhw - (cd * P.H_in + chh) * P.W_in;
#pragma unroll
        for (int u = 0; u < XPER; ++u) {
            if (u < 2 || u < xused) {
                const unsigned off = ((bad >> xrw[u]) << 31) | (4u * (unsigned)(xo[u] + xst));
                xpre[u] = buf_load4(rx, off);
            }
        }
    };
    auto stash = [&](int b) {
#pragma unroll
        for (int u = 0; u < WPER; ++u) {
            (&Wl[b][0][0][0])[wlo[u]] = wpre[u].x;
            (&Wl[b][1][0][0])[wlo[u]] = wpre[u].y;
            (&Wl[b][2][0][0])[wlo[u]] = wpre[u].z;
            if constexpr (KW == 4) (&Wl[b][KW - 1][0][0])[wlo[u]] = wpre[u].w;
        }
#pragma unroll
        for (int u = 0; u < XPER; ++u)
            if ((u < 2 || u < xused) && xlo[u] >= 0) *reinterpret_cast<f4 *>(&Xl[b][0][0] + xlo[u]) = xpre[u];
    };

    f4 acc[MT][NPH][NWB];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
            for (int t = 0; t < NWB; ++t) acc[m][ph][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    __syncthreads(); // halo zeros in place
    if (nstages > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();
    const bool active = wv < nrows;
    for (int sidx = 0; sidx < nstages; ++sidx) {
        const int b = sidx & 1;
        const bool has_next = sidx + 1 < nstages;
        if (has_next) fetch(sidx + 1);
        if (active && Ph::count() > 0) {
            typedef const __attribute__((address_space(3))) float *lds_ptr;
            typedef const __attribute__((address_space(3))) amt *lds_aptr;
            const lds_ptr abase = (lds_ptr)(&Wl[b][0][g4][MT * j]);
            // one base per (W phase, tap shift), relations hidden (see k_igemm3d)
            constexpr int CM = Ph::cmax() + 1;
            lds_ptr bb[SW][CM];
#pragma unroll
            for (int rw = 0; rw < SW; ++rw)
#pragma unroll
                for (int c = 0; c < CM; ++c) {
                    bb[rw][c] = (lds_ptr)(&Xl[b][wv][0] + g4 * XG + (P.qw0[rw] + j - c - P.iw_lo) * XP);
                    asm volatile("" : "+v"(bb[rw][c]));
                }
#pragma unroll
            for (int cig = 0; cig < CC / 4; ++cig) {
#pragma unroll
                for (int kw = 0; kw < KW; ++kw) {
                    const int rw = Ph::r_of(kw);
                    const int ph = Ph::slot(rw);
                    const int c = Ph::c_of(kw);
                    const amt a = *(lds_aptr)(abase + (kw * CC + 4 * cig) * COB);
#pragma unroll
                    for (int t = 0; t < NWB; ++t) {
                        const float bv = bb[rw][c][cig * XCI + t * XT];
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            acc[m][ph][t] =
                                __builtin_amdgcn_mfma_f32_16x16x4f32(aget(a, m), bv, acc[m][ph][t], 0, 0, 0);
                    }
                }
            }
        }
        if (has_next) stash(b ^ 1);
        __syncthreads();
    }

    if (!active) return;
    const RowPos R = pick_row(__builtin_amdgcn_readfirstlane(wv), R0, R1, R2, R3);
    if constexpr (CL) {
        // lane: 4 consecutive channels of a position, one float4 per (m, W-block,
        // output); a W-block wholly inside the row (a uniform test) stores without
        // per-lane guards
        const int64_t pbase = (((int64_t)R.n * P.D_out + R.od) * P.H_out + R.oh) * P.W_out;
        float bco[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bco[m][e] = bias ? bias[grp * P.Cog + cbg * COB + 16 * m + 4 * g4 + e] : 0.0f;
        auto put = [&](int t, int m, int rr, bool guard) {
            const int ow0 = SW * (16 * (NWB * seg + t) + j);
            if (guard && ow0 + rr >= P.W_out) return;
            f4 v = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int rw = 0; rw < SW; ++rw)
                if constexpr (Ph::count() > 0)
                    if (Ph::nonempty(rw))
                        if (P.sigma[rw] == rr) v = acc[m][Ph::slot(rw)][t];
            const int64_t o = (pbase + ow0 + rr) * P.C_out + grp * P.Cog + cbg * COB + 16 * m + 4 * g4;
            f4 a4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (epi_add(EPI)) a4 = load4u(add + o);
            f4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = epilogue<EPI>(v[e], bco[m][e], a4[e]);
            __builtin_memcpy(y + o, &r, 16); // 4-byte alignment suffices
        };
#pragma unroll
        for (int t = 0; t < NWB; ++t) {
            if (SW * 16 * (NWB * seg + t + 1) <= P.W_out) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr) put(t, m, rr, false);
            } else {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int rr = 0; rr < SW; ++rr) put(t, m, rr, true);
            }
        }
        return;
    }
    const int64_t dhw_out = (int64_t)P.D_out * P.H_out * P.W_out;
    const int64_t row_base =
        (int64_t)R.n * P.C_out * dhw_out + ((int64_t)R.od * P.H_out + R.oh) * P.W_out;
    if constexpr (SW == 2 && Ph::count() == 2) {
        // a lane's two outputs of a channel are adjacent: one 8-byte store; W
        // phase 0 lands on the odd outputs when sigma(0) = 1.  A W-block wholly
        // inside the row (a uniform test) stores without per-lane guards.
        const bool swp = P.sigma[0] != 0;
        float bco[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bco[m][e] = bias ? bias[grp * P.Cog + cbg * COB + 16 * m + 4 * g4 + e] : 0.0f;
        auto put = [&](int t, int m, int e, bool guard) {
            const int co = grp * P.Cog + cbg * COB + 16 * m + 4 * g4 + e;
            const int ow0 = 2 * (16 * (NWB * seg + t) + j);
            const float a0 = acc[m][Ph::slot(0)][t][e], a1 = acc[m][Ph::slot(1)][t][e];
            const float v0 = swp ? a1 : a0, v1 = swp ? a0 : a1;
            const int64_t o = row_base + (int64_t)co * dhw_out + ow0;
            if (!guard || ow0 + 1 < P.W_out) {
                float ad[2] = {0.0f, 0.0f};
                if constexpr (epi_add(EPI)) __builtin_memcpy(ad, add + o, 8);
                const float r[2] = {epilogue<EPI>(v0, bco[m][e], ad[0]), epilogue<EPI>(v1, bco[m][e], ad[1])};
                __builtin_memcpy(y + o, r, 8); // 4-byte alignment suffices
            } else if (ow0 < P.W_out) {
                const float ad = epi_add(EPI) ? add[o] : 0.0f;
                y[o] = epilogue<EPI>(v0, bco[m][e], ad);
            }
        };
#pragma unroll
        for (int t = 0; t < NWB; ++t) {
            if (32 * (NWB * seg + t + 1) <= P.W_out) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) put(t, m, e, false);
            } else {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) put(t, m, e, true);
            }
        }
        return;
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int co = grp * P.Cog + cbg * COB + 16 * m + 4 * g4 + e;
            const float bco = bias ? bias[co] : 0.0f;
#pragma unroll
            for (int t = 0; t < NWB; ++t) {
                const int ow0 = SW * (16 * (NWB * seg + t) + j);
                float v[SW];
#pragma unroll
                for (int rr = 0; rr < SW; ++rr) v[rr] = 0.0f;
#pragma unroll
                for (int rw = 0; rw < SW; ++rw)
                    if constexpr (Ph::count() > 0)
                        if (Ph::nonempty(rw)) {
                            const float a = acc[m][Ph::slot(rw)][t][e];
#pragma unroll
                            for (int rr = 0; rr < SW; ++rr)
                                if (P.sigma[rw] == rr) v[rr] = a;
                        }
                const int64_t o = row_base + (int64_t)co * dhw_out + ow0;
#pragma unroll
                for (int rr = 0; rr < SW; ++rr) {
                    if (ow0 + rr < P.W_out) {
                        const float a1 = epi_add(EPI) ? add[o + rr] : 0.0f;
                        y[o + rr] = epilogue<EPI>(v[rr], bco, a1);
                    }
                }
            }
        }
}

// ---------------------------------------------------------------- host side
struct Variant {
    int cig, cog, KW, SW, DW, TDM, THM, NWBM, PWM, W4M;
};
constexpr int kPW = 48; // LDS pitch: 16 mod 32 spreads the 4 ci rows of a B read over the banks
constexpr Variant kVariants[] = {
    {32, 64, 3, 2, 1, 2, 2, 1, kPW, 4}, // 32 -> 64 channels, kernel 3, stride 2 (the fused layer)
    {32, 64, 3, 2, 1, 2, 2, 2, kPW, 8}, // same, input rows up to 32 wide
    {16, 32, 4, 2, 1, 2, 2, 2, kPW, 8}, // 16 -> 32 channels, kernel 4, stride 2
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

int ceil_div(int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); }

struct Layout {
    int iw_lo, need, nwb;
    int qw0[kMaxSW], sigma[kMaxSW];
    int cmax;
};

bool w_layout(const convt_plan &P, const Variant &v, Layout &L, bool last = false) {
    const AxisPlan &A = P.ax[2];
    if (A.K != v.KW || A.s != v.SW || A.d != v.DW) return false;
    L.cmax = 0;
    for (int k = 0; k < v.KW; ++k) L.cmax = std::max(L.cmax, (k * v.DW) / v.SW);
    int qmax = 0;
    for (int r = 0; r < v.SW; ++r) {
        L.qw0[r] = std::max(0, ceil_div(A.p - r, v.SW));
        L.sigma[r] = L.qw0[r] * v.SW + r - A.p;
        qmax = std::max(qmax, L.qw0[r]);
    }
    L.nwb = (A.L_out + 16 * v.SW - 1) / (16 * v.SW);
    L.iw_lo = -((L.cmax + 3) / 4) * 4;
    const int iw_hi = std::max(qmax + 16 * L.nwb, A.L_in); // exclusive
    L.need = iw_hi - L.iw_lo;
    // the W-block count is a compile-time constant; channels last stages
    // 16*NWBM + 8 positions per tap row
    return L.nwb == v.NWBM && L.need <= (last ? 16 * v.NWBM + 8 : v.PWM);
}

int find_variant(const convt_plan &P, Layout *Lout = nullptr) {
    // 2D plans run as depth-1 3D problems (their leading axis has one position
    // and one tap)
    if (P.ndim < 2 || P.G != 1) return -1;
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    if (AW.L_in % 4 != 0) return -1;
    // per-sample byte offsets of x, y and add_input stay below 2^31 (buffer addressing)
    if ((int64_t)P.C_in * AD.L_in * AH.L_in * AW.L_in * 4 >= INT32_MAX ||
        (int64_t)P.C_out * AD.L_out * AH.L_out * AW.L_out * 4 >= INT32_MAX)
        return -1;
    const int W4 = AW.L_in / 4;
    if (AD.s * AH.s > kMaxClasses) return -1;
    // taps per class on D and H
    int tdm = 0, thm = 0;
    for (int r = 0; r < AD.s; ++r) tdm = std::max(tdm, AD.tap_start[r + 1] - AD.tap_start[r]);
    for (int r = 0; r < AH.s; ++r) thm = std::max(thm, AH.tap_start[r + 1] - AH.tap_start[r]);
    for (int i = 0; i < kNumVariants; ++i) {
        const Variant &v = kVariants[i];
        if (P.Cig != v.cig || P.Cog != v.cog || tdm > v.TDM || thm > v.THM || W4 > v.W4M) continue;
        Layout L;
        if (!w_layout(P, v, L, P.layout == CONVT_LAYOUT_CHANNELS_LAST)) continue;
        if (Lout) *Lout = L;
        return i;
    }
    return -1;
}

int num_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    return cus;
}

// Fills P from the plan and the W layout: sizes, W phases and the class table
// (classes ordered heaviest first).  Returns the total number of output rows.
int64_t fill_params(const convt_plan &Pl, const Layout &L, int SW, Igemm3dParams &P) {
    const AxisPlan &AD = Pl.ax[0], &AH = Pl.ax[1], &AW = Pl.ax[2];
    memset(&P, 0, sizeof(P));
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.D_in = AD.L_in;
    P.H_in = AH.L_in;
    P.W_in = AW.L_in;
    P.D_out = AD.L_out;
    P.H_out = AH.L_out;
    P.W_out = AW.L_out;
    P.KD = AD.K;
    P.KH = AH.K;
    P.s_d = AD.s;
    P.s_h = AH.s;
    P.iw_lo = L.iw_lo;
    P.nwb = L.nwb;
    for (int r = 0; r < SW; ++r) {
        P.qw0[r] = L.qw0[r];
        P.sigma[r] = L.sigma[r];
    }
    struct Cls {
        int rd, rh, taps;
    } cl[kMaxClasses];
    int nc = 0;
    for (int rd = 0; rd < AD.s; ++rd)
        for (int rh = 0; rh < AH.s; ++rh) {
            const int td = AD.tap_start[rd + 1] - AD.tap_start[rd];
            const int th = AH.tap_start[rh + 1] - AH.tap_start[rh];
            cl[nc++] = {rd, rh, td * th};
        }
    for (int a = 0; a < nc; ++a)
        for (int b = a + 1; b < nc; ++b)
            if (cl[b].taps > cl[a].taps) std::swap(cl[a], cl[b]);
    int64_t total_rows = 0;
    int kept = 0;
    for (int i = 0; i < nc; ++i) {
        const int rd = cl[i].rd, rh = cl[i].rh;
        const int qd0 = std::max(0, ceil_div(AD.p - rd, AD.s));
        const int od0 = qd0 * AD.s + rd - AD.p;
        const int nqd = od0 < AD.L_out ? (AD.L_out - 1 - od0) / AD.s + 1 : 0;
        const int qh0 = std::max(0, ceil_div(AH.p - rh, AH.s));
        const int oh0 = qh0 * AH.s + rh - AH.p;
        const int nqh = oh0 < AH.L_out ? (AH.L_out - 1 - oh0) / AH.s + 1 : 0;
        if (nqd == 0 || nqh == 0) continue;
        const int c = kept++;
        P.cls_td[c] = AD.tap_start[rd + 1] - AD.tap_start[rd];
        P.cls_th[c] = AH.tap_start[rh + 1] - AH.tap_start[rh];
        for (int t = 0; t < P.cls_td[c]; ++t) {
            P.cls_kd[c][t] = AD.tap_k[AD.tap_start[rd] + t];
            P.cls_cd[c][t] = AD.tap_c[AD.tap_start[rd] + t];
        }
        for (int t = 0; t < P.cls_th[c]; ++t) {
            P.cls_kh[c][t] = AH.tap_k[AH.tap_start[rh] + t];
            P.cls_ch[c][t] = AH.tap_c[AH.tap_start[rh] + t];
        }
        P.cls_qd0[c] = qd0;
        P.cls_od0[c] = od0;
        P.cls_nqd[c] = nqd;
        P.cls_qh0[c] = qh0;
        P.cls_oh0[c] = oh0;
        P.cls_nqh[c] = nqh;
        P.cls_rows[c] = (int)(Pl.N * nqd * nqh);
        P.cls_rstep[c] = 1;
        total_rows += P.cls_rows[c];
    }
    P.n_class = kept;
    return total_rows;
}

// Blocks of rpb rows per class; returns the grid size.  With xcd_order the
// block count of each class is a multiple of the XCD count (blocks whose chunk
// lies past the class's rows exit at once).
int assign_blocks(Igemm3dParams &P, int rpb, bool xcd_order = false) {
    P.rows_per_block = rpb;
    P.xcd_order = xcd_order ? 1 : 0;
    int blocks = 0;
    for (int c = 0; c < P.n_class; ++c) {
        P.cls_block0[c] = blocks;
        P.cls_chunks[c] = (P.cls_rows[c] + rpb - 1) / rpb;
        blocks += xcd_order ? (P.cls_chunks[c] + kXcds - 1) / kXcds * kXcds : P.cls_chunks[c];
    }
    P.cls_block0[P.n_class] = blocks;
    return blocks;
}

template <int CIG, int COG, int KW, int SW, int DW, int TDM, int THM, int NWBM, int PWM, int W4M>
int launch_variant(const convt_plan &Pl, const Layout &L, const float *x, const float *w,
                   const float *bias, const float *add, int act, float *y, hipStream_t st) {
    Igemm3dParams P;
    const int64_t total_rows = fill_params(Pl, L, SW, P);
    // rows per block: enough blocks to fill the CUs several times over
    const int64_t target_blocks = (int64_t)num_cus() * CONVT_IG_BLOCKS_PER_CU;
    int rpb = (int)std::max<int64_t>(1, std::min<int64_t>(CONVT_IG_MAX_ROWS, total_rows / target_blocks));
    const bool last = Pl.layout == CONVT_LAYOUT_CHANNELS_LAST;
    // Multi-row steps (the kernel compiles them for channels first, 4 tap
    // slots and one W-block): a class of 1 or 2 taps whose H runs split into
    // whole steps; blocks then start on a step (rows per block a multiple of 4).
    if (CONVT_IG_MULTIROW && !last && TDM * THM == 4 && NWBM == 1) {
        bool any = false;
        for (int c = 0; c < P.n_class; ++c) {
            const int nt = P.cls_td[c] * P.cls_th[c];
            if ((nt == 1 || nt == 2) && P.cls_nqh[c] % (4 / nt) == 0) {
                P.cls_rstep[c] = 4 / nt;
                any = true;
            }
        }
        if (any) rpb = (rpb + 3) / 4 * 4;
    }
    const int blocks = assign_blocks(P, rpb, CONVT_IG_XCD_ORDER != 0);
    if (blocks == 0) return 0;
    constexpr int NT = COG * 4;
    constexpr int PER = (TDM * THM * CIG * W4M + NT - 1) / NT; // W_in <= 4*W4M is checked
    const int need_f = TDM * THM * CIG * (Pl.ax[2].L_in / 4);
    if (need_f > PER * NT) return (int)hipErrorInvalidValue;
    // every lane of every W-block inside the row
    const bool fullw = Pl.ax[2].L_out == SW * 16 * NWBM;
    auto launch = [&](auto epi, auto full, auto swap) {
        if (last) { // channels last: the staged epilogue guards the row end itself
            if constexpr (!decltype(full)::value)
                hipLaunchKernelGGL((k_igemm3d<CIG, COG, KW, SW, DW, TDM, THM, NWBM, PWM, PER, decltype(epi)::value,
                                              false, decltype(swap)::value, true>),
                                   dim3(blocks), dim3(NT), 0, st, P, x, w, bias, add, y);
            return;
        }
        hipLaunchKernelGGL((k_igemm3d<CIG, COG, KW, SW, DW, TDM, THM, NWBM, PWM, PER, decltype(epi)::value,
                                      decltype(full)::value, decltype(swap)::value, false>),
                           dim3(blocks), dim3(NT), 0, st, P, x, w, bias, add, y);
    };
    auto with_swap = [&](auto fused, auto full) {
        if constexpr (SW == 2) {
            if (P.sigma[0] != 0) { // W phase 0 lands on the odd outputs
                launch(fused, full, std::true_type{});
                return;
            }
        }
        launch(fused, full, std::false_type{});
    };
    auto with_full = [&](auto fused) {
        if (fullw && !last) with_swap(fused, std::true_type{});
        else with_swap(fused, std::false_type{});
    };
    with_epi(add != nullptr, act, with_full);
    return (int)hipGetLastError();
}

// Streamed-weight shapes (either layout): kernel 3 or 4 along W with stride 2, or
// kernel 3 with stride 1, on rows of any length that is a multiple of 4 (one or
// two W-blocks per segment), output
// channels of a group in blocks of 64, 32 or 16 (the largest that divides
// C_out/G; 16 only with C_in/G >= 64); C_in/G is any multiple of the chunk.
struct WideVariant {
    int KW, SW, NWB, MT;
};
constexpr WideVariant kWide[] = {
    {4, 2, 2, 4}, {4, 2, 1, 4}, {3, 2, 2, 4}, {3, 2, 1, 4}, // kernel 4 (the channel-heavy layer) or 3
    {4, 2, 2, 2}, {4, 2, 1, 2}, {3, 2, 2, 2}, {3, 2, 1, 2}, // 32-channel blocks
    {3, 1, 2, 4}, {3, 1, 1, 4}, {3, 1, 2, 2}, {3, 1, 1, 2}, // kernel 3, stride 1
    {4, 2, 2, 1}, {4, 2, 1, 1}, {3, 2, 2, 1}, {3, 2, 1, 1}, // 16-channel blocks
    {3, 1, 2, 1}, {3, 1, 1, 1},
};
constexpr int kNumWide = (int)(sizeof(kWide) / sizeof(kWide[0]));
constexpr int kWideCC = 16; // input channels per stage
constexpr int kWidePWX = 48; // LDS pitch of a staged input row

struct WideLayout {
    Layout L;
    int nseg; // W segments per row
    int nf;   // float4s staged per input row and segment
};

// W layout of the wide variant: two W-blocks per segment when the row has more
// than 16*S_W outputs, enough segments to cover the row, and the staged input
// positions of a segment (its 16*NWB positions plus the halo of the taps).
bool wide_layout(const convt_plan &P, int KW, int SW, int NWB, WideLayout &WL) {
    constexpr int DW = 1;
    const AxisPlan &A = P.ax[2];
    if (A.K != KW || A.s != SW || A.d != DW) return false;
    Layout &L = WL.L;
    L.cmax = 0;
    for (int k = 0; k < KW; ++k) L.cmax = std::max(L.cmax, (k * DW) / SW);
    int qmax = 0;
    for (int r = 0; r < SW; ++r) {
        L.qw0[r] = std::max(0, ceil_div(A.p - r, SW));
        L.sigma[r] = L.qw0[r] * SW + r - A.p;
        qmax = std::max(qmax, L.qw0[r]);
    }
    L.nwb = A.L_out > 16 * SW ? 2 : 1;
    if (L.nwb != NWB) return false;
    L.iw_lo = -((L.cmax + 3) / 4) * 4;
    L.need = qmax + 16 * NWB - L.iw_lo; // LDS positions the B reads of a segment reach
    WL.nseg = (A.L_out + 16 * SW * NWB - 1) / (16 * SW * NWB);
    WL.nf = (L.need + 3) / 4;
    return 4 * WL.nf <= kWidePWX;
}

int find_wide(const convt_plan &P, WideLayout *out) {
    if (P.ndim < 2) return -1;
    if (P.Cig % kWideCC != 0 || P.Cog % 16 != 0) return -1;
    const int mt = P.Cog % 64 == 0 ? 4 : P.Cog % 32 == 0 ? 2 : 1;
    // 16-channel blocks pay the staging of 16 input channels per 8 MFMAs of a
    // W-block: ahead of the generic kernels only with 64 or more input channels
    if (mt == 1 && P.Cig < 64) return -1;
    const AxisPlan &AD = P.ax[0], &AH = P.ax[1], &AW = P.ax[2];
    // one buffer resource spans x, one the weights (31-bit byte offsets); per-sample y
    // as in the VGPR variant
    if (4 * P.N * P.C_in * P.in_sp >= INT32_MAX || 4 * P.C_out * P.out_sp >= INT32_MAX ||
        4 * P.C_in * P.Cog * AD.K * AH.K * AW.K >= INT32_MAX)
        return -1;
    if (AW.L_in % 4 != 0) return -1; // staged float4s lie wholly inside or outside a row
    if (AD.s * AH.s > kMaxClasses) return -1;
    int tdm = 0, thm = 0;
    for (int r = 0; r < AD.s; ++r) tdm = std::max(tdm, AD.tap_start[r + 1] - AD.tap_start[r]);
    for (int r = 0; r < AH.s; ++r) thm = std::max(thm, AH.tap_start[r + 1] - AH.tap_start[r]);
    if (tdm > kTapMax || thm > kTapMax) return -1;
    for (int i = 0; i < kNumWide; ++i) {
        const WideVariant &v = kWide[i];
        if (v.MT != mt) continue;
        WideLayout WL;
        if (!wide_layout(P, v.KW, v.SW, v.NWB, WL)) continue;
        if (out) *out = WL;
        return i;
    }
    return -1;
}

template <int KW, int SW, int NWB, int MT>
int launch_wide(const convt_plan &Pl, const WideLayout &WL, const float *x, const float *w,
                const float *bias, const float *add, int act, float *y, hipStream_t st) {
    Igemm3dParams P;
    fill_params(Pl, WL.L, SW, P);
    P.x_bytes = (int)(4 * Pl.N * Pl.C_in * Pl.in_sp);
    P.wseg = WL.nseg;
    P.wnf = WL.nf;
    P.G = (int)Pl.G;
    P.Cig = (int)Pl.Cig;
    P.Cog = (int)Pl.Cog;
    const int64_t blocks = (int64_t)assign_blocks(P, 4) * WL.nseg * (Pl.C_out / (16 * MT));
    if (blocks == 0) return 0;
    if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    const bool last = Pl.layout == CONVT_LAYOUT_CHANNELS_LAST;
    with_epi(add != nullptr, act, [&](auto E) {
        if (last)
            hipLaunchKernelGGL((k_igemm3d_wide<KW, SW, 1, NWB, MT, kWideCC, kWidePWX, decltype(E)::value, true>),
                               dim3((unsigned)blocks), dim3(256), 0, st, P, x, w, bias, add, y);
        else
            hipLaunchKernelGGL((k_igemm3d_wide<KW, SW, 1, NWB, MT, kWideCC, kWidePWX, decltype(E)::value, false>),
                               dim3((unsigned)blocks), dim3(256), 0, st, P, x, w, bias, add, y);
    });
    return (int)hipGetLastError();
}

} // namespace

bool igemm3d_supports(const convt_plan &P) {
    if (P.ndim < 2) return false;
    Layout L;
    if (find_variant(P, &L) < 0 && find_wide(P, nullptr) < 0) return false;
    return P.N * P.ax[0].L_out * P.ax[1].L_out < (int64_t(1) << 31);
}

const char *igemm3d_kernel_name(const convt_plan &P) {
    Layout L;
    if (find_variant(P, &L) >= 0) return "k_igemm3d";
    return find_wide(P, nullptr) >= 0 ? "k_igemm3d_wide" : "none";
}

int launch_igemm3d(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                   const float *add, int act, float *y, void *stream) {
    Layout L;
    const int v = find_variant(Pl, &L); // weights in VGPRs when they fit, else streamed
    hipStream_t st = (hipStream_t)stream;
    switch (v) {
    case 0: return launch_variant<32, 64, 3, 2, 1, 2, 2, 1, kPW, 4>(Pl, L, x, w, bias, add, act, y, st);
    case 1: return launch_variant<32, 64, 3, 2, 1, 2, 2, 2, kPW, 8>(Pl, L, x, w, bias, add, act, y, st);
    case 2: return launch_variant<16, 32, 4, 2, 1, 2, 2, 2, kPW, 8>(Pl, L, x, w, bias, add, act, y, st);
    default: break;
    }
    WideLayout WL;
    switch (find_wide(Pl, &WL)) {
    case 0: return launch_wide<4, 2, 2, 4>(Pl, WL, x, w, bias, add, act, y, st);
    case 1: return launch_wide<4, 2, 1, 4>(Pl, WL, x, w, bias, add, act, y, st);
    case 2: return launch_wide<3, 2, 2, 4>(Pl, WL, x, w, bias, add, act, y, st);
    case 3: return launch_wide<3, 2, 1, 4>(Pl, WL, x, w, bias, add, act, y, st);
    case 4: return launch_wide<4, 2, 2, 2>(Pl, WL, x, w, bias, add, act, y, st);
    case 5: return launch_wide<4, 2, 1, 2>(Pl, WL, x, w, bias, add, act, y, st);
    case 6: return launch_wide<3, 2, 2, 2>(Pl, WL, x, w, bias, add, act, y, st);
    case 7: return launch_wide<3, 2, 1, 2>(Pl, WL, x, w, bias, add, act, y, st);
    case 8: return launch_wide<3, 1, 2, 4>(Pl, WL, x, w, bias, add, act, y, st);
    case 9: return launch_wide<3, 1, 1, 4>(Pl, WL, x, w, bias, add, act, y, st);
    case 10: return launch_wide<3, 1, 2, 2>(Pl, WL, x, w, bias, add, act, y, st);
    case 11: return launch_wide<3, 1, 1, 2>(Pl, WL, x, w, bias, add, act, y, st);
    case 12: return launch_wide<4, 2, 2, 1>(Pl, WL, x, w, bias, add, act, y, st);
    case 13: return launch_wide<4, 2, 1, 1>(Pl, WL, x, w, bias, add, act, y, st);
    case 14: return launch_wide<3, 2, 2, 1>(Pl, WL, x, w, bias, add, act, y, st);
    case 15: return launch_wide<3, 2, 1, 1>(Pl, WL, x, w, bias, add, act, y, st);
    case 16: return launch_wide<3, 1, 2, 1>(Pl, WL, x, w, bias, add, act, y, st);
    case 17: return launch_wide<3, 1, 1, 1>(Pl, WL, x, w, bias, add, act, y, st);
    default: return (int)hipErrorInvalidValue;
    }
}

} // namespace convt
