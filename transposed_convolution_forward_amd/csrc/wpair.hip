// Groups of 8 output channels with stride 2 and dilation 1 along W: the two W
// phases of each pair of adjacent outputs share the 16 rows of one fp32 MFMA
// tile (v_mfma_f32_16x16x4_f32), so that a store instruction writes whole
// lines and the contraction needs no row sharing along H.
//
// Method (the phase decomposition of convt_internal.h).  Along W, output
// o = 2m + delta (delta = 0, 1) has residue r(delta) = (delta + p) mod 2 and
// position q = m + e(delta), e(delta) = (delta + p - r(delta)) / 2; its taps k
// (k = r(delta) mod 2) read input q - c_k = m - (c_k - e(delta)).  So with the
// shift sl = c_k - e(delta) the two phases of pair m read the same input
// column m - sl, and one B operand (4 input channels x 16 pairs m) serves the
// tile's rows i = 8*delta + co: A holds, per shift sl, tap k of phase delta
// (zero where a phase has no tap at that shift).  Along D and H a class fixes
// the taps ("Kimi-K2.6 l1_p72" transcript, ConvTranspose3d with groups 4 and
// kernel 3x5x7: the parity-class blocking and the per-group channel mapping).
//
// Mapping.  A workgroup of four waves holds one (class, group) and walks a run
// of steps; a step is four consecutive output rows along H (wave w: row w) of
// one (n, qd).  The class's weights for the group are copied once through LDS
// into VGPRs (every wave holds the same A operands); runs are sized so that
// every workgroup has the same number of MFMAs and the grid is one round of
// resident workgroups.  The input rows of a step (D taps x (H taps + 3)
// rows x 8 channels x W_in) are fetched into registers during the previous
// step's contraction and staged in LDS (double buffer, zero columns at both
// ends).  D[i][j] sits at lane j + 16(i/4), register i%4: for register e the
// lanes of g4 = 0 and 2 hold channel e at outputs 2m and 2m+1 of 16 pairs, 32
// consecutive floats.  Atomic-free: every output is stored once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "convt_internal.h"
#include "epilogue.hpp"

namespace convt {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000; // raw (untyped) buffer access
constexpr unsigned kOutOfRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ f4 buf_load4(rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ float buf_load1(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store1(float v, rsrc_t r, unsigned voff, unsigned soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, voff, soff, 0);
}

// Tuning knob: rounds of resident workgroups (three per CU) the grid aims
// for when sizing the steps per block.
#ifndef CONVT_WPAIR_ROUNDS
#define CONVT_WPAIR_ROUNDS 1
#endif

constexpr int kCg = 8;       // input and output channels per group
constexpr int kTDM = 2;      // D taps per class
constexpr int kTHM = 5;      // H taps per class (at shifts 0 .. th-1)
constexpr int kNS = 4;       // W shifts
constexpr int kRows = kTHM + 3; // staged H rows per D tap
constexpr int kNT = 2;       // tiles of 16 pairs per output row
constexpr int kW4M = 8;      // float4 per staged input row (W_in <= 32)
constexpr int kPW = 48;      // LDS pitch per channel row (48 mod 64: the 4 rows of a B read on distinct banks)
constexpr int kMaxCls = 16;
constexpr int kBlockT = 256;
constexpr int kPer = (kTDM * kRows * kCg * kW4M + kBlockT - 1) / kBlockT; // staged float4 per thread
constexpr int kMaxKvol = 2 * kTDM * kRows * kCg * kPW / (kCg * kCg); // KD*KH*KW whose group weights fit the LDS buffers
constexpr int kWPer = kCg * kCg * kMaxKvol / 4 / kBlockT;            // weight float4 per thread at most

struct WpParams {
    int C_in, C_out, G;
    int D_in, H_in, W_in, D_out, H_out, W_out;
    int KD, KH, KW, s_d, s_h;
    int nm;        // pairs per output row
    int smin;      // shift of slot 0
    int col0;      // LDS column of input position 0 (a multiple of 4)
    int wtap[2][kNS]; // kw of (delta, slot), -1 none
    int n_class;
    int cls_spb[kMaxCls];   // steps per block (fewer for classes with more D taps)
    int cls_bpg[kMaxCls];   // blocks per group (a block's run stays in one group)
    int cls_block0[kMaxCls + 1];
    int cls_steps[kMaxCls]; // N * nqd * ceil(nqh / 4) steps per group, ordered (n, qd, qh block)
    int cls_td[kMaxCls], cls_th[kMaxCls];
    int cls_kd[kMaxCls][kTDM], cls_cd[kMaxCls][kTDM];
    int cls_kh[kMaxCls][kTHM];
    int cls_qd0[kMaxCls], cls_nqd[kMaxCls], cls_od0[kMaxCls];
    int cls_qh0[kMaxCls], cls_nqh[kMaxCls], cls_oh0[kMaxCls];
};

struct Step {
    int g, n, iqd, iqh0; // iqh0: first of the step's four rows within the class
};

__device__ __forceinline__ Step step_at(const WpParams &P, int cls, int g, int k) {
    const int nqhb = (P.cls_nqh[cls] + 3) / 4, nqd = P.cls_nqd[cls];
    Step S;
    S.iqh0 = 4 * (k % nqhb);
    k /= nqhb;
    S.iqd = k % nqd;
    S.n = k / nqd;
    S.g = g;
    // uniform across the wave (the buffer resources built from them must sit
    // in scalar registers)
    S.n = __builtin_amdgcn_readfirstlane(S.n);
    S.iqd = __builtin_amdgcn_readfirstlane(S.iqd);
    S.iqh0 = __builtin_amdgcn_readfirstlane(S.iqh0);
    return S;
}

template <int TH, int EPI>
__global__ __launch_bounds__(kBlockT) __attribute__((amdgpu_waves_per_eu(3))) void k_generic_wpair(const WpParams P, int N, const float *__restrict__ x,
                                                           const float *__restrict__ w,
                                                           const float *__restrict__ bias, const float *add,
                                                           float *y) {
    constexpr bool FUSED = epi_add(EPI);
    constexpr int SLOT = kCg * kPW;            // floats per staged row (8 channels)
    constexpr int BUF = kTDM * kRows * SLOT;   // floats per buffer
    __shared__ __attribute__((aligned(16))) float lds[2][BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6); // this wave's row of the step
    const int j = lane & 15, g4 = lane >> 4;

    int cls = 0;
    while (cls + 1 < P.n_class && (int)blockIdx.x >= P.cls_block0[cls + 1]) ++cls;
    const int bl = (int)blockIdx.x - P.cls_block0[cls];
    const int grp = __builtin_amdgcn_readfirstlane(bl / P.cls_bpg[cls]);
    const int k_begin = (bl % P.cls_bpg[cls]) * P.cls_spb[cls];
    const int k_end = min(k_begin + P.cls_spb[cls], P.cls_steps[cls]);
    if (k_begin >= k_end) return;
    static_assert(TH >= 1 && TH <= kTHM, "H taps");
    const int td = P.cls_td[cls]; // every class of the launch has TH H taps
    constexpr int th = TH;

    // Staged float4 f = tid + u*256: D tap dt, row r, channel ci, float4 c4
    // (fastest); its byte offset in the group's channels of the sample is
    // rowpart + xo[u], and it is valid when bit dt*kRows + r of the step's
    // mask is clear.
    const int W4 = P.W_in >> 2;
    const int nf = kTDM * kRows * kCg * W4;
    const int dhw = P.D_in * P.H_in * P.W_in;
    int xo[kPer], lo[kPer], sb[kPer];
    // (parameter fields are read with uniform indices only: a per-lane index
    // into the kernel arguments would copy them to scratch memory)
    const int cd0 = P.cls_cd[cls][0], cd1 = P.cls_cd[cls][1];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int f = tid + u * kBlockT;
        const int c4 = f % W4, t1 = f / W4;
        const int ci = t1 % kCg, t2 = t1 / kCg;
        const int r = t2 % kRows, dt = t2 / kRows;
        const int cd = dt == 0 ? cd0 : dt == 1 ? cd1 : 0;
        xo[u] = 4 * (ci * dhw + (-cd * P.H_in + r) * P.W_in + 4 * c4);
        lo[u] = f < nf ? (dt * kRows + r) * SLOT + ci * kPW + P.col0 + 4 * c4 : -1;
        sb[u] = f < nf ? dt * kRows + r : 31;
    }
    const int xbytes = 4 * kCg * dhw;

    // rows of step S: D position qd, first H position qh0 - (th - 1)
    auto fetch = [&](f4 (&rv)[kPer], const Step &S) __attribute__((always_inline)) {
        const int qd = P.cls_qd0[cls] + S.iqd;
        const int qh = P.cls_qh0[cls] + S.iqh0 - (th - 1);
        unsigned bad = 0xffffffffu;
#pragma unroll
        for (int dt = 0; dt < kTDM; ++dt) {
            const int id = qd - P.cls_cd[cls][dt];
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const int ih = qh + r;
                const bool ok = (dt < td) & (r < th + 3) & ((unsigned)id < (unsigned)P.D_in) &
                                ((unsigned)ih < (unsigned)P.H_in);
                bad &= ~((unsigned)ok << (dt * kRows + r));
            }
        }
        const rsrc_t rx = make_rsrc(x + ((int64_t)S.n * P.C_in + (int64_t)S.g * kCg) * dhw, xbytes);
        const int rowpart = 4 * (qd * P.H_in + qh) * P.W_in;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            // an invalid row gets bit 31 set: past num_records, the load returns zeros
            const unsigned off = ((bad >> sb[u]) << 31) | (unsigned)(rowpart + xo[u]);
            rv[u] = buf_load4(rx, off);
        }
    };
    auto stage = [&](float *l, const f4 (&rv)[kPer]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
            if (lo[u] >= 0) *reinterpret_cast<f4 *>(l + lo[u]) = rv[u];
    };

    // A operands of the block's group: lane (g4, j) holds row i = j (phase
    // delta = j/8, channel co = j%8) and input channel 4cq + g4 of each (D
    // tap, H tap, shift slot).  The group's weights (8 x 8 x KD x KH x KW,
    // contiguous) are first copied to LDS with coalesced loads: read per lane
    // from global memory, each load instruction would touch some 32 cache
    // lines.  (Every lambda here is inlined: a call would take the address of
    // the kernel arguments and copy them to scratch memory.)
    float wr[kTDM][kTHM][kNS][kCg / 4];
    float bo[4]; // bias of the lane's output channels 4*(g4 & 1) + e
    // W taps of both phases per slot, as scalars (selected per lane below;
    // a per-lane select of their addresses would copy the kernel arguments
    // to scratch memory)
    int wt[2][kNS];
#pragma unroll
    for (int dl = 0; dl < 2; ++dl)
#pragma unroll
        for (int sl = 0; sl < kNS; ++sl) wt[dl][sl] = __builtin_amdgcn_readfirstlane(P.wtap[dl][sl]);
    const int kvol = P.KD * P.KH * P.KW;
    float *wl = &lds[0][0];
    {
        const int n4 = kCg * kCg * kvol / 4; // kCg * kCg is a multiple of 4
        const rsrc_t rw = make_rsrc(w + (int64_t)grp * kCg * kCg * kvol, 4 * kCg * kCg * kvol);
        f4 tw[kWPer]; // every load in flight before the first write
#pragma unroll
        for (int u = 0; u < kWPer; ++u) {
            const int i = tid + u * kBlockT;
            tw[u] = buf_load4(rw, i < n4 ? 16u * i : kOutOfRange);
        }
#pragma unroll
        for (int u = 0; u < kWPer; ++u) {
            const int i = tid + u * kBlockT;
            if (i < n4) *reinterpret_cast<f4 *>(wl + 4 * i) = tw[u];
        }
    }
    __syncthreads();
    {
        const int g = grp;
        const int delta = j >> 3, co = j & 7;
        int kdv[kTDM], khv[kTHM]; // the class's taps (table entries past td, th are 0)
#pragma unroll
        for (int dt = 0; dt < kTDM; ++dt) kdv[dt] = __builtin_amdgcn_readfirstlane(P.cls_kd[cls][dt]);
#pragma unroll
        for (int t = 0; t < kTHM; ++t) khv[t] = __builtin_amdgcn_readfirstlane(P.cls_kh[cls][t]);
#pragma unroll
        for (int dt = 0; dt < kTDM; ++dt)
#pragma unroll
            for (int t = 0; t < kTHM; ++t)
#pragma unroll
                for (int sl = 0; sl < kNS; ++sl)
#pragma unroll
                    for (int cq = 0; cq < kCg / 4; ++cq) {
                        // (a mask, not a select: a select of two table
                        // entries becomes a per-lane index into scratch)
                        const int kw = (wt[0][sl] & (delta - 1)) | (wt[1][sl] & -delta);
                        const bool used = dt < td && t < th && kw >= 0;
                        // (every operand of the index is valid whatever `used`
                        // says, so the read needs no branch)
                        const int idx = (((4 * cq + g4) * kCg + co) * P.KD + kdv[dt]) * P.KH * P.KW + khv[t] * P.KW +
                                        max(kw, 0);
                        wr[dt][t][sl][cq] = used ? wl[idx] : 0.0f;
                    }
#pragma unroll
        for (int e = 0; e < 4; ++e) bo[e] = bias ? bias[g * kCg + 4 * (g4 & 1) + e] : 0.0f;
        // wait for these here, not in the step loop (vmcnt is in order)
#pragma unroll
        for (int dt = 0; dt < kTDM; ++dt)
#pragma unroll
            for (int t = 0; t < kTHM; ++t)
#pragma unroll
                for (int sl = 0; sl < kNS; ++sl)
#pragma unroll
                    for (int cq = 0; cq < kCg / 4; ++cq) asm volatile("" : "+v"(wr[dt][t][sl][cq]));
#pragma unroll
        for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(bo[e]));
    }
    __syncthreads(); // weights read before the buffers are cleared
    for (int i = tid; i < 2 * BUF / 4; i += kBlockT)
        *reinterpret_cast<f4 *>(&lds[0][0] + 4 * i) = f4{0.0f, 0.0f, 0.0f, 0.0f};

    // Outputs of lane (g4, j), register e: channel co = 4(g4 & 1) + e, W
    // position o = 2(16 tile + j) + (g4 >> 1).
    const int dhw_out = P.D_out * P.H_out * P.W_out;
    const int ybytes = 4 * P.C_out * dhw_out;
    const int co_l = 4 * (g4 & 1), delta_l = g4 >> 1;

    // Steps k, k + 1 and k + 2 (the last two clamped to the run's last step);
    // later ones by advancing a cursor, not by dividing
    Step S = step_at(P, cls, grp, k_begin);
    Step S1 = step_at(P, cls, grp, min(k_begin + 1, k_end - 1));
    int k2 = min(k_begin + 2, k_end - 1);
    Step S2 = step_at(P, cls, grp, k2);
    const int nqh4 = 4 * ((P.cls_nqh[cls] + 3) / 4), nqd = P.cls_nqd[cls];
    auto advance = [&](Step &T) __attribute__((always_inline)) {
        if (k2 < k_end - 1) {
            ++k2;
            T.iqh0 += 4;
            if (T.iqh0 == nqh4) {
                T.iqh0 = 0;
                if (++T.iqd == nqd) {
                    T.iqd = 0;
                    ++T.n;
                }
            }
        }
    };
    f4 pre0[kPer], pre1[kPer];
    __syncthreads(); // LDS zeroed before the first rows land
    fetch(pre0, S);
    stage(lds[0], pre0);
    fetch(pre0, S1);
    __syncthreads();

    // One step; the loop below runs it twice per trip with the prefetch
    // register sets and the LDS buffers exchanged (compile-time indices).
    auto step = [&](const int k, f4 (&pre)[kPer], f4 (&pre2)[kPer], auto bufc) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        fetch(pre2, S2);

        const f4 zero4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
        f4 acc[kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) acc[t] = zero4;
        // lane's B column: row (dt, r) with r = wv + TH - 1 - t (input H
        // position qh - t), channel 4cq + g4, position m - (smin + sl) with
        // m = 16 tile + j; every read is this base plus a non-negative
        // immediate offset
        typedef const __attribute__((address_space(3))) float *lds_ptr;
        lds_ptr bb = (lds_ptr)(lds[buf] + wv * SLOT + g4 * kPW + P.col0 + j - P.smin - (kNS - 1));
        asm volatile("" : "+v"(bb));
        // B operands of tap group gi = (D tap, H tap), read one group ahead:
        // the reads of group gi + 1 are in flight during group gi's MFMAs
        typedef float BGroup[kCg / 4][kNS][kNT];
        auto load_b = [&](BGroup &b, const int gi) __attribute__((always_inline)) {
            const int dt = gi / TH, t = gi % TH;
#pragma unroll
            for (int cq = 0; cq < kCg / 4; ++cq)
#pragma unroll
                for (int sl = 0; sl < kNS; ++sl)
#pragma unroll
                    for (int tl = 0; tl < kNT; ++tl)
                        b[cq][sl][tl] = bb[(dt * kRows + TH - 1 - t) * SLOT + 4 * cq * kPW + 16 * tl + kNS - 1 - sl];
        };
        auto contract = [&](auto tdc) __attribute__((always_inline)) {
            constexpr int NG = decltype(tdc)::value * TH;
            BGroup bq[2];
            load_b(bq[0], 0);
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                if (gi + 1 < NG) load_b(bq[(gi + 1) & 1], gi + 1);
                const int dt = gi / TH, t = gi % TH;
#pragma unroll
                for (int cq = 0; cq < kCg / 4; ++cq)
#pragma unroll
                    for (int sl = 0; sl < kNS; ++sl)
#pragma unroll
                        for (int tl = 0; tl < kNT; ++tl)
                            acc[tl] = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[dt][t][sl][cq], bq[gi & 1][cq][sl][tl],
                                                                           acc[tl], 0, 0, 0);
            }
        };
        if (td == 2) contract(std::integral_constant<int, 2>{});
        else if (td == 1) contract(std::integral_constant<int, 1>{});

        // the next step's rows go to the other buffer (free since the last
        // barrier) before this step's stores (vmcnt retires in issue order)
#pragma unroll
        for (int u = 0; u < kPer; ++u) asm volatile("" : "+v"(pre[u]));
        stage(lds[buf ^ 1], pre);

        // epilogue: this wave's row qh = qh0 + iqh0 + wv
        const int iqh = S.iqh0 + wv;
        if (iqh < P.cls_nqh[cls]) {
            const int od = P.cls_od0[cls] + S.iqd * P.s_d;
            const int oh = P.cls_oh0[cls] + iqh * P.s_h;
            const int64_t base = ((int64_t)S.n * P.C_out + (int64_t)S.g * kCg) * dhw_out;
            const rsrc_t ry = make_rsrc(y + base, ybytes - 4 * (int)(S.g * kCg) * dhw_out);
            const rsrc_t ra = make_rsrc(FUSED ? add + base : y + base, ybytes - 4 * (int)(S.g * kCg) * dhw_out);
            const unsigned rowoff = 4u * (unsigned)((od * P.H_out + oh) * P.W_out);
#pragma unroll
            for (int tl = 0; tl < kNT; ++tl) {
                const int o = 2 * (16 * tl + j) + delta_l;
                const unsigned vo = o < P.W_out ? rowoff + 4u * (unsigned)(co_l * dhw_out + o) : kOutOfRange;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned so = 4u * (unsigned)(e * dhw_out);
                    const float a = FUSED ? buf_load1(ra, vo, so) : 0.0f;
                    buf_store1(epilogue<EPI>(acc[tl][e], bo[e], a), ry, vo, so);
                }
            }
        }
        __syncthreads();
        S = S1;
        S1 = S2;
        advance(S2);
    };
    for (int k = k_begin; k < k_end; k += 2) {
        step(k, pre0, pre1, std::integral_constant<int, 0>{});
        if (k + 1 < k_end) step(k + 1, pre1, pre0, std::integral_constant<int, 1>{});
    }
}

// W pairing of plan P (stride 2, dilation 1 along W): the shift range and the
// tap of each (phase delta, shift slot).  False when it does not apply.
bool w_pairing(const convt_plan &Pl, WpParams &P) {
    const AxisPlan &A = Pl.ax[2];
    if (A.s != 2 || A.d != 1 || A.K > 8) return false;
    int e[2], r[2];
    for (int dl = 0; dl < 2; ++dl) {
        r[dl] = (dl + A.p) % 2;
        e[dl] = (dl + A.p - r[dl]) / 2;
    }
    int smin = 1 << 30, smax = -(1 << 30);
    for (int dl = 0; dl < 2; ++dl)
        for (int t = A.tap_start[r[dl]]; t < A.tap_start[r[dl] + 1]; ++t) {
            const int sl = A.tap_c[t] - e[dl];
            smin = std::min(smin, sl);
            smax = std::max(smax, sl);
        }
    if (smin > smax || smax - smin + 1 > kNS) return false;
    for (int dl = 0; dl < 2; ++dl)
        for (int s = 0; s < kNS; ++s) P.wtap[dl][s] = -1;
    for (int dl = 0; dl < 2; ++dl)
        for (int t = A.tap_start[r[dl]]; t < A.tap_start[r[dl] + 1]; ++t)
            P.wtap[dl][A.tap_c[t] - e[dl] - smin] = A.tap_k[t];
    P.smin = smin;
    P.nm = (A.L_out + 1) / 2;
    if (P.nm > 16 * kNT) return false;
    // LDS columns: input positions m - sl for m < 16*kNT, sl in [smin, smin + kNS)
    // must fall inside the row; position 0 at col0 (a multiple of 4)
    const int lo = -(smin + kNS - 1);   // lowest input position read
    const int hi = 16 * kNT - 1 - smin; // highest
    P.col0 = lo < 0 ? (-lo + 3) / 4 * 4 : 0;
    if (P.col0 + lo < 0 || P.col0 + std::max(hi + 1, A.L_in) > kPW) return false;
    return true;
}

// Classes along D and H (only those with th_only H taps when th_only > 0);
// false when a class needs more taps than the kernel holds or H taps that are
// not at shifts 0, 1, ...
bool wpair_plan(const convt_plan &Pl, WpParams &P, int th_only = 0) {
    memset(&P, 0, sizeof(P));
    if (Pl.layout != CONVT_LAYOUT_CHANNELS_FIRST || Pl.Cig != kCg || Pl.Cog != kCg) return false;
    const AxisPlan &AD = Pl.ax[0], &AH = Pl.ax[1], &AW = Pl.ax[2];
    if (AW.L_in % 4 != 0 || AW.L_in / 4 > kW4M) return false;
    if (AH.d != 1) return false;
    if (!w_pairing(Pl, P)) return false;
    if (AD.s * AH.s > kMaxCls) return false;
    // the group's weights fit the two LDS buffers while the A operands load
    if (AD.K * AH.K * AW.K > kMaxKvol) return false;
    // 31-bit byte offsets per sample
    if (4 * Pl.C_in * Pl.in_sp >= INT32_MAX || 4 * Pl.C_out * Pl.out_sp >= INT32_MAX) return false;
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.G = (int)Pl.G;
    P.D_in = AD.L_in;
    P.H_in = AH.L_in;
    P.W_in = AW.L_in;
    P.D_out = AD.L_out;
    P.H_out = AH.L_out;
    P.W_out = AW.L_out;
    P.KD = AD.K;
    P.KH = AH.K;
    P.KW = AW.K;
    P.s_d = AD.s;
    P.s_h = AH.s;
    auto cdiv = [](int a, int b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); };
    int c = 0;
    for (int rd = 0; rd < AD.s; ++rd)
        for (int rh = 0; rh < AH.s; ++rh) {
            const int td = AD.tap_start[rd + 1] - AD.tap_start[rd];
            const int th = AH.tap_start[rh + 1] - AH.tap_start[rh];
            if (td > kTDM || th > kTHM) return false;
            for (int t = 0; t < th; ++t)
                if (AH.tap_c[AH.tap_start[rh] + t] != t) return false;
            const int qd0 = std::max(0, cdiv(AD.p - rd, AD.s));
            const int od0 = qd0 * AD.s + rd - AD.p;
            const int nqd = od0 < AD.L_out ? (AD.L_out - 1 - od0) / AD.s + 1 : 0;
            const int qh0 = std::max(0, cdiv(AH.p - rh, AH.s));
            const int oh0 = qh0 * AH.s + rh - AH.p;
            const int nqh = oh0 < AH.L_out ? (AH.L_out - 1 - oh0) / AH.s + 1 : 0;
            if (nqd == 0 || nqh == 0) continue;
            if (th == 0) return false; // a class with no H tap: not this kernel's shape
            if (th_only > 0 && th != th_only) continue;
            P.cls_td[c] = td;
            P.cls_th[c] = th;
            for (int t = 0; t < td; ++t) {
                P.cls_kd[c][t] = AD.tap_k[AD.tap_start[rd] + t];
                P.cls_cd[c][t] = AD.tap_c[AD.tap_start[rd] + t];
            }
            for (int t = 0; t < th; ++t) P.cls_kh[c][t] = AH.tap_k[AH.tap_start[rh] + t];
            P.cls_qd0[c] = qd0;
            P.cls_od0[c] = od0;
            P.cls_nqd[c] = nqd;
            P.cls_qh0[c] = qh0;
            P.cls_oh0[c] = oh0;
            P.cls_nqh[c] = nqh;
            const int64_t steps = Pl.N * (int64_t)nqd * ((nqh + 3) / 4);
            if (steps >= INT32_MAX / 4) return false;
            P.cls_steps[c] = (int)steps;
            ++c;
        }
    P.n_class = c;
    return th_only > 0 || c > 0;
}

} // namespace

bool wpair_supports(const convt_plan &P) {
    WpParams Q;
    return wpair_plan(P, Q);
}

int launch_wpair(const convt_plan &Pl, const float *x, const float *w, const float *bias, const float *add,
                 int act, float *y, void *stream) {
    WpParams all;
    if (!wpair_plan(Pl, all)) return (int)hipErrorInvalidValue;
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    // one launch per H tap count present, over the classes with that many
    for (int th = 1; th <= kTHM; ++th) {
        WpParams P;
        if (!wpair_plan(Pl, P, th)) return (int)hipErrorInvalidValue;
        if (P.n_class == 0) continue;
        // Steps per block: the grid holds about CONVT_WPAIR_ROUNDS rounds of
        // resident workgroups (three per CU), each with the same work (a step
        // costs its class's D taps), so that no CU keeps the heavy blocks alone.
        int64_t work = 0;
        for (int c = 0; c < P.n_class; ++c) work += Pl.G * (int64_t)P.cls_steps[c] * std::max(1, P.cls_td[c]);
        const int64_t target = (int64_t)cus * 3 * CONVT_WPAIR_ROUNDS;
        const double per_block = (double)work / (double)std::max<int64_t>(1, target);
        int blocks = 0;
        for (int c = 0; c < P.n_class; ++c) {
            const int64_t spb = std::max<int64_t>(2, (int64_t)(per_block / std::max(1, P.cls_td[c]) + 0.999));
            P.cls_spb[c] = (int)std::min<int64_t>(spb, P.cls_steps[c]);
            P.cls_bpg[c] = (P.cls_steps[c] + P.cls_spb[c] - 1) / P.cls_spb[c];
            P.cls_block0[c] = blocks;
            if ((int64_t)blocks + Pl.G * (int64_t)P.cls_bpg[c] >= INT32_MAX) return (int)hipErrorInvalidValue;
            blocks += (int)Pl.G * P.cls_bpg[c];
        }
        P.cls_block0[P.n_class] = blocks;
        if (blocks == 0) continue;
        auto go = [&](auto thc) {
            with_epi(add != nullptr, act, [&](auto E) {
                hipLaunchKernelGGL((k_generic_wpair<decltype(thc)::value, decltype(E)::value>), dim3(blocks),
                                   dim3(kBlockT), 0, (hipStream_t)stream, P, (int)Pl.N, x, w, bias, add, y);
            });
        };
        switch (th) {
        case 1: go(std::integral_constant<int, 1>{}); break;
        case 2: go(std::integral_constant<int, 2>{}); break;
        case 3: go(std::integral_constant<int, 3>{}); break;
        case 4: go(std::integral_constant<int, 4>{}); break;
        default: go(std::integral_constant<int, 5>{}); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

} // namespace convt
