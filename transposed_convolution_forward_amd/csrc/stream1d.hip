// 1D streaming path: phase-decomposed gather with the channel contraction on
// fp32 MFMA (v_mfma_f32_16x16x4_f32) and the group's weights resident in VGPRs.
//
// Method.  With t = o + p = q*S + r (0 <= r < S), tap k feeds output o iff
// k*D = r (mod S), from input i = q - c_k, c_k = floor(k*D/S) (the per-axis
// phase tables of convt_internal.h, fixed here at compile time by K, S, D).  So
// for one position q all S outputs o = q*S + r - p, r = 0..S-1, form one
// contiguous run, and phase r is the dense stride-1 contraction
//   Y_r[co, q] = sum_{k in T_r} sum_ci W[ci, co, k] * X[ci, q - c_k].
// An empty T_r leaves the bias.  "Kimi-K2.6 l1_p79" transcript (ConvTranspose1d,
// dilation 2): with stride 2, padding 1, dilation 2 the odd outputs o = 2m-1
// are sum_k x[:, m-k] @ w[:, :, k] and the even outputs hold no term; the page
// reads this as a stride-1 convolution interleaved with empty positions and
// reuses one input load across all output channels.
//
// Mapping (one wave = 64 lanes, lane = 16*g4 + j):
//   work item = (n, g, 64 consecutive positions q0 .. q0+63).
//   MFMA D[co][col] = sum_kk A[co][kk] B[kk][col] with A = W^T (16 co x 4 ci,
//   held in VGPRs for the whole kernel) and B = X (4 ci x 16 positions).
//   Column j of N-tile t is position q0 + 4j + t, so lane (g4, j) loads one
//   float4 x[ci = 4*cig + g4][q0 + 4j .. +3] (coalesced, 256 B per ci row) and
//   one more float4 four positions back; every shift q - c (c <= 4) is then a
//   register of one of the two loads.  The accumulator of lane (g4, j),
//   register e, holds co = 16*ct + 4*g4 + e at positions q0 + 4j + t, t = 0..3:
//   4*S consecutive outputs of one row, written with S float4 stores
//   (dword-aligned; rows of odd length are not 16-byte aligned).
// Atomic-free: every output element is stored once, by one lane.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "convt_internal.h"
#include "epilogue.hpp"

namespace convt {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kTileQ = 64; // positions per work item

__device__ __forceinline__ f4 load4u(const float *p) {
    f4 v;
    __builtin_memcpy(&v, p, 16);
    return v;
}

// A buffer resource over one batch sample of y: the common-path stores then
// take a row-invariant lane offset plus a uniform item offset (no 64-bit
// address arithmetic per store).  Per-sample byte offsets stay below 2^31.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}
// The common-path segment stores are non-temporal (cache policy nt): the
// output is written once and never read back here, and on the 1D layer that
// streams 1.07 GB of output this is 3.5% faster than default-policy stores.
constexpr int kStoreNT = 2;
__device__ __forceinline__ void buf_store4(f4 v, rsrc_t r, unsigned voff, unsigned soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, v),
                                           r, voff, soff, kStoreNT);
}

__device__ __forceinline__ f4 buf_load4(rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Compile-time phase table of one axis.
template <int K, int S, int D> struct Phases {
    static constexpr int r_of(int k) { return (k * D) % S; }
    static constexpr int c_of(int k) { return (k * D) / S; }
    static constexpr bool nonempty(int r) {
        for (int k = 0; k < K; ++k)
            if (r_of(k) == r) return true;
        return false;
    }
    static constexpr int slot(int r) { // index of phase r among the non-empty ones
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

struct Stream1dParams {
    int C_in, C_out, G;
    int L_in, L_out, p;
    int n_st;      // work items (64-position tiles) per (n, g) row
    int st_lo;     // first tile index (tile t covers q in [64t, 64t+64))
    int per_block; // consecutive work items per workgroup
    int64_t total; // N * G * n_st
};

// The x tile of one work item: CIG rows (input channels of the group) of
// positions q0-4 .. q0+63, 17 float4 per row.  In LDS the rows go in groups
// of four (the channels one MFMA step reads): positions q0 .. q0+63 of row
// 4g + i at group g, offset 64i, so the four rows of one 16-byte operand read
// start on the same bank (conflict-free), and the four halo float4s
// (q0-4 .. q0-1) after them at offset 256 + 4i.
constexpr int kRowF4 = (kTileQ + 4) / 4;
constexpr int kGrpF = 4 * kTileQ + 16; // floats per group of four rows

// LDS float offset of float4 f (row f / 17, column f % 17) of the tile.
__device__ __forceinline__ int tile_lds_off(int f) {
    const int row = f / kRowF4, c4 = f % kRowF4;
    const int grp = row >> 2, i = row & 3;
    return grp * kGrpF + (c4 == 0 ? 4 * kTileQ + 4 * i : 64 * i + 4 * (c4 - 1));
}

// Fetch of one x tile into registers, branch-free so that the loads stay in
// flight across the contraction of the current tile: every float4 is loaded
// from a position clamped into the row (needs L_in >= 4); the shift back and
// the zeroing of positions outside [0, L_in) happen when the tile is written
// to LDS.  Offsets are 32-bit, relative to the thread's fixed offset xo[u]
// (row and float4 column in a tile wholly inside the row), through the
// resource over the row set's input rows: per-lane 64-bit addresses would
// cost registers the contraction needs.
template <int CIG, int NT>
__device__ __forceinline__ void tile_fetch(f4 (&r)[(CIG * kRowF4 + NT - 1) / NT], rsrc_t rx,
                                           const unsigned (&xo)[(CIG * kRowF4 + NT - 1) / NT], int L_in,
                                           int q0, int tid) {
    constexpr int NF = CIG * kRowF4;
    constexpr int PER = (NF + NT - 1) / NT;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c4 = min(tid + u * NT, NF - 1) % kRowF4;
        const int pos = q0 - 4 + 4 * c4;
        const int cp = min(max(pos, 0), L_in - 4);
        // xo[u] holds 4*(row*L_in + 4*c4); the sum wraps back into range
        r[u] = buf_load4(rx, xo[u] + 4u * (unsigned)(cp - 4 * c4), 0);
    }
}

__device__ __forceinline__ float pick4(const f4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The same fetch for a tile wholly inside the row (q0 >= 4, q0 + 64 <= L_in),
// through a buffer resource over the row set's CIG input rows: per thread a
// fixed byte offset xo[u] (row and float4 column) plus the uniform
// 4*(q0 - 4) in the scalar offset, so no address arithmetic per tile.
template <int CIG, int NT>
__device__ __forceinline__ void tile_fetch_inner(f4 (&r)[(CIG * kRowF4 + NT - 1) / NT], rsrc_t rx,
                                                 const unsigned (&xo)[(CIG * kRowF4 + NT - 1) / NT],
                                                 int q0) {
    constexpr int PER = (CIG * kRowF4 + NT - 1) / NT;
#pragma unroll
    for (int u = 0; u < PER; ++u) r[u] = buf_load4(rx, xo[u], 4u * (unsigned)(q0 - 4));
}

template <int CIG, int NT>
__device__ __forceinline__ void tile_store_lds(float *lds, const f4 (&r)[(CIG * kRowF4 + NT - 1) / NT],
                                               const int (&lo)[(CIG * kRowF4 + NT - 1) / NT], int L_in,
                                               int q0, int tid) {
    constexpr int NF = CIG * kRowF4;
    constexpr int PER = (NF + NT - 1) / NT;
    if (q0 - 4 >= 0 && q0 + kTileQ <= L_in) { // whole tile inside the row (uniform)
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int f = tid + u * NT;
            if (f < NF) {
                *reinterpret_cast<f4 *>(lds + lo[u]) = r[u];
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int f = tid + u * NT;
        if (f < NF) {
            const int c4 = f % kRowF4;
            const int pos = q0 - 4 + 4 * c4;
            const int sh = pos - min(max(pos, 0), L_in - 4); // in [-3, 3]
            f4 v;
            v.x = (pos + 0 >= 0 && pos + 0 < L_in) ? pick4(r[u], sh + 0) : 0.0f;
            v.y = (pos + 1 >= 0 && pos + 1 < L_in) ? pick4(r[u], sh + 1) : 0.0f;
            v.z = (pos + 2 >= 0 && pos + 2 < L_in) ? pick4(r[u], sh + 2) : 0.0f;
            v.w = (pos + 3 >= 0 && pos + 3 < L_in) ? pick4(r[u], sh + 3) : 0.0f;
            *reinterpret_cast<f4 *>(lds + lo[u]) = v;
        }
    }
}

// Winograd F(4,3) (Lavin and Gray, "Fast Algorithms for Convolutional Neural
// Networks", CVPR 2016) for a layer whose one phase has three taps at input
// shifts 0, 1, 2 (K = 3 and dilation = stride, e.g. stride 2, dilation 2):
// the four outputs y[q+i] = sum_c w_c x[q+i-c], i = 0..3, are
// A^T [(G g) . (B^T d)] with d = x[q-2 .. q+3] and g_k = w_{2-k}.  The
// contraction over input channels then runs on the six transformed
// components (six MFMAs per 4 channels and 16 tiles of 4 positions, against
// twelve for the taps directly), the input transform B^T d once per tile when
// it is staged in LDS, the weight transform G g once per kernel, and the
// output transform A^T m in registers before the epilogue.  fp32 throughout;
// the transforms' constants (4, 5, 2, 8, 1/6, 1/12, 1/24) raise the rounding
// error a few times over the direct sum (about 3e-6 absolute on unit-variance
// inputs with 96 products per output).
#ifndef CONVT_S1D_WINOGRAD
#define CONVT_S1D_WINOGRAD 1
#endif
constexpr int kWinoTau = kTileQ / 4; // tiles of 4 positions per work item

// Thread tid stages (channel ci, tile tau) pairs p = tid + u*NT of the item,
// ci = p / 16, tau = p % 16: inputs q0 + 4tau - 4 .. q0 + 4tau + 3 as two
// float4 (positions clamped into the row, as in tile_fetch).
template <int CIG, int NT> constexpr int kWinoPairs = (CIG * kWinoTau + NT - 1) / NT;
template <int CIG, int NT> using WinoRegs = f4[2 * kWinoPairs<CIG, NT>];
template <int CIG, int NT> using WinoOffs = unsigned[kWinoPairs<CIG, NT>];

template <int CIG, int NT>
__device__ __forceinline__ void wino_fetch(WinoRegs<CIG, NT> &r, rsrc_t rx, const WinoOffs<CIG, NT> &xo,
                                           int L_in, int q0, int tid) {
#pragma unroll
    for (int u = 0; u < kWinoPairs<CIG, NT>; ++u) {
        const int tau = min(tid + u * NT, CIG * kWinoTau - 1) % kWinoTau;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int pos = q0 + 4 * tau - 4 + 4 * h;
            const int cp = min(max(pos, 0), L_in - 4);
            // xo[u] holds 4*(ci*L_in + 4*tau); the sum wraps back into range
            r[2 * u + h] = buf_load4(rx, xo[u] + 4u * (unsigned)(cp - 4 * tau), 0);
        }
    }
}

// The same for a tile wholly inside the row: fixed byte offsets xo[u] of the
// pair's first float4 relative to position q0 - 4.
template <int CIG, int NT>
__device__ __forceinline__ void wino_fetch_inner(WinoRegs<CIG, NT> &r, rsrc_t rx,
                                                 const WinoOffs<CIG, NT> &xo, int q0) {
#pragma unroll
    for (int u = 0; u < kWinoPairs<CIG, NT>; ++u) {
        r[2 * u] = buf_load4(rx, xo[u], 4u * (unsigned)(q0 - 4));
        r[2 * u + 1] = buf_load4(rx, xo[u] + 16u, 4u * (unsigned)(q0 - 4));
    }
}

// Input transform of the staged pairs into LDS: component xi of (ci, tau) at
// xi*CIG*16 + ci*16 + tau, so the B operand of (component, 4 channels) is 64
// consecutive floats (lane 16*g4 + j reads channel 4cig + g4, tile j).
template <int CIG, int NT>
__device__ __forceinline__ void wino_store_lds(float *lds, const WinoRegs<CIG, NT> &r, int L_in,
                                               int q0, int tid) {
    const bool inner = q0 - 4 >= 0 && q0 + kTileQ <= L_in;
#pragma unroll
    for (int u = 0; u < kWinoPairs<CIG, NT>; ++u) {
        const int pr = tid + u * NT;
        if (pr >= CIG * kWinoTau) continue;
        const int tau = pr % kWinoTau;
        f4 h[2] = {r[2 * u], r[2 * u + 1]};
        if (!inner) { // shift back from the clamped position, zero outside the row
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int pos = q0 + 4 * tau - 4 + 4 * b;
                const int sh = pos - min(max(pos, 0), L_in - 4);
                const f4 v = h[b];
                h[b].x = (pos + 0 >= 0 && pos + 0 < L_in) ? pick4(v, sh + 0) : 0.0f;
                h[b].y = (pos + 1 >= 0 && pos + 1 < L_in) ? pick4(v, sh + 1) : 0.0f;
                h[b].z = (pos + 2 >= 0 && pos + 2 < L_in) ? pick4(v, sh + 2) : 0.0f;
                h[b].w = (pos + 3 >= 0 && pos + 3 < L_in) ? pick4(v, sh + 3) : 0.0f;
            }
        }
        const float d0 = h[0].z, d1 = h[0].w, d2 = h[1].x, d3 = h[1].y, d4 = h[1].z, d5 = h[1].w;
        // B^T d
        const float t1 = fmaf(-4.0f, d2, d4), t2 = fmaf(-4.0f, d1, d3);
        const float t3 = d4 - d2, t4 = 2.0f * (d3 - d1);
        float *o = lds + pr;
        o[0 * CIG * kWinoTau] = fmaf(4.0f, d0, fmaf(-5.0f, d2, d4));
        o[1 * CIG * kWinoTau] = t1 + t2;
        o[2 * CIG * kWinoTau] = t1 - t2;
        o[3 * CIG * kWinoTau] = t3 + t4;
        o[4 * CIG * kWinoTau] = t3 - t4;
        o[5 * CIG * kWinoTau] = fmaf(4.0f, d1, fmaf(-5.0f, d3, d5));
    }
}

// Output lines.  Rows may have any length, so the outputs o_t .. o_t + 64S - 1
// of a work item start anywhere in a 128-byte cache line, at a different place
// in every row; stored as they stand, the line at each end of the run is split
// between two items written microseconds apart, and such partly written lines
// drain to HBM far slower than whole ones (runs aligned to 64 bytes only are
// still 15% slower than runs aligned to 128).  So for each row an item stores
// the 64S outputs from the line boundary at or before o_t: the first a of them
// (0 <= a < 32, the offset of o_t in its line) are the previous item's last
// outputs, carried over, and its own last a outputs are carried to the next
// item.  The row-dependent shift by a and the carry pass through LDS that
// belongs to one wave (no barrier): a staging row per accumulator row group,
// holding the carry at [32 - a, 32) and the item's outputs at [32, 32 + 64S),
// and a 32-float carry slot per output row.  Store c of lane j then writes
// the 16 bytes at 64c + 4j of its row's segment, so one store instruction
// covers four rows with 256 contiguous, line-aligned bytes each.
constexpr int kLineF = 32; // floats per 128-byte line
// A multiple of 64 dwords, so the four rows a store instruction reads start
// on the same LDS bank (16-byte reads of such rows are conflict-free); it
// holds the common path's layout (up to 31 + 32 + 64S floats).
template <int S> constexpr int stage_pitch() { return (kLineF + 64 * S + kLineF + 63) / 64 * 64; }

// Tuning knobs: minimum waves per SIMD the register allocation must allow,
// and how many rounds of resident workgroups the grid holds (one round: every
// workgroup starts at once and walks a long run of items, so the per-workgroup
// start-up is paid once per CU slot; measured 2.5% faster than two rounds).
#ifndef CONVT_S1D_WAVES_PER_EU
#define CONVT_S1D_WAVES_PER_EU 3
#endif
#ifndef CONVT_S1D_ROUNDS
#define CONVT_S1D_ROUNDS 1
#endif
// Channels-last kernel: waves per SIMD the register allocation must allow,
// and how many items ahead a wave loads its inputs (1 or 2).
#ifndef CONVT_NLC_WAVES_PER_EU
#define CONVT_NLC_WAVES_PER_EU 2
#endif
#ifndef CONVT_NLC_PREFETCH
#define CONVT_NLC_PREFETCH 2
#endif

// One workgroup = COG/16 waves; wave w owns output channels 16w .. 16w+15 of
// the group and all 64 positions of the work item; the waves share the x tile
// through LDS, double-buffered: the tile of the next work item is fetched
// from HBM into registers while the current one is contracted.
template <int CIG, int COG, int K, int S, int D, int EPI>
__global__ __launch_bounds__(COG * 4)
__attribute__((amdgpu_waves_per_eu(CONVT_S1D_WAVES_PER_EU))) void k_stream1d(const Stream1dParams P,
                                                      const float *__restrict__ x,
                                                      const float *__restrict__ w,
                                                      const float *__restrict__ bias,
                                                      const float *add, float *y) {
    using Ph = Phases<K, S, D>;
    constexpr bool ADD = epi_add(EPI);
    constexpr int NCIG = CIG / 4;
    constexpr int COT = COG / 16;
    constexpr int NT = COG * 4; // threads per workgroup
    constexpr int NP = Ph::count() > 0 ? Ph::count() : 1;
    constexpr int PER = (CIG * kRowF4 + NT - 1) / NT;
    // Winograd F(4,3) for one phase of three taps at shifts 0, 1, 2
    constexpr bool WINO = CONVT_S1D_WINOGRAD && K == 3 && S == D;
    constexpr int NPAIR = kWinoPairs<CIG, NT>;
    constexpr int NPRE = WINO ? 2 * NPAIR : PER; // prefetch registers (float4)
    constexpr int NXO = WINO ? NPAIR : PER;
    constexpr int NWR = WINO ? 6 : K;             // weight registers per channel group
    static_assert(CIG % 4 == 0 && COG % 16 == 0, "tile shape");
    static_assert(Ph::cmax() <= 4, "input shift beyond the 4-position halo");

    __shared__ __attribute__((aligned(16))) float lds[2][WINO ? 6 * CIG * kWinoTau : CIG / 4 * kGrpF];
    __shared__ __attribute__((aligned(16))) float ostage[COT][4][stage_pitch<S>()];
    __shared__ __attribute__((aligned(16))) float ocarry[COT][4][4][kLineF]; // [wave][g4][e][slot]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ct = tid >> 6; // this wave's co-tile
    const int j = lane & 15;
    const int g4 = lane >> 4;
    const int64_t it0 = (int64_t)blockIdx.x * P.per_block;
    const int64_t it_end = it0 + P.per_block < P.total ? it0 + P.per_block : P.total;
    if (it0 >= it_end) return;
    const int n_items = (int)(it_end - it0);

    // (n, g, tile) of the first item; later items advance incrementally
    int st = (int)(it0 % P.n_st);
    int ng = (int)(it0 / P.n_st);
    auto xrow_of = [&](int ng_) { return x + (int64_t)ng_ * CIG * P.L_in; }; // (n*G+g)*CIG = n*C_in + g*CIG

    unsigned xo[NXO]; // byte offsets of this thread's float4 (pair) in a tile wholly inside the row
#pragma unroll
    for (int u = 0; u < NXO; ++u) {
        if constexpr (WINO) {
            const int pr = min(tid + u * NT, CIG * kWinoTau - 1);
            xo[u] = 4u * (unsigned)((pr / kWinoTau) * P.L_in + 4 * (pr % kWinoTau));
        } else {
            const int f = min(tid + u * NT, CIG * kRowF4 - 1);
            xo[u] = 4u * (unsigned)((f / kRowF4) * P.L_in + 4 * (f % kRowF4));
        }
    }
    int lo[PER]; // LDS offsets of this thread's float4 of the tile
#pragma unroll
    for (int u = 0; u < PER; ++u) lo[u] = tile_lds_off(min(tid + u * NT, CIG * kRowF4 - 1));
    const int x_bytes = 4 * CIG * P.L_in; // one row set's input rows (below 2 GiB)
    // Tiles inside the row take buffer loads at fixed offsets; the others clamp.
    auto fetch = [&](f4 (&r)[NPRE], int ng_, int q0_) {
        const bool inner = q0_ - 4 >= 0 && q0_ + kTileQ <= P.L_in;
        const rsrc_t rx = make_rsrc(const_cast<float *>(xrow_of(ng_)), x_bytes);
        if constexpr (WINO) {
            if (inner) wino_fetch_inner<CIG, NT>(r, rx, xo, q0_);
            else wino_fetch<CIG, NT>(r, rx, xo, P.L_in, q0_, tid);
        } else {
            if (inner) tile_fetch_inner<CIG, NT>(r, rx, xo, q0_);
            else tile_fetch<CIG, NT>(r, rx, xo, P.L_in, q0_, tid);
        }
    };
    auto stage = [&](float *l, const f4 (&r)[NPRE], int q0_) {
        if constexpr (WINO) wino_store_lds<CIG, NT>(l, r, P.L_in, q0_, tid);
        else tile_store_lds<CIG, NT>(l, r, lo, P.L_in, q0_, tid);
    };

    f4 pre[NPRE];
    fetch(pre, ng, (P.st_lo + st) * kTileQ);
    stage(lds[0], pre, (P.st_lo + st) * kTileQ);
    __syncthreads();

    // A operands: W[g*CIG + 4*cig + g4][16*ct + j][k], or with Winograd the
    // six components of G g for g_k = W[..][2-k]
    float wr[NWR][NCIG];
    float br[4];       // bias of rows co = 16ct + 4g4 + e
    bool chain = false; // the previous item left its last outputs of each row in ocarry
    // Per row set (n, g): the sample's y resource, and per row group e the
    // lane's byte offset of its segment relative to the item offset
    // 4*(o_t - 32), folding in a (the run's offset in its 128-byte line, the
    // same for every item of a row since items advance 64S floats).
    int rs_ng = -1;
    rsrc_t ry = make_rsrc(y, 0);
    unsigned lane_off[4] = {0u, 0u, 0u, 0u};
    int a_row[4] = {0, 0, 0, 0};
    float *srow = &ostage[ct][g4][0];
    // Common-path staging of row group e: run output m (m = -32 .. 64S-1,
    // negative = carried) at srow[32 + a + m].  The line-aligned segment then
    // starts at srow[32] in every row, whatever a is, so chunk c of lane j is
    // the aligned float4 at srow[32 + 4j + 64c].  cb[e] points at the lane's
    // carry slot srow[a + j]; the lane's own outputs m = 4Sj + u are written
    // at cb[e][32 + (4S - 1)j + u] straight from the accumulators (dword
    // writes, no register packing).
    typedef __attribute__((address_space(3))) float *lds_fptr;
    lds_fptr cb[4];
    const int own = kLineF + (4 * S - 1) * j;
    const f4 *segp = reinterpret_cast<const f4 *>(srow + kLineF + 4 * j);

    // The weights of group g (A operands) and its bias.
    auto load_group = [&](int g) {
            if constexpr (WINO) {
#pragma unroll
                for (int cig = 0; cig < NCIG; ++cig) {
                    const float *wp = w + ((int64_t)(g * CIG + 4 * cig + g4) * COG + 16 * ct + j) * K;
                    const float g0 = wp[2], g1 = wp[1], g2 = wp[0]; // g_k = w_{2-k}
                    // G g, G = [1/4 0 0; -1/6 -1/6 -1/6; -1/6 1/6 -1/6; 1/24 1/12 1/6; 1/24 -1/12 1/6; 0 0 1]
                    const float s02 = g0 + g2;
                    wr[0][cig] = 0.25f * g0;
                    wr[1][cig] = -(s02 + g1) * (1.0f / 6.0f);
                    wr[2][cig] = -(s02 - g1) * (1.0f / 6.0f);
                    const float e02 = fmaf(g0, 1.0f / 24.0f, g2 * (1.0f / 6.0f));
                    wr[3][cig] = fmaf(g1, 1.0f / 12.0f, e02);
                    wr[4][cig] = fmaf(g1, -1.0f / 12.0f, e02);
                    wr[5][cig] = g2;
                }
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int cig = 0; cig < NCIG; ++cig)
                        wr[k][cig] = w[((int64_t)(g * CIG + 4 * cig + g4) * COG + 16 * ct + j) * K + k];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) br[e] = bias ? bias[g * COG + 16 * ct + 4 * g4 + e] : 0.0f;
            // Wait for these loads here: an empty asm that reads and redefines
            // the registers puts the wait at the group change, so the MFMA
            // block never waits on them (which, vmcnt being in order, would
            // also wait on the prefetched tiles).
#pragma unroll
            for (int k = 0; k < NWR; ++k)
#pragma unroll
                for (int cig = 0; cig < NCIG; ++cig) asm volatile("" : "+v"(wr[k][cig]));
#pragma unroll
            for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(br[e]));
    };
    auto advance = [&](int &st_, int &ng_) {
        if (++st_ == P.n_st) {
            st_ = 0;
            ++ng_;
        }
    };

    // Tiles are fetched two items ahead, into two register sets that swap
    // roles every item (the loop below runs the item twice per trip with the
    // sets and the LDS buffers exchanged, all compile-time indices): the wait
    // before a tile is staged then covers only loads issued an item earlier.
    // Items ii+1 and ii+2 are (st1, ng1) and (st2, ng2), clamped to the
    // workgroup's last item (fetched again, never used).
    int st1 = st, ng1 = ng;
    if (n_items > 1) advance(st1, ng1);
    int st2 = st1, ng2 = ng1;
    if (n_items > 2) advance(st2, ng2);
    int wg = ng % P.G;
    load_group(wg);
    f4 pre2[NPRE];
    fetch(pre, ng1, (P.st_lo + st1) * kTileQ);

    int ii = 0;
    auto item = [&](f4 (&preN)[NPRE], f4 (&preF)[NPRE], auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        if (P.G > 1 && ng % P.G != wg) { // a new group: its weights
            wg = ng % P.G;
            load_group(wg);
        }
        const int g = wg;
        const int n = ng / P.G;
        const int q0 = (P.st_lo + st) * kTileQ;
        const bool has_next = ii + 1 < n_items;
        // the tile of item ii+2 (clamped), in flight across this item and the next
        fetch(preF, ng2, (P.st_lo + st2) * kTileQ);

        // The bias enters as the accumulators' start value: the first MFMA of
        // each phase takes it as its accumulator input.
        const f4 bias4 = f4{br[0], br[1], br[2], br[3]};
        f4 acc[NP][4];
        if constexpr (Ph::count() == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[0][t] = bias4;
        } else if constexpr (WINO) {
            // m_xi[co][tile j] = sum_ci U_xi[co][ci] V_xi[ci][j]; the bias
            // enters through m_1, whose A^T column is all ones
            const float *vb = lds[buf] + 16 * g4 + j;
            const f4 zero4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
            f4 m[6];
#pragma unroll
            for (int cig = 0; cig < NCIG; ++cig)
#pragma unroll
                for (int xi = 0; xi < 6; ++xi)
                    m[xi] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        wr[xi][cig], vb[(xi * CIG + 4 * cig) * kWinoTau],
                        cig == 0 ? (xi == 1 ? bias4 : zero4) : m[xi], 0, 0, 0);
            // A^T m: positions q0 + 4j + t
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s12 = m[1][e] + m[2][e], d12 = m[1][e] - m[2][e];
                const float s34 = m[3][e] + m[4][e], d34 = m[3][e] - m[4][e];
                acc[0][0][e] = m[0][e] + s12 + s34;
                acc[0][1][e] = fmaf(2.0f, d34, d12);
                acc[0][2][e] = fmaf(4.0f, s34, s12);
                acc[0][3][e] = fmaf(8.0f, d34, d12) + m[5][e];
            }
        } else {
            // lane j's float4 at q0+4j (row 4cig+g4) and the one before it
            // (the halo float4 for lane 0)
            const float *cp = lds[buf] + 64 * g4 + 4 * j;
            const float *pp = lds[buf] + (j > 0 ? 64 * g4 + 4 * j - 4 : 4 * kTileQ + 4 * g4);
#pragma unroll
            for (int cig = 0; cig < NCIG; ++cig) {
                const f4 pv = *reinterpret_cast<const f4 *>(pp + cig * kGrpF); // q0+4j-4 .. -1
                const f4 cv = *reinterpret_cast<const f4 *>(cp + cig * kGrpF); // q0+4j .. +3
                const float cur[4] = {cv.x, cv.y, cv.z, cv.w};
                const float prv[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int c = Ph::c_of(k);
                    const int r = Ph::r_of(k);
                    const int sl = Ph::slot(r);
                    const bool first = cig == 0 && k == Ph::first_k(r);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float bv = (t >= c) ? cur[(t - c) & 3] : prv[(t - c + 4) & 3];
                        acc[sl][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            wr[k][cig], bv, first ? bias4 : acc[sl][t], 0, 0, 0);
                    }
                }
            }
        }

        // The next tile goes to the other LDS buffer (free since the last
        // barrier) before this item's stores are issued: the one vector-memory
        // counter retires loads and stores in issue order, so the wait for the
        // prefetch must not come after the stores.  The write is unconditional
        // (after the last item it copies stale registers into a buffer nobody
        // reads): were it conditional, the compiler would keep the prefetch
        // pending along the skipping path and wait for it, and with it for every
        // store, before the next fetch.
#pragma unroll
        for (int u = 0; u < NPRE; ++u) asm volatile("" : "+v"(preN[u])); // item ii+1's tile landed here
        stage(lds[buf ^ 1], preN, (P.st_lo + st1) * kTileQ);

        // Epilogue (see stage_pitch).  Rows co = g*COG + 16ct + 4g4 + e; the
        // item's outputs of a row are o_t .. o_t + 64S - 1, o_t = q0*S - p.
        // Items touching a row end take a guarded element-wise path and break
        // the carry chain: the item before flushes its carry itself, the one
        // after leaves the first a outputs of its segment alone.
        const int o_t = q0 * S - P.p;
        const bool interior = (o_t >= 0) && (o_t + 64 * S <= P.L_out);
        const bool chain_in = chain;
        const bool chain_out =
            interior && has_next && st1 != 0 && o_t + 128 * S <= P.L_out; // next: same rows, interior
        chain = chain_out;
        if (rs_ng != ng) { // a new row set
            rs_ng = ng;
            ry = make_rsrc(y + (int64_t)n * P.C_out * P.L_out, (int)(4 * (int64_t)P.C_out * P.L_out));
            const unsigned yel = (unsigned)((uintptr_t)y >> 2) + (unsigned)((int64_t)n * P.C_out * P.L_out);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = g * COG + 16 * ct + 4 * g4 + e;
                a_row[e] = (int)((yel + (unsigned)row * (unsigned)P.L_out + (unsigned)o_t) & (kLineF - 1u));
                // non-negative (the range check drops a store whose vector
                // offset wraps): kLineF floats are moved out of the scalar
                // item offset, which stays >= 0 since a chained item has
                // o_t >= 64S
                lane_off[e] = 4u * ((unsigned)row * (unsigned)P.L_out + (unsigned)(4 * j + kLineF - a_row[e]));
                cb[e] = (lds_fptr)(srow + a_row[e] + j);
            }
        }
        if (!ADD && interior && chain_in && chain_out) {
            // The common item: staging, carry and whole-line stores, with no
            // per-store address arithmetic.
            const unsigned item4 = 4u * (unsigned)(o_t - kLineF);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const lds_fptr c = cb[e];
                // The previous run's last 32 outputs, then this run's outputs.
                c[0] = ocarry[ct][g4][e][j];
                c[16] = ocarry[ct][g4][e][j + 16];
                const lds_fptr o = c + own;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int r = 0; r < S; ++r) {
                        float a = br[e];
                        if constexpr (Ph::count() > 0)
                            if (Ph::nonempty(r)) a = acc[Ph::slot(r)][t][e];
                        o[S * t + r] = activate<EPI>(a);
                    }
                // This run's last 32 outputs (m = 64S - 32 + i) become the next
                // run's carry (one wave's LDS accesses are performed in order).
                ocarry[ct][g4][e][j] = c[64 * S];
                ocarry[ct][g4][e][j + 16] = c[64 * S + 16];
#pragma unroll
                for (int q = 0; q < S; ++q) buf_store4(segp[16 * q], ry, lane_off[e] + 256u * q, item4);
            }
        } else {
        float *yrow = y + ((int64_t)n * P.C_out + (int64_t)g * COG + 16 * ct + 4 * g4) * P.L_out + o_t;
        const float *arow = ADD ? add + (yrow - y) : nullptr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float *yr = yrow + (int64_t)e * P.L_out;
            const float *ar = ADD ? arow + (int64_t)e * P.L_out : nullptr;
            float v[4 * S];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < S; ++r) {
                    float a = br[e];
                    if constexpr (Ph::count() > 0)
                        if (Ph::nonempty(r)) a = acc[Ph::slot(r)][t][e];
                    v[t * S + r] = a;
                }
            if (interior) {
                if constexpr (ADD) {
#pragma unroll
                    for (int c = 0; c < S; ++c) {
                        const f4 a4 = load4u(ar + 4 * S * j + 4 * c); // add_input: any alignment
                        v[4 * c + 0] = finish<EPI>(v[4 * c + 0], a4.x);
                        v[4 * c + 1] = finish<EPI>(v[4 * c + 1], a4.y);
                        v[4 * c + 2] = finish<EPI>(v[4 * c + 2], a4.z);
                        v[4 * c + 3] = finish<EPI>(v[4 * c + 3], a4.w);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 4 * S; ++u) v[u] = activate<EPI>(v[u]);
                }
                const int a = (int)(((uintptr_t)yr >> 2) & (kLineF - 1)); // o_t's offset in its line
                if (chain_in) { // the previous run's last 32 outputs
                    srow[j] = ocarry[ct][g4][e][j];
                    srow[j + 16] = ocarry[ct][g4][e][j + 16];
                }
#pragma unroll
                for (int c = 0; c < S; ++c)
                    *reinterpret_cast<f4 *>(srow + kLineF + 4 * S * j + 4 * c) =
                        f4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
                if (chain_out) { // this run's last 32 outputs, straight from the lanes holding them
#pragma unroll
                    for (int c = 0; c < S; ++c) {
                        const int i0 = 4 * S * j + 4 * c - (64 * S - kLineF);
                        if (i0 >= 0)
                            *reinterpret_cast<f4 *>(&ocarry[ct][g4][e][i0]) =
                                f4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
                    }
                }
                float *ys = yr - a;               // line-aligned segment start
                const float *ss = srow + kLineF - a; // segment in the staging row
#pragma unroll
                for (int c = 0; c < S; ++c) {
                    const int s0 = 64 * c + 4 * j;
                    const f4 val = f4{ss[s0], ss[s0 + 1], ss[s0 + 2], ss[s0 + 3]};
                    if (c > 0 || chain_in) {
                        *reinterpret_cast<f4 *>(ys + s0) = val;
                    } else { // chain start: the segment's first a outputs are not this item's
                        if (s0 >= a) *reinterpret_cast<f4 *>(ys + s0) = val;
                        else {
                            if (s0 + 1 >= a) ys[s0 + 1] = val.y;
                            if (s0 + 2 >= a) ys[s0 + 2] = val.z;
                            if (s0 + 3 >= a) ys[s0 + 3] = val.w;
                        }
                    }
                }
                if (!chain_out) { // chain end: the carry
                    if (j < a) ys[64 * S + j] = ss[64 * S + j];
                    if (j + 16 < a) ys[64 * S + j + 16] = ss[64 * S + j + 16];
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4 * S; ++u) {
                    const int o = o_t + 4 * S * j + u;
                    if (o >= 0 && o < P.L_out) {
                        const float a = ADD ? ar[4 * S * j + u] : 0.0f;
                        yr[4 * S * j + u] = finish<EPI>(v[u], a);
                    }
                }
            }
        }
        }

        __syncthreads();
        ++ii;
        st = st1;
        ng = ng1;
        st1 = st2;
        ng1 = ng2;
        if (ii + 2 < n_items) advance(st2, ng2);
    };
    for (;;) {
        item(pre, pre2, std::integral_constant<int, 0>{});
        if (ii >= n_items) break;
        item(pre2, pre, std::integral_constant<int, 1>{});
        if (ii >= n_items) break;
    }
}

// ------------------------------------------------------------ channels last
// The same phase decomposition for x (N, L_in, C_in) and y (N, L_out, C_out).
// The output of one position is C_out contiguous floats, so an
// output-stationary tile can store whole lines: a wave owns 16 consecutive
// positions q0 .. q0+15 of one (n, g) and all COG output channels (COG/16
// accumulator tiles per phase), with every weight of the group in VGPRs.
// Waves are independent: no barrier.
//
// MFMA D[co][col] = sum_k A[co][k] B[k][col], A = W^T (16 co x 4 ci), B = X
// (4 ci x 16 positions), column j = position q0 + j.  At step kk the lane
// (g4, j) supplies input channel 16*(kk/4) + 4*g4 + kk%4, so for one position
// and one tap shift c it loads its CIG/4 channels as CIG/16 float4s at
// channel offsets 16u + 4g4: one load instruction covers 16 positions x 64
// contiguous bytes.  Positions outside [0, L_in) read zeros through the
// buffer resource's range check (a negative offset wraps past it).  The
// inputs of an item are loaded PF items ahead (CONVT_NLC_PREFETCH), in
// rotating register sets.
//
// The accumulator of lane (g4, j), register e, holds channel 16ct + 4g4 + e at
// position q0 + j.  Stored as they are, one instruction would write half
// lines (64 of each 128 bytes), which costs HBM bandwidth when the lines are
// not in the cache (0.44 against 0.30 ms on the long 1D layer after a cache
// flush).  So each wave stages its item's 16*S outputs x COG channels in its
// own LDS region (row p = output offset in the item, float4 column c4 stored
// at c4 ^ key(p), key(p) = (p/S) mod (COG/4): the accumulator writes, 16 lanes
// j of one g4 on rows S*j + r, and the row reads fall on distinct banks), and
// each store instruction writes 1 KB of whole lines; add_input is read at the
// same contiguous offsets.  One wave's LDS accesses are performed in order,
// so the region needs no barrier.  Outputs outside [0, L_out) are dropped by
// the range check.
template <int CIG, int COG, int K, int S, int D, int EPI>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(CONVT_NLC_WAVES_PER_EU))) void k_stream1d_nlc(const Stream1dParams P,
                                                          const float *__restrict__ x,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ bias,
                                                          const float *add, float *y) {
    using Ph = Phases<K, S, D>;
    constexpr bool ADD = epi_add(EPI);
    constexpr int NKK = CIG / 4;   // MFMA steps per tap
    constexpr int NU = CIG / 16;   // float4 per lane per (position, shift)
    constexpr int COT = COG / 16;  // accumulator tiles
    constexpr int NC = Ph::cmax() + 1;
    constexpr int NP = Ph::count() > 0 ? Ph::count() : 1;
    constexpr int PF = CONVT_NLC_PREFETCH;
    constexpr int C4 = COG / 4;
    constexpr int SROWS = 16 * S;
    constexpr int NST = SROWS * C4 / 64; // stores per lane and item
    static_assert(CIG % 16 == 0 && COG % 16 == 0, "tile shape");
    static_assert(PF == 1 || PF == 2, "prefetch distance");

    const int lane = threadIdx.x & 63;
    const int j = lane & 15;
    const int g4 = lane >> 4;
    // uniform across the wave: the item walk and the buffer resources stay in
    // scalar registers
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t it0 = ((int64_t)blockIdx.x * 4 + wv) * P.per_block;
    const int64_t it_end = it0 + P.per_block < P.total ? it0 + P.per_block : P.total;
    if (it0 >= it_end) return;

    __shared__ __attribute__((aligned(16))) float ostage[4][SROWS * COG];
    float *stg = &ostage[wv][0];

    const unsigned xrow = 4u * (unsigned)P.C_in, yrow = 4u * (unsigned)P.C_out;
    const int x_bytes = 4 * P.L_in * P.C_in, y_bytes = 4 * P.L_out * P.C_out;
    // lane-invariant parts of the load offsets: position j, channel 16u + 4g4
    unsigned xl[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) xl[u] = (unsigned)j * xrow + 4u * (unsigned)(16 * u + 4 * g4);

    // the inputs of item (ng_ = n*G + g, tile st_) into xb: per shift c the
    // uniform offset of position q0 - c and channel g*CIG
    auto fetch = [&](f4 (&xb)[NC][NU], int ng_, int st_) {
        const int n = P.G == 1 ? ng_ : ng_ / P.G, g = ng_ - n * P.G;
        const rsrc_t rx = make_rsrc(const_cast<float *>(x) + (int64_t)n * P.L_in * P.C_in, x_bytes);
        const int q0 = (P.st_lo + st_) * 16;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const unsigned su = (unsigned)(q0 - c) * xrow + 4u * (unsigned)(g * CIG);
#pragma unroll
            for (int u = 0; u < NU; ++u) xb[c][u] = buf_load4(rx, xl[u] + su, 0u);
        }
    };

    float wr[COT][K][NKK]; // A operands: W[g*CIG + ci(kk)][16ct + j][k]
    f4 b4[COT];            // bias of channels 16ct + 4g4 .. +3
    f4 xa[NC][NU], xb[NC][NU], xc[NC][NU];
    // cursors: the current item (it; ng, st) and the last one whose inputs
    // were fetched (pit; png, pst), advanced one tile at a time
    int64_t it = it0;
    int ng = (int)(it0 / P.n_st), st = (int)(it0 - (int64_t)ng * P.n_st);
    int64_t pit = it0;
    int png = ng, pst = st;
    auto advance = [&](int &ng_, int &st_) {
        if (++st_ == P.n_st) { st_ = 0; ++ng_; }
    };
    fetch(xa, png, pst);
    if constexpr (PF == 2) {
        if (pit + 1 < it_end) { ++pit; advance(png, pst); }
        fetch(xb, png, pst);
    }

    // One item with its inputs in cur; the inputs of the item PF ahead (the
    // current one's again past the wave's last item, so that every step
    // issues the same loads and the compiler's wait counts stay exact) go to
    // nxt.
    auto step = [&](const f4 (&cur)[NC][NU], f4 (&nxt)[NC][NU]) {
        const int n = P.G == 1 ? ng : ng / P.G, g = ng - n * P.G;
        if (pit + 1 < it_end) { ++pit; advance(png, pst); }
        fetch(nxt, png, pst);
        // nothing moves across the steps: the scheduler would otherwise pull
        // the next item's MFMAs up to its just-issued loads and wait for them
        __builtin_amdgcn_sched_barrier(0);

        f4 acc[NP][COT];
        if constexpr (Ph::count() > 0) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int c = Ph::c_of(k);
                const int sl = Ph::slot(Ph::r_of(k));
                const bool first = k == Ph::first_k(Ph::r_of(k));
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const float bv = cur[c][kk / 4][kk % 4];
#pragma unroll
                    for (int ct = 0; ct < COT; ++ct)
                        acc[sl][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[ct][k][kk], bv,
                                                                         (first && kk == 0) ? b4[ct] : acc[sl][ct],
                                                                         0, 0, 0);
                }
            }
        }

        // stage: phase r of position q0 + j is item row S*j + r
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
            for (int ct = 0; ct < COT; ++ct) {
                f4 v = b4[ct];
                if constexpr (Ph::count() > 0)
                    if (Ph::nonempty(r)) v = acc[Ph::slot(r)][ct];
                const int c4 = (4 * ct + g4) ^ (j & (C4 - 1));
                *reinterpret_cast<f4 *>(stg + (S * j + r) * COG + 4 * c4) = v;
            }
        // store: float4 f = 64u + lane of the item's outputs is row f / C4,
        // column f % C4; item row p is output o0 + p
        const rsrc_t ry = make_rsrc(y + (int64_t)n * P.L_out * P.C_out, y_bytes);
        const rsrc_t ra = make_rsrc(const_cast<float *>(ADD ? add : y) + (int64_t)n * P.L_out * P.C_out, y_bytes);
        const unsigned so = (unsigned)((P.st_lo + st) * 16 * S - P.p) * yrow + 4u * (unsigned)(g * COG);
#pragma unroll
        for (int u = 0; u < NST; ++u) {
            const int f = 64 * u + lane;
            const int row = f / C4, c4 = f % C4;
            f4 v = *reinterpret_cast<const f4 *>(stg + row * COG + 4 * (c4 ^ ((row / S) & (C4 - 1))));
            const unsigned off = so + (unsigned)row * yrow + 16u * (unsigned)c4;
            if constexpr (ADD) {
                const f4 a = buf_load4(ra, off, 0u);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = finish<EPI>(v[e], a[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = activate<EPI>(v[e]);
            }
            buf_store4(v, ry, off, 0u);
        }
        __builtin_amdgcn_sched_barrier(0);
        ++it;
        advance(ng, st);
    };

    // Runs of consecutive items of one group share the weights: load them
    // once per run, before the loop that carries the prefetch.
    while (it < it_end) {
        const int g = P.G == 1 ? 0 : ng % P.G;
        const int64_t left = P.G == 1 ? it_end - it : min(it_end - it, (int64_t)(P.n_st - st));
#pragma unroll
        for (int ct = 0; ct < COT; ++ct) {
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const int ci = g * CIG + 16 * (kk / 4) + 4 * g4 + kk % 4;
                    wr[ct][k][kk] = w[((int64_t)ci * COG + 16 * ct + j) * K + k];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[ct][e] = bias ? bias[g * COG + 16 * ct + 4 * g4 + e] : 0.0f;
        }
        // wait for these here (an empty asm that reads and redefines them
        // puts the wait before the loop, whose waits then cover only the
        // prefetch)
#pragma unroll
        for (int ct = 0; ct < COT; ++ct) {
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(wr[ct][k][kk]));
            asm volatile("" : "+v"(b4[ct]));
        }
        const int64_t run_end = it + left;
        if constexpr (PF == 1) {
            // two items per trip with the input sets swapped (no copies)
            while (it + 1 < run_end) {
                step(xa, xb);
                step(xb, xa);
            }
            if (it < run_end) { // an odd item: its prefetch lands in xb; move it
                step(xa, xb);
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int u = 0; u < NU; ++u) xa[c][u] = xb[c][u];
            }
        } else {
            // three items per trip, the sets rotating: xa and xb hold the next
            // two items' inputs at every trip start
            while (it + 2 < run_end) {
                step(xa, xc);
                step(xb, xa);
                step(xc, xb);
            }
            // the run's last one or two items; then rotate so that xa and xb
            // again hold the next two items' inputs (once per run)
            if (it < run_end) {
                step(xa, xc);
                if (it < run_end) {
                    step(xb, xa);
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int u = 0; u < NU; ++u) {
                            xb[c][u] = xa[c][u];
                            xa[c][u] = xc[c][u];
                        }
                } else {
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int u = 0; u < NU; ++u) {
                            xa[c][u] = xb[c][u];
                            xb[c][u] = xc[c][u];
                        }
                }
            }
        }
    }
}

// Instantiated shapes: (C_in/g, C_out/g, K, S, D).
struct Variant {
    int cig, cog, K, S, D;
    bool nlc; // also compiled for channels last (the 64-channel groups would spill there)
};
constexpr Variant kVariants[] = {
    {32, 64, 3, 2, 2, true},  // long-sequence layer: N x 32 -> 64, K=3, stride 2, dilation 2
    {32, 64, 3, 2, 1, true},  // stride-2 upsampling, K=3
    {32, 32, 4, 2, 1, true},  // stride-2 upsampling, K=4 (two phases, two taps each)
    {16, 16, 3, 3, 2, true},  // stride 3, dilation 2: three phases, one tap each
    {16, 32, 5, 4, 2, true},  // stride 4 > taps per phase: two empty phases
    {64, 64, 3, 2, 2, false}, // the long-sequence layer's pattern with 64-channel groups
    {32, 32, 3, 2, 2, true},  // ... and with 32 -> 32 channels
    {64, 64, 3, 2, 1, false}, // stride-2 upsampling, K=3, 64-channel groups
};

int find_variant(const convt_plan &P) {
    if (P.ndim != 1) return -1;
    const AxisPlan &A = P.ax[2];
    for (int i = 0; i < (int)(sizeof(kVariants) / sizeof(kVariants[0])); ++i) {
        const Variant &v = kVariants[i];
        if (P.Cig == v.cig && P.Cog == v.cog && A.K == v.K && A.s == v.S && A.d == v.D)
            return P.layout == CONVT_LAYOUT_CHANNELS_LAST && !v.nlc ? -1 : i;
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

template <int CIG, int COG, int K, int S, int D>
int launch_variant(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                   const float *add, int act, float *y, hipStream_t st) {
    const AxisPlan &A = Pl.ax[2];
    Stream1dParams P;
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.G = (int)Pl.G;
    P.L_in = A.L_in;
    P.L_out = A.L_out;
    P.p = A.p;
    // positions q with some output o = q*S + r - p in [0, L_out)
    const int64_t q_lo = A.p / S;
    const int64_t q_hi = ((int64_t)A.L_out - 1 + A.p) / S + 1;
    const int64_t st_lo = q_lo / kTileQ;
    const int64_t st_hi = (q_hi + kTileQ - 1) / kTileQ;
    P.st_lo = (int)st_lo;
    P.n_st = (int)(st_hi - st_lo);
    P.total = Pl.N * Pl.G * P.n_st;
    constexpr int NT = COG * 4;
    with_epi(add != nullptr, act, [&](auto E) {
        constexpr auto kern = k_stream1d<CIG, COG, K, S, D, decltype(E)::value>;
        // one round of resident workgroups (see CONVT_S1D_ROUNDS): CONVT_S1D_WAVES_PER_EU
        // waves on each of the 4 SIMDs, COG/16 waves per workgroup, or fewer where
        // the instantiation's registers or LDS allow fewer (queried once)
        static const int resident = [&] {
            int nb = 0;
            const int want = 4 * CONVT_S1D_WAVES_PER_EU / (COG / 16);
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, NT, 0) != hipSuccess || nb < 1) nb = want;
            return std::min(nb, want);
        }();
        const int64_t blocks_target = (int64_t)num_cus() * CONVT_S1D_ROUNDS * resident;
        int64_t per_block = (P.total + blocks_target - 1) / blocks_target;
        if (per_block < 1) per_block = 1;
        P.per_block = (int)per_block;
        const unsigned grid = (unsigned)((P.total + per_block - 1) / per_block);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, P, x, w, bias, add, y);
    });
    return (int)hipGetLastError();
}

template <int CIG, int COG, int K, int S, int D>
int launch_variant_nlc(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                       const float *add, int act, float *y, hipStream_t st) {
    const AxisPlan &A = Pl.ax[2];
    Stream1dParams P;
    P.C_in = (int)Pl.C_in;
    P.C_out = (int)Pl.C_out;
    P.G = (int)Pl.G;
    P.L_in = A.L_in;
    P.L_out = A.L_out;
    P.p = A.p;
    // positions q with some output o = q*S + r - p in [0, L_out), in tiles of 16
    const int64_t q_lo = A.p / S;
    const int64_t q_hi = ((int64_t)A.L_out - 1 + A.p) / S + 1;
    const int64_t st_lo = q_lo / 16;
    P.st_lo = (int)st_lo;
    P.n_st = (int)((q_hi + 15) / 16 - st_lo);
    P.total = Pl.N * Pl.G * P.n_st;
    // one round of resident waves, each walking a run of consecutive tiles
    const int64_t waves = (int64_t)num_cus() * 4 * CONVT_NLC_WAVES_PER_EU;
    int64_t per_wave = (P.total + waves - 1) / waves;
    if (per_wave < 1) per_wave = 1;
    P.per_block = (int)per_wave;
    const int64_t nw = (P.total + per_wave - 1) / per_wave;
    const unsigned grid = (unsigned)((nw + 3) / 4);
    with_epi(add != nullptr, act, [&](auto E) {
        hipLaunchKernelGGL((k_stream1d_nlc<CIG, COG, K, S, D, decltype(E)::value>), dim3(grid), dim3(256), 0, st,
                           P, x, w, bias, add, y);
    });
    return (int)hipGetLastError();
}

} // namespace

bool stream1d_supports(const convt_plan &P) {
    if (find_variant(P) < 0) return false;
    if (P.layout == CONVT_LAYOUT_CHANNELS_LAST)
        // per-sample x and y below 2 GiB (31-bit buffer offsets); positions
        // and outputs index within int
        return P.ax[2].L_out < (1 << 30) && P.ax[2].L_in < (1 << 30) &&
               4 * P.C_out * P.ax[2].L_out < INT32_MAX && 4 * P.C_in * P.ax[2].L_in < INT32_MAX;
    // 64-position tiles of one row must index within int range; the tile
    // fetch reads whole float4 inside a row
    // (one sample of y and one row set of x below 2 GiB: the common-path
    // stores and the inner-tile loads use 31-bit offsets)
    return P.ax[2].L_out < (1 << 30) && P.ax[2].L_in < (1 << 30) && P.ax[2].L_in >= 4 &&
           4 * P.C_out * P.ax[2].L_out < INT32_MAX && 4 * P.Cig * P.ax[2].L_in < INT32_MAX;
}

int launch_stream1d(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                    const float *add, int act, float *y, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    if (Pl.layout == CONVT_LAYOUT_CHANNELS_LAST) {
        switch (find_variant(Pl)) {
        case 0: return launch_variant_nlc<32, 64, 3, 2, 2>(Pl, x, w, bias, add, act, y, st);
        case 1: return launch_variant_nlc<32, 64, 3, 2, 1>(Pl, x, w, bias, add, act, y, st);
        case 2: return launch_variant_nlc<32, 32, 4, 2, 1>(Pl, x, w, bias, add, act, y, st);
        case 3: return launch_variant_nlc<16, 16, 3, 3, 2>(Pl, x, w, bias, add, act, y, st);
        case 4: return launch_variant_nlc<16, 32, 5, 4, 2>(Pl, x, w, bias, add, act, y, st);
        case 6: return launch_variant_nlc<32, 32, 3, 2, 2>(Pl, x, w, bias, add, act, y, st);
        default: return (int)hipErrorInvalidValue;
        }
    }
    switch (find_variant(Pl)) {
    case 0: return launch_variant<32, 64, 3, 2, 2>(Pl, x, w, bias, add, act, y, st);
    case 1: return launch_variant<32, 64, 3, 2, 1>(Pl, x, w, bias, add, act, y, st);
    case 2: return launch_variant<32, 32, 4, 2, 1>(Pl, x, w, bias, add, act, y, st);
    case 3: return launch_variant<16, 16, 3, 3, 2>(Pl, x, w, bias, add, act, y, st);
    case 4: return launch_variant<16, 32, 5, 4, 2>(Pl, x, w, bias, add, act, y, st);
    case 5: return launch_variant<64, 64, 3, 2, 2>(Pl, x, w, bias, add, act, y, st);
    case 6: return launch_variant<32, 32, 3, 2, 2>(Pl, x, w, bias, add, act, y, st);
    case 7: return launch_variant<64, 64, 3, 2, 1>(Pl, x, w, bias, add, act, y, st);
    default: return (int)hipErrorInvalidValue;
    }
}

} // namespace convt
