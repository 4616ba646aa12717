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
__device__ __forceinline__ void store4u(float *p, f4 v) { __builtin_memcpy(p, &v, 16); }

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
};

struct Stream1dParams {
    int C_in, C_out, G;
    int L_in, L_out, p;
    int n_st;      // work items (64-position tiles) per (n, g) row
    int st_lo;     // first tile index (tile t covers q in [64t, 64t+64))
    int per_block; // consecutive work items per workgroup
    int64_t total; // N * G * n_st
};

// The x tile of one work item in LDS: CIG rows (input channels of the group)
// of positions q0-4 .. q0+63, i.e. 17 float4 per row (pitch 68 floats).
constexpr int kRowF4 = (kTileQ + 4) / 4;
constexpr int kPitch = kRowF4 * 4;

template <int CIG, int NT>
__device__ __forceinline__ void tile_fetch(f4 (&r)[(CIG * kRowF4 + NT - 1) / NT], const float *xrow,
                                           int L_in, int q0, int tid) {
    constexpr int NF = CIG * kRowF4;
    constexpr int PER = (NF + NT - 1) / NT;
    const bool interior = (q0 - 4 >= 0) && (q0 + kTileQ <= L_in);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int f = tid + u * NT;
        if (f < NF) {
            const int row = f / kRowF4, c4 = f % kRowF4;
            const float *src = xrow + (int64_t)row * L_in;
            const int pos = q0 - 4 + 4 * c4;
            if (interior) {
                r[u] = load4u(src + pos);
            } else {
                f4 v;
                v.x = (pos + 0 >= 0 && pos + 0 < L_in) ? src[pos + 0] : 0.0f;
                v.y = (pos + 1 >= 0 && pos + 1 < L_in) ? src[pos + 1] : 0.0f;
                v.z = (pos + 2 >= 0 && pos + 2 < L_in) ? src[pos + 2] : 0.0f;
                v.w = (pos + 3 >= 0 && pos + 3 < L_in) ? src[pos + 3] : 0.0f;
                r[u] = v;
            }
        }
    }
}

template <int CIG, int NT>
__device__ __forceinline__ void tile_store_lds(float *lds, const f4 (&r)[(CIG * kRowF4 + NT - 1) / NT],
                                               int tid) {
    constexpr int NF = CIG * kRowF4;
    constexpr int PER = (NF + NT - 1) / NT;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int f = tid + u * NT;
        if (f < NF) {
            const int row = f / kRowF4, c4 = f % kRowF4;
            *reinterpret_cast<f4 *>(lds + row * kPitch + 4 * c4) = r[u];
        }
    }
}

// One workgroup = COG/16 waves; wave w owns output channels 16w .. 16w+15 of
// the group and all 64 positions of the work item; the waves share the x tile
// through LDS, double-buffered: the tile of the next work item is fetched
// from HBM into registers while the current one is contracted.
template <int CIG, int COG, int K, int S, int D, bool FUSED>
__global__ __launch_bounds__(COG * 4) void k_stream1d(const Stream1dParams P,
                                                      const float *__restrict__ x,
                                                      const float *__restrict__ w,
                                                      const float *__restrict__ bias,
                                                      const float *add, float *y) {
    using Ph = Phases<K, S, D>;
    constexpr int NCIG = CIG / 4;
    constexpr int NT = COG * 4; // threads per workgroup
    constexpr int NP = Ph::count() > 0 ? Ph::count() : 1;
    constexpr int PER = (CIG * kRowF4 + NT - 1) / NT;
    static_assert(CIG % 4 == 0 && COG % 16 == 0, "tile shape");
    static_assert(Ph::cmax() <= 4, "input shift beyond the 4-position halo");

    __shared__ __attribute__((aligned(16))) float lds[2][CIG * kPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ct = tid >> 6; // this wave's co-tile
    const int j = lane & 15;
    const int g4 = lane >> 4;
    int64_t it = (int64_t)blockIdx.x * P.per_block;
    const int64_t it_end = it + P.per_block < P.total ? it + P.per_block : P.total;
    if (it >= it_end) return;

    auto item_n_g_q0 = [&](int64_t item, int &n, int &g, int &q0) {
        const int st = (int)(item % P.n_st);
        const int64_t ng = item / P.n_st;
        g = (int)(ng % P.G);
        n = (int)(ng / P.G);
        q0 = (P.st_lo + st) * kTileQ;
    };
    auto xrow_of = [&](int n, int g) {
        return x + ((int64_t)n * P.C_in + (int64_t)g * CIG) * P.L_in;
    };

    f4 pre[PER];
    {
        int n, g, q0;
        item_n_g_q0(it, n, g, q0);
        tile_fetch<CIG, NT>(pre, xrow_of(n, g), P.L_in, q0, tid);
        tile_store_lds<CIG, NT>(lds[0], pre, tid);
    }
    __syncthreads();

    float wr[K][NCIG]; // A operands: W[g*CIG + 4*cig + g4][16*ct + j][k]
    float br[4];       // bias of co = 16*ct + 4*g4 + e
    int cur_g = -1;
    int buf = 0;

    for (; it < it_end; ++it) {
        int n, g, q0;
        item_n_g_q0(it, n, g, q0);
        const bool has_next = it + 1 < it_end;
        if (has_next) {
            int n1, g1, q1;
            item_n_g_q0(it + 1, n1, g1, q1);
            tile_fetch<CIG, NT>(pre, xrow_of(n1, g1), P.L_in, q1, tid);
        }
        if (g != cur_g) {
            cur_g = g;
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int cig = 0; cig < NCIG; ++cig)
                    wr[k][cig] = w[((int64_t)(g * CIG + 4 * cig + g4) * COG + 16 * ct + j) * K + k];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                br[e] = bias ? bias[g * COG + 16 * ct + 4 * g4 + e] : 0.0f;
        }

        f4 acc[NP][4];
#pragma unroll
        for (int s = 0; s < NP; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[s][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

        if constexpr (Ph::count() > 0) {
            const float *tile = lds[buf];
#pragma unroll
            for (int cig = 0; cig < NCIG; ++cig) {
                const float *rowp = tile + (4 * cig + g4) * kPitch + 4 * j;
                const f4 pv = *reinterpret_cast<const f4 *>(rowp);     // q0+4j-4 .. -1
                const f4 cv = *reinterpret_cast<const f4 *>(rowp + 4); // q0+4j .. +3
                const float cur[4] = {cv.x, cv.y, cv.z, cv.w};
                const float prv[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int c = Ph::c_of(k);
                    const int sl = Ph::slot(Ph::r_of(k));
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float bv = (t >= c) ? cur[(t - c) & 3] : prv[(t - c + 4) & 3];
                        acc[sl][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(wr[k][cig], bv,
                                                                          acc[sl][t], 0, 0, 0);
                    }
                }
            }
        }

        // Epilogue: lane owns outputs o0 .. o0 + 4S - 1 of rows co = 16ct + 4g4 + e.
        const int o0 = (q0 + 4 * j) * S - P.p;
        const bool vec = (o0 >= 0) && (o0 + 4 * S <= P.L_out);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int co = g * COG + 16 * ct + 4 * g4 + e;
            const int64_t row = ((int64_t)n * P.C_out + co) * P.L_out;
            float v[4 * S];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < S; ++r) {
                    float a = 0.0f;
                    if constexpr (Ph::count() > 0)
                        if (Ph::nonempty(r)) a = acc[Ph::slot(r)][t][e];
                    v[t * S + r] = a;
                }
            if (vec) {
#pragma unroll
                for (int h = 0; h < S; ++h) {
                    f4 a4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (FUSED) a4 = load4u(add + row + o0 + 4 * h);
                    f4 out;
                    out.x = epilogue<FUSED>(v[4 * h + 0], br[e], a4.x);
                    out.y = epilogue<FUSED>(v[4 * h + 1], br[e], a4.y);
                    out.z = epilogue<FUSED>(v[4 * h + 2], br[e], a4.z);
                    out.w = epilogue<FUSED>(v[4 * h + 3], br[e], a4.w);
                    store4u(y + row + o0 + 4 * h, out);
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4 * S; ++u) {
                    const int o = o0 + u;
                    if (o >= 0 && o < P.L_out) {
                        const float a1 = FUSED ? add[row + o] : 0.0f;
                        y[row + o] = epilogue<FUSED>(v[u], br[e], a1);
                    }
                }
            }
        }

        if (has_next) tile_store_lds<CIG, NT>(lds[buf ^ 1], pre, tid);
        __syncthreads();
        buf ^= 1;
    }
}

// Instantiated shapes: (C_in/g, C_out/g, K, S, D).
struct Variant {
    int cig, cog, K, S, D;
};
constexpr Variant kVariants[] = {
    {32, 64, 3, 2, 2}, // long-sequence layer: N x 32 -> 64, K=3, stride 2, dilation 2
    {32, 64, 3, 2, 1}, // stride-2 upsampling, K=3
    {32, 32, 4, 2, 1}, // stride-2 upsampling, K=4 (two phases, two taps each)
    {16, 16, 3, 3, 2}, // stride 3, dilation 2: three phases, one tap each
    {16, 32, 5, 4, 2}, // stride 4 > taps per phase: two empty phases
};

int find_variant(const convt_plan &P) {
    if (P.ndim != 1) return -1;
    const AxisPlan &A = P.ax[2];
    for (int i = 0; i < (int)(sizeof(kVariants) / sizeof(kVariants[0])); ++i) {
        const Variant &v = kVariants[i];
        if (P.Cig == v.cig && P.Cog == v.cog && A.K == v.K && A.s == v.S && A.d == v.D) return i;
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
                   const float *add, float *y, hipStream_t st) {
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
    // enough workgroups to fill every CU several times over
    const int64_t blocks_target = (int64_t)num_cus() * 6;
    int64_t per_block = (P.total + blocks_target - 1) / blocks_target;
    if (per_block < 1) per_block = 1;
    P.per_block = (int)per_block;
    const unsigned grid = (unsigned)((P.total + per_block - 1) / per_block);
    constexpr int NT = COG * 4;
    if (add)
        hipLaunchKernelGGL((k_stream1d<CIG, COG, K, S, D, true>), dim3(grid), dim3(NT), 0, st, P,
                           x, w, bias, add, y);
    else
        hipLaunchKernelGGL((k_stream1d<CIG, COG, K, S, D, false>), dim3(grid), dim3(NT), 0, st, P,
                           x, w, bias, add, y);
    return (int)hipGetLastError();
}

} // namespace

bool stream1d_supports(const convt_plan &P) {
    if (find_variant(P) < 0) return false;
    // 64-position tiles of one row must index within int range
    return P.ax[2].L_out < (1 << 30) && P.ax[2].L_in < (1 << 30);
}

int launch_stream1d(const convt_plan &Pl, const float *x, const float *w, const float *bias,
                    const float *add, float *y, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    switch (find_variant(Pl)) {
    case 0: return launch_variant<32, 64, 3, 2, 2>(Pl, x, w, bias, add, y, st);
    case 1: return launch_variant<32, 64, 3, 2, 1>(Pl, x, w, bias, add, y, st);
    case 2: return launch_variant<32, 32, 4, 2, 1>(Pl, x, w, bias, add, y, st);
    case 3: return launch_variant<16, 16, 3, 3, 2>(Pl, x, w, bias, add, y, st);
    case 4: return launch_variant<16, 32, 5, 4, 2>(Pl, x, w, bias, add, y, st);
    default: return (int)hipErrorInvalidValue;
    }
}

} // namespace convt
