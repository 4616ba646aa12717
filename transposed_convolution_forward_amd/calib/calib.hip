// Calibration kernels for the measurements: what HBM and the fp32 matrix
// cores deliver on this GPU for the access and instruction patterns the
// transposed-convolution kernels use, with no convolution arithmetic.  They are
// measurement infrastructure, kept out of libconvt.so and its C ABI; the bench
// loads this library by itself.
//
//   convt_calib_fill      write n float4 (non-temporal), a write-only stream
//   convt_calib_read      read n float4 and write one float per workgroup
//   convt_calib_copy      read n float4 and write them elsewhere (1:1 streams)
//   convt_calib_mixed     read nx float4 and write ny float4 as two flat
//                         streams, interleaved per work item like the 1D
//                         layer's items (item i reads rx and writes wy float4;
//                         the next item's reads are issued before the current
//                         item's writes)
//   convt_calib_ncl_1d    the long 1D layer's own memory pattern: per work item
//                         (sample n, 64 positions) a C_in-row x tile with its
//                         4-position halo, and for each of the C_out output rows
//                         the 128-byte-aligned segment of 64*S floats at or
//                         before the item's first output; same grid and item
//                         walk as that kernel, values copied from the tile
//   convt_calib_mfma_f32  register-only chains of v_mfma_f32_16x16x4_f32,
//                         8 independent accumulators per wave
// Every call is asynchronous on the given stream and returns the launch status.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

#define CALIB_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kBlock = 256;
constexpr int kNT = 2; // cache policy nt (streaming) on stores

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int nb = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nb, 0x00020000);
}
__device__ __forceinline__ void st4(rsrc_t r, f4 v, unsigned voff, unsigned soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, v), r,
                                           voff, soff, kNT);
}
__device__ __forceinline__ void st4_global(f4 *p, f4 v) { __builtin_nontemporal_store(v, p); }

// Flat streams walked in work items: item i reads x[i*RX, (i+1)*RX) and
// writes y[i*WY, (i+1)*WY) (float4 units), one workgroup per run of
// consecutive items, the next item's reads issued before the current item's
// writes.  RX = 0 is a write-only fill, WY = 0 a read-only pass (the sum is
// stored only if it equals a value the inputs never give, so the loads stay
// live), RX = WY a copy.
template <int RX, int WY>
__global__ __launch_bounds__(kBlock) void k_stream(const f4 *x, f4 *y, int64_t items, int64_t per_block,
                                                   int64_t nx, int64_t ny, float *sink) {
    constexpr int R = RX / kBlock > 0 ? RX / kBlock : 1, W = WY / kBlock;
    static_assert(RX % kBlock == 0 && WY % kBlock == 0, "item shape");
    const int64_t i0 = (int64_t)blockIdx.x * per_block;
    const int64_t i1 = i0 + per_block < items ? i0 + per_block : items;
    if (i0 >= i1) return;
    const int t = threadIdx.x;
    f4 cur[R], nxt[R], acc = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t k = i0 * RX + u * kBlock + t;
        cur[u] = (RX > 0 && k < nx) ? x[k] : f4{1, 1, 1, 1};
    }
    for (int64_t it = i0; it < i1; ++it) {
        if constexpr (RX > 0) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int64_t k = (it + 1) * RX + u * kBlock + t;
                nxt[u] = (it + 1 < i1 && k < nx) ? x[k] : f4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < W; ++u) {
            const int64_t k = it * WY + u * kBlock + t;
            if (k < ny) st4_global(y + k, cur[u % R]);
        }
        if constexpr (RX > 0) {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                if constexpr (WY == 0) acc += cur[u];
                cur[u] = nxt[u];
            }
        }
    }
    if constexpr (WY == 0) {
        const float s = acc.x + acc.y + acc.z + acc.w;
        if (s == 12345.0f) sink[blockIdx.x] = s;
    }
}

template <int RX, int WY>
int launch_stream(const float *x, int64_t nx4, float *y, int64_t ny4, int blocks, float *sink, hipStream_t st) {
    int64_t items = RX > 0 ? (nx4 + RX - 1) / RX : 0;
    const int64_t iy = WY > 0 ? (ny4 + WY - 1) / WY : 0;
    if (iy > items) items = iy;
    if (blocks < 1 || blocks > 8192 || items < 1) return (int)hipErrorInvalidValue;
    const int64_t per_block = (items + blocks - 1) / blocks;
    const unsigned grid = (unsigned)((items + per_block - 1) / per_block);
    hipLaunchKernelGGL((k_stream<RX, WY>), dim3(grid), dim3(kBlock), 0, st, (const f4 *)x, (f4 *)y, items,
                       per_block, nx4, ny4, sink);
    return (int)hipGetLastError();
}

// The 1D layer's pattern (C_in = CI, C_out = CO, 64 positions per item, S
// outputs per position).  Item (n, tile): the CI x (64 + 4) tile at positions
// q0 - 4 .. q0 + 63, clamped into the row; then for each output row the
// 64*S floats from the 128-byte line boundary at or before o_t = q0*S - p.
// Stores go through a buffer resource over all of y, so a segment running
// past y's end is dropped by the hardware range check.
template <int CI, int CO, int S>
__global__ __launch_bounds__(kBlock) void k_ncl_1d(const float *x, float *y, int L_in, int L_out, int p,
                                                   int n_st, int st_lo, int64_t total, int64_t per_block,
                                                   int64_t y_bytes) {
    constexpr int TF4 = CI * 17;                        // tile float4s
    constexpr int R = (TF4 + kBlock - 1) / kBlock;
    constexpr int SEG4 = 16 * S;                        // float4 per row segment (64*S floats)
    constexpr int W = CO * SEG4 / kBlock;
    static_assert(CO * SEG4 % kBlock == 0, "segment tiling");
    const int64_t i0 = (int64_t)blockIdx.x * per_block;
    const int64_t i1 = i0 + per_block < total ? i0 + per_block : total;
    if (i0 >= i1) return;
    const int t = threadIdx.x;
    auto load = [&](f4 (&r)[R], int64_t it) {
        const int64_t ng = it / n_st;
        const int q0 = (st_lo + (int)(it % n_st)) * 64;
        const float *xr = x + ng * CI * (int64_t)L_in;
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int f = min(u * kBlock + t, TF4 - 1);
            const int row = f / 17, c4 = f % 17;
            const int pos = min(max(q0 - 4 + 4 * c4, 0), L_in - 4);
            f4 v;
            __builtin_memcpy(&v, xr + (int64_t)row * L_in + pos, 16);
            r[u] = v;
        }
    };
    const rsrc_t ry = make_rsrc(y, y_bytes);
    f4 cur[R], nxt[R];
    load(cur, i0);
    for (int64_t it = i0; it < i1; ++it) {
        if (it + 1 < i1) load(nxt, it + 1);
        const int64_t n = it / n_st;
        const int q0 = (st_lo + (int)(it % n_st)) * 64;
        const int64_t o_t = (int64_t)q0 * S - p;
#pragma unroll
        for (int u = 0; u < W; ++u) {
            const int f = u * kBlock + t;
            const int row = f / SEG4, c4 = f % SEG4;
            const int64_t e = (n * CO + row) * (int64_t)L_out + o_t; // first output's element index
            const int64_t seg = (e & ~(int64_t)31) + 4 * c4;          // line-aligned segment
            if (seg >= 0 && o_t < L_out) {
                // the whole byte offset in the vector field, which the range
                // check covers (y is below 2 GiB)
                st4(ry, cur[u % R], (unsigned)(4 * seg), 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < R; ++u) cur[u] = nxt[u];
    }
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1))) void k_mfma(int iters, float *out) {
    typedef float v4 __attribute__((ext_vector_type(4)));
    v4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = v4{0, 0, 0, 0};
    float a = 1.0f + 1e-7f * threadIdx.x, b = 1.0f - 1e-7f * threadIdx.x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i].x + acc[i].y + acc[i].z + acc[i].w;
    if (s == 12345.0f) out[blockIdx.x] = s;
}

} // namespace

// Flat streams over `blocks` workgroups (at most 8192), items of 8 float4 per
// thread and direction: a write-only fill of n4 float4, a read-only pass, a
// copy, and the long 1D layer's byte mix (nx4 float4 read and ny4 written in
// items of 512 read and 2048 written, its 32 x 64 input and 64 x 128 output
// floats per item).  sink8192 receives nothing in practice (see k_stream).
CALIB_API int convt_calib_fill(float *y, int64_t n4, int blocks, void *stream) {
    return launch_stream<0, 2048>(nullptr, 0, y, n4, blocks, nullptr, (hipStream_t)stream);
}

CALIB_API int convt_calib_read(const float *x, int64_t n4, int blocks, float *sink8192, void *stream) {
    return launch_stream<2048, 0>(x, n4, nullptr, 0, blocks, sink8192, (hipStream_t)stream);
}

CALIB_API int convt_calib_copy(const float *x, float *y, int64_t n4, int blocks, void *stream) {
    return launch_stream<2048, 2048>(x, n4, y, n4, blocks, nullptr, (hipStream_t)stream);
}

CALIB_API int convt_calib_mixed(const float *x, int64_t nx4, float *y, int64_t ny4, int blocks, void *stream) {
    return launch_stream<512, 2048>(x, nx4, y, ny4, blocks, nullptr, (hipStream_t)stream);
}

// The long 1D layer's pattern: x (N, 32, L_in), y (N, 64, L_out) with S = 2
// outputs per position and padding p; `blocks` workgroups each walking
// consecutive (n, 64-position) items.  Needs L_in >= 4 and y below 2 GiB.
CALIB_API int convt_calib_ncl_1d(const float *x, float *y, int64_t N, int L_in, int L_out, int p, int blocks,
                                 void *stream) {
    const int64_t y_bytes = 4 * N * 64 * (int64_t)L_out;
    if (L_in < 4 || blocks < 1 || y_bytes > 0x7fffffff) return (int)hipErrorInvalidValue;
    const int64_t q_lo = p / 2, q_hi = ((int64_t)L_out - 1 + p) / 2 + 1;
    const int st_lo = (int)(q_lo / 64);
    const int n_st = (int)((q_hi + 63) / 64 - st_lo);
    const int64_t total = N * n_st;
    const int64_t per_block = (total + blocks - 1) / blocks;
    const unsigned grid = (unsigned)((total + per_block - 1) / per_block);
    hipLaunchKernelGGL((k_ncl_1d<32, 64, 2>), dim3(grid), dim3(kBlock), 0, (hipStream_t)stream, x, y, L_in, L_out,
                       p, n_st, st_lo, total, per_block, y_bytes);
    return (int)hipGetLastError();
}

// waves_per_simd waves on each of the cus x 4 SIMDs, iters x 8 MFMAs each;
// returns the launch status.  FLOPs = cus*4*waves_per_simd * iters * 8 * 2048.
CALIB_API int convt_calib_mfma_f32(int cus, int waves_per_simd, int iters, float *out, void *stream) {
    const int waves = cus * 4 * waves_per_simd;
    hipLaunchKernelGGL(k_mfma, dim3(waves / 4), dim3(kBlock), 0, (hipStream_t)stream, iters, out);
    return (int)hipGetLastError();
}
