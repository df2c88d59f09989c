// Diagonal second-order weight h_j = sum_t x_tj^2 over calibration activations X [tokens, in]
// ([HS] §3 / App. B: h = diag(X^T X); [SR] §3).
//
// Two passes, no atomics, fixed combination order:
//   partial: a 1024-thread workgroup owns one (column strip, token tile). Each lane loads 16 B
//            of a row (8 bf16 or 4 f32 columns), squares them exactly in binary64 and keeps
//            binary64 sums; the 16 waves take interleaved rows of the 128-row tile; the wave
//            sums are combined through LDS in wave order and written as one binary64 partial
//            per column and tile.
//   finalize: one thread per (segment, column) adds the tiles of its segment in tile order to
//            the running sum h_acc and rounds once to binary32.
// HBM traffic: X once (2 or 4 B per element) plus 8 B per column per 128-row tile, written
// and read back once (~3% of X for bf16).
#include <hip/hip_runtime.h>

#include "device_formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 64 * kHessWaves;
constexpr int kRowsPerWave = kHessRowsPerTile / kHessWaves;  // 8

template <bool BF16>
struct XTraits;
template <>
struct XTraits<true> {
    static constexpr int kCols = 8;  // columns per 16-byte load
};
template <>
struct XTraits<false> {
    static constexpr int kCols = 4;
};

// Token tile -> rows [row0, row1) and segment. Single segment: tiles cover [0, tokens).
// Batched: tile_prefix[e] = first tile of segment e (computed by k_hess_tile_prefix).
struct TileMap {
    const int64_t* seg_offsets;  // NULL for one segment
    const int32_t* tile_prefix;
    int64_t segments;
    int64_t tokens;
};

__device__ __forceinline__ bool map_tile(const TileMap& m, int64_t tile, int64_t& row0,
                                         int64_t& row1) {
    if (m.seg_offsets == nullptr) {
        row0 = tile * kHessRowsPerTile;
        row1 = min(row0 + (int64_t)kHessRowsPerTile, m.tokens);
        return row0 < m.tokens;
    }
    if (tile >= m.tile_prefix[m.segments]) return false;
    int64_t lo = 0, hi = m.segments - 1;  // largest e with tile_prefix[e] <= tile
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (m.tile_prefix[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    const int64_t local = tile - m.tile_prefix[lo];
    row0 = m.seg_offsets[lo] + local * kHessRowsPerTile;
    row1 = min(row0 + (int64_t)kHessRowsPerTile, m.seg_offsets[lo + 1]);
    return row0 < row1;
}

__global__ void k_hess_tile_prefix(const int64_t* __restrict__ seg_offsets, int64_t segments,
                                   int32_t* __restrict__ tile_prefix) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int64_t acc = 0;
    for (int64_t e = 0; e < segments; ++e) {
        tile_prefix[e] = (int32_t)acc;
        const int64_t n = seg_offsets[e + 1] - seg_offsets[e];
        acc += n > 0 ? (n + kHessRowsPerTile - 1) / kHessRowsPerTile : 0;
    }
    tile_prefix[segments] = (int32_t)acc;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_hess_partial(const uint8_t* __restrict__ X,
                                                           int64_t in, int64_t ldx_bytes,
                                                           TileMap map, int64_t n_col_tiles,
                                                           double* __restrict__ partial) {
    constexpr int C = XTraits<BF16>::kCols;
    constexpr int kStrip = 64 * C;
    __shared__ double red[kHessWaves][kStrip];

    const int64_t col_tile = blockIdx.x % n_col_tiles;
    const int64_t tile = blockIdx.x / n_col_tiles;
    int64_t row0, row1;
    if (!map_tile(map, tile, row0, row1)) return;  // uniform per workgroup

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t col = col_tile * kStrip + (int64_t)lane * C;
    const bool active = col < in;

    double acc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) acc[i] = 0.0;

    uint4 v[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int64_t r = row0 + wave + (int64_t)k * kHessWaves;
        if (active && r < row1)
            v[k] = *reinterpret_cast<const uint4*>(X + r * ldx_bytes + col * (BF16 ? 2 : 4));
        else
            v[k] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        const uint32_t d[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        if constexpr (BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double lo = (double)bf16_lo(d[i]), hi = (double)bf16_hi(d[i]);
                acc[2 * i] = __builtin_fma(lo, lo, acc[2 * i]);
                acc[2 * i + 1] = __builtin_fma(hi, hi, acc[2 * i + 1]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double x = (double)__uint_as_float(d[i]);
                acc[i] = __builtin_fma(x, x, acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < C; ++i) red[wave][lane * C + i] = acc[i];
    __syncthreads();
    for (int t = threadIdx.x; t < kStrip; t += kThreads) {
        const int64_t c = col_tile * kStrip + t;
        if (c < in) {
            double s = red[0][t];
#pragma unroll
            for (int w = 1; w < kHessWaves; ++w) s += red[w][t];
            partial[tile * in + c] = s;
        }
    }
}

__global__ void k_hess_finalize(const double* __restrict__ partial, int64_t in, TileMap map,
                                int64_t n_tiles_single, double* __restrict__ h_acc,
                                float* __restrict__ h, int accumulate) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= map.segments * in) return;
    const int64_t e = idx / in, j = idx - e * in;
    int64_t t0 = 0, t1 = n_tiles_single;
    if (map.seg_offsets != nullptr) {
        t0 = map.tile_prefix[e];
        t1 = map.tile_prefix[e + 1];
    }
    double acc = accumulate ? h_acc[idx] : 0.0;
    for (int64_t t = t0; t < t1; ++t) acc += partial[t * in + j];
    h_acc[idx] = acc;
    if (h) h[idx] = (float)acc;
}

constexpr size_t kPrefixBytesAlign = 256;

size_t prefix_bytes(int64_t segments) {
    if (segments <= 1) return 0;
    const size_t b = (size_t)(segments + 1) * sizeof(int32_t);
    return (b + kPrefixBytesAlign - 1) / kPrefixBytesAlign * kPrefixBytesAlign;
}

}  // namespace

int64_t hessian_max_tiles(int64_t tokens, int64_t segments) {
    const int64_t t = (tokens + kHessRowsPerTile - 1) / kHessRowsPerTile;
    return segments > 1 ? t + segments : t;
}

size_t hessian_workspace_bytes(int64_t tokens, int64_t in, int64_t segments) {
    return prefix_bytes(segments) +
           (size_t)hessian_max_tiles(tokens, segments) * (size_t)in * sizeof(double);
}

hipError_t launch_diag_hessian(const void* X, bool bf16, int64_t tokens, int64_t in, int64_t ldx,
                               const int64_t* seg_offsets, int64_t segments, double* h_acc,
                               float* h, bool accumulate, void* workspace, hipStream_t stream) {
    const bool batched = seg_offsets != nullptr;
    TileMap map{batched ? seg_offsets : nullptr, nullptr, batched ? segments : 1, tokens};
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (batched) {
        map.tile_prefix = reinterpret_cast<int32_t*>(ws);
        hipLaunchKernelGGL(k_hess_tile_prefix, dim3(1), dim3(64), 0, stream, seg_offsets, segments,
                           const_cast<int32_t*>(map.tile_prefix));
    }
    double* partial = reinterpret_cast<double*>(ws + prefix_bytes(batched ? segments : 1));
    const int64_t max_tiles = hessian_max_tiles(tokens, batched ? segments : 1);
    const int cols = bf16 ? 8 : 4;
    const int64_t n_col_tiles = (in + 64 * cols - 1) / (64 * cols);
    if (max_tiles > 0 && n_col_tiles > 0) {
        const int64_t blocks = n_col_tiles * max_tiles;
        const int64_t ldx_bytes = ldx * (bf16 ? 2 : 4);
        if (bf16)
            hipLaunchKernelGGL(k_hess_partial<true>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                               stream, static_cast<const uint8_t*>(X), in, ldx_bytes, map,
                               n_col_tiles, partial);
        else
            hipLaunchKernelGGL(k_hess_partial<false>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                               stream, static_cast<const uint8_t*>(X), in, ldx_bytes, map,
                               n_col_tiles, partial);
    }
    const int64_t n = map.segments * in;
    if (n > 0) {
        const int threads = 256;
        hipLaunchKernelGGL(k_hess_finalize, dim3((uint32_t)((n + threads - 1) / threads)),
                           dim3(threads), 0, stream, partial, in, map, max_tiles, h_acc, h,
                           accumulate ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
