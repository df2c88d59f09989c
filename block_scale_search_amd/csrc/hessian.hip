// Diagonal second-order weight h_j = sum_t x_tj^2 over calibration activations X [tokens, in]
// ([HS] §3 / App. B: h = diag(X^T X); [SR] §3).
//
// Two kernels, no atomics, fixed combination order:
//   partial:  a 1024-thread workgroup owns one (column strip, 512-row token tile); 16 lanes
//             cover one row of the strip (16 B each: 8 bf16 or 4 f32 columns), so a wave load
//             reads 4 rows and a lane keeps 8 loads in flight; squares are exact in binary64
//             and summed in binary64; the lanes of a column are combined by fixed xor-shuffles
//             and the 16 waves in wave order through LDS; one binary64 partial per column and
//             tile goes to the workspace.
//   finalize: four threads per (segment, column) add interleaved tiles with all their loads in
//             flight, combine in a fixed order, add the running sum h_acc and round once to
//             binary32.
// The kernel boundary makes the partials of every XCD visible to the finalize kernel.
// HBM traffic: X once plus 16 B per column per 512-row tile (0.8% of X for bf16).
#include <hip/hip_runtime.h>

#include "device_formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = kHessWaves;            // 16
constexpr int kThreads = 64 * kWaves;         // 1024
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerLoad = 64 / kLanesPerRow;  // 4
constexpr int kLoads = 8;                     // loads in flight per lane
constexpr int kRowsPerWave = kRowsPerLoad * kLoads;  // 32
static_assert(kWaves * kRowsPerWave == kHessRowsPerTile, "tile geometry");

template <bool BF16>
struct XCols {
    static constexpr int kCols = BF16 ? 8 : 4;              // columns per 16-byte load
    static constexpr int kStrip = kLanesPerRow * kCols;     // columns per workgroup
};

struct TileMap {
    const int64_t* seg_offsets;  // NULL: one segment [0, tokens)
    const int32_t* tile_prefix;  // first tile of each segment (segments + 1 entries)
    int64_t segments;
    int64_t tokens;
};

__host__ __device__ __forceinline__ int64_t tiles_for(int64_t rows) {
    return rows > 0 ? (rows + kHessRowsPerTile - 1) / kHessRowsPerTile : 1;
}

// tile -> segment e, rows [row0, row1), the segment's first tile and tile count.
__device__ __forceinline__ bool map_tile(const TileMap& m, int64_t tile, int64_t& e,
                                         int64_t& row0, int64_t& row1, int64_t& first,
                                         int64_t& count) {
    if (m.seg_offsets == nullptr) {
        count = tiles_for(m.tokens);
        if (tile >= count) return false;
        e = 0;
        first = 0;
        row0 = tile * kHessRowsPerTile;
        row1 = min(row0 + (int64_t)kHessRowsPerTile, m.tokens);
        return true;
    }
    if (tile >= m.tile_prefix[m.segments]) return false;
    int64_t lo = 0, hi = m.segments - 1;  // last segment whose first tile <= tile
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (m.tile_prefix[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    e = lo;
    first = m.tile_prefix[lo];
    count = m.tile_prefix[lo + 1] - first;
    row0 = m.seg_offsets[lo] + (tile - first) * kHessRowsPerTile;
    row1 = min(row0 + (int64_t)kHessRowsPerTile, m.seg_offsets[lo + 1]);
    return true;
}

// Exclusive prefix of per-segment tile counts (every segment gets at least one tile, so an
// empty segment still writes its h).
__global__ __launch_bounds__(256) void k_hess_tile_prefix(const int64_t* __restrict__ seg_offsets,
                                                          int64_t segments,
                                                          int32_t* __restrict__ tile_prefix) {
    __shared__ int64_t part[256];
    const int t = threadIdx.x;
    const int64_t per = (segments + 255) / 256;
    const int64_t e0 = min(segments, t * per), e1 = min(segments, e0 + per);
    int64_t s = 0;
    for (int64_t e = e0; e < e1; ++e) s += tiles_for(seg_offsets[e + 1] - seg_offsets[e]);
    part[t] = s;
    __syncthreads();
    if (t == 0) {
        int64_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int64_t v = part[i];
            part[i] = run;
            run += v;
        }
        tile_prefix[segments] = (int32_t)run;
    }
    __syncthreads();
    int64_t run = part[t];
    for (int64_t e = e0; e < e1; ++e) {
        tile_prefix[e] = (int32_t)run;
        run += tiles_for(seg_offsets[e + 1] - seg_offsets[e]);
    }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_hess_partial(const uint8_t* __restrict__ X,
                                                           int64_t in, int64_t ldx_bytes,
                                                           TileMap map, int64_t n_strips,
                                                           double* __restrict__ partial) {
    constexpr int C = XCols<BF16>::kCols;
    constexpr int SW = XCols<BF16>::kStrip;
    __shared__ double red[kWaves][SW];

    const int64_t strip = blockIdx.x % n_strips;
    const int64_t tile = blockIdx.x / n_strips;
    int64_t e, row0, row1, first, count;
    if (!map_tile(map, tile, e, row0, row1, first, count)) return;  // uniform per workgroup

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & (kLanesPerRow - 1), rs = lane / kLanesPerRow;
    const int64_t col = strip * SW + (int64_t)lr * C;
    const bool active = col < in;

    uint4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const int64_t r = row0 + (int64_t)wave * kRowsPerWave + k * kRowsPerLoad + rs;
        if (active && r < row1)
            v[k] = *reinterpret_cast<const uint4*>(X + r * ldx_bytes + col * (BF16 ? 2 : 4));
        else
            v[k] = make_uint4(0u, 0u, 0u, 0u);
    }
    double acc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) acc[i] = 0.0;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
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
    // the four lanes of a column (row subsets) in a fixed tree, then waves in order
#pragma unroll
    for (int i = 0; i < C; ++i) {
        acc[i] += __shfl_xor(acc[i], 16, 64);
        acc[i] += __shfl_xor(acc[i], 32, 64);
    }
    if (rs == 0) {
#pragma unroll
        for (int i = 0; i < C; ++i) red[wave][lr * C + i] = acc[i];
    }
    __syncthreads();
    if (threadIdx.x < SW) {
        const int64_t c = strip * SW + threadIdx.x;
        double s = red[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) s += red[w][threadIdx.x];
        if (c < in) partial[tile * in + c] = s;
    }
}

// Four threads per column: thread `sub` adds tiles sub, sub + 4, ... (8 loads in flight at a
// time), then the four sums are combined in sub order.
constexpr int kFinThreads = 256;
constexpr int kFinSubs = 4;
constexpr int kFinCols = kFinThreads / kFinSubs;

__global__ __launch_bounds__(kFinThreads) void k_hess_finalize(const double* __restrict__ partial,
                                                               int64_t in, TileMap map,
                                                               double* __restrict__ h_acc,
                                                               float* __restrict__ h,
                                                               int accumulate) {
    __shared__ double red[kFinSubs][kFinCols];
    const int64_t e = blockIdx.y;
    const int cl = threadIdx.x % kFinCols, sub = threadIdx.x / kFinCols;
    const int64_t c = (int64_t)blockIdx.x * kFinCols + cl;
    int64_t first = 0, count = tiles_for(map.tokens);
    if (map.seg_offsets != nullptr) {
        first = map.tile_prefix[e];
        count = map.tile_prefix[e + 1] - first;
    }
    double s = 0.0;
    if (c < in) {
        for (int64_t t0 = sub; t0 < count; t0 += 8 * kFinSubs) {
            double v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int64_t t = t0 + (int64_t)k * kFinSubs;
                v[k] = t < count ? partial[(first + t) * in + c] : 0.0;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) s += v[k];
        }
    }
    red[sub][cl] = s;
    __syncthreads();
    if (sub == 0 && c < in) {
        const double total = ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
        const int64_t idx = e * in + c;
        const double a = (accumulate ? h_acc[idx] : 0.0) + total;
        h_acc[idx] = a;
        if (h) h[idx] = (float)a;
    }
}

constexpr size_t kAlign = 256;

size_t round_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

int64_t strips_for(int64_t in, bool bf16) {
    const int sw = bf16 ? XCols<true>::kStrip : XCols<false>::kStrip;
    return (in + sw - 1) / sw;
}

size_t prefix_bytes(int64_t segments) {
    return segments > 1 ? round_up((size_t)(segments + 1) * sizeof(int32_t)) : 0;
}

}  // namespace

int64_t hessian_max_tiles(int64_t tokens, int64_t segments) {
    const int64_t t = (tokens + kHessRowsPerTile - 1) / kHessRowsPerTile;
    return segments > 1 ? t + segments : (t > 0 ? t : 1);
}

size_t hessian_workspace_bytes(int64_t tokens, int64_t in, int64_t segments) {
    return prefix_bytes(segments) +
           (size_t)hessian_max_tiles(tokens, segments) * (size_t)in * sizeof(double);
}

hipError_t launch_diag_hessian(const void* X, bool bf16, int64_t tokens, int64_t in, int64_t ldx,
                               const int64_t* seg_offsets, int64_t segments, double* h_acc,
                               float* h, bool accumulate, void* workspace, hipStream_t stream) {
    const bool batched = seg_offsets != nullptr;
    const int64_t E = batched ? segments : 1;
    TileMap map{batched ? seg_offsets : nullptr, nullptr, E, tokens};
    // workspace: [tile prefix (batched only) | tile partials]
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (batched) {
        map.tile_prefix = reinterpret_cast<int32_t*>(ws);
        hipLaunchKernelGGL(k_hess_tile_prefix, dim3(1), dim3(256), 0, stream, seg_offsets, E,
                           const_cast<int32_t*>(map.tile_prefix));
    }
    double* partial = reinterpret_cast<double*>(ws + prefix_bytes(E));
    const int64_t n_strips = strips_for(in, bf16);
    const int64_t blocks = n_strips * hessian_max_tiles(tokens, E);
    const int64_t ldx_bytes = ldx * (bf16 ? 2 : 4);
    const uint8_t* Xb = static_cast<const uint8_t*>(X);
    if (bf16)
        hipLaunchKernelGGL(k_hess_partial<true>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                           stream, Xb, in, ldx_bytes, map, n_strips, partial);
    else
        hipLaunchKernelGGL(k_hess_partial<false>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                           stream, Xb, in, ldx_bytes, map, n_strips, partial);
    const dim3 fgrid((uint32_t)((in + kFinCols - 1) / kFinCols), (uint32_t)E);
    hipLaunchKernelGGL(k_hess_finalize, fgrid, dim3(kFinThreads), 0, stream, partial, in, map,
                       h_acc, h, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace nvfp4
