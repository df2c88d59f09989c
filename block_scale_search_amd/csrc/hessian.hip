// Diagonal second-order weight h_j = sum_t x_tj^2 over calibration activations X [tokens, in]
// ([HS] §3 / App. B: h = diag(X^T X); [SR] §3).
//
// Two kernels, no atomics, fixed combination order:
//   partial:  a workgroup of V waves (V = 8 for X below 256 MiB, else 4) owns one (column
//             strip, row group). A lane reads 16 B of a row (8 bf16 or 4 f32 columns), so a
//             wave reads one contiguous 1 KB row segment and the V waves read V consecutive
//             rows. The row groups of a segment take its V-row blocks round-robin (group g:
//             blocks g, g + RG, g + 2 RG, ...), so at any time the whole grid streams one band
//             of full rows; each lane keeps 4 non-temporal loads in flight (X is read once).
//             Squares are exact in binary64 and summed in binary64; the waves are combined in
//             wave order through LDS into one binary64 partial per column and row group. About
//             512 workgroups are launched in all (2 per CU).
//   finalize: eight threads per (segment, column) add interleaved row-group partials with 8
//             loads in flight each, combine in a fixed order, add the running sum h_acc and
//             round once to binary32.
// Deferred mode (one segment): a sequence of token chunks may run the partial pass only, each
// adding its row-group sums into the workspace slots, and one finalize at the end. The slots
// of a row group hold binary64 sums of disjoint token sets, so the final sum over slots is the
// sum over all chunks.
// The kernel boundary makes the partials of every XCD visible to the finalize kernel.
// HBM traffic: X once plus 16 B per column per row group (partial written and read back).
// Layer statistics (one matrix, one chunk): the same two passes with the global scale's amax
// pass (amax_device.h) as a second workgroup role of the partial launch and the S computation
// as one more workgroup of the finalize launch.
#include <hip/hip_runtime.h>

#include "amax_device.h"
#include "device_formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kLoads = 4;              // loads in flight per lane
constexpr int kTargetGroups = 512;     // workgroups per launch (all strips)
constexpr int64_t kWideBytes = (int64_t)256 << 20;  // X from this size up: 4-wave workgroups

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (streamed once, not kept in the caches).
__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

template <bool BF16>
struct XCols {
    static constexpr int kCols = BF16 ? 8 : 4;          // columns per 16-byte load
    static constexpr int kStrip = 64 * kCols;           // columns per workgroup (1 KB per row)
};

// Row groups: segment e has groups [group_prefix[e], group_prefix[e+1]); one segment without
// an offsets array has groups [0, single_groups). The kernels only need the group count: the
// groups of a segment take its V-row blocks round-robin, which works for any count >= 1.
struct GroupMap {
    const int64_t* seg_offsets;  // NULL: one segment [0, tokens)
    const int32_t* group_prefix;
    int64_t segments;
    int64_t tokens;
    int64_t rows_per_group;      // several segments: rows per group of every segment
    int64_t single_groups;       // one segment: its group count
};

// Token chunks of one set at separate addresses (one partial launch over all of them).
struct ChunkTable {
    const uint8_t* x[kMaxHessianChunks];
    int64_t tokens[kMaxHessianChunks];
    int32_t blk_prefix[kMaxHessianChunks + 1];   // first workgroup of each chunk
    int32_t slot_prefix[kMaxHessianChunks + 1];  // first workspace slot of each chunk
    int32_t n;
};

__host__ __device__ __forceinline__ int64_t groups_for(int64_t rows, int64_t rows_per_group) {
    return rows > 0 ? (rows + rows_per_group - 1) / rows_per_group : 0;
}

// global group index -> segment e, its rows [row0, row1), group g within it and group count.
__device__ __forceinline__ bool map_group(const GroupMap& m, int64_t grp, int64_t& e,
                                          int64_t& row0, int64_t& row1, int64_t& g,
                                          int64_t& count) {
    if (m.seg_offsets == nullptr) {
        count = m.single_groups;
        if (grp >= count) return false;
        e = 0;
        g = grp;
        row0 = 0;
        row1 = m.tokens;
        return true;
    }
    if (grp >= m.group_prefix[m.segments]) return false;
    int64_t lo = 0, hi = m.segments - 1;  // last segment whose first group <= grp
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (m.group_prefix[mid] <= grp) lo = mid;
        else hi = mid - 1;
    }
    e = lo;
    g = grp - m.group_prefix[lo];
    count = m.group_prefix[lo + 1] - m.group_prefix[lo];
    row0 = m.seg_offsets[lo];
    row1 = m.seg_offsets[lo + 1];
    return g < count;
}

// Exclusive prefix of per-segment row-group counts.
__global__ __launch_bounds__(256) void k_hess_group_prefix(const int64_t* __restrict__ seg_offsets,
                                                           int64_t segments, int64_t rows_per_group,
                                                           int32_t* __restrict__ group_prefix) {
    __shared__ int64_t part[256];
    const int t = threadIdx.x;
    const int64_t per = (segments + 255) / 256;
    const int64_t e0 = min(segments, t * per), e1 = min(segments, e0 + per);
    int64_t s = 0;
    for (int64_t e = e0; e < e1; ++e)
        s += groups_for(seg_offsets[e + 1] - seg_offsets[e], rows_per_group);
    part[t] = s;
    __syncthreads();
    if (t == 0) {
        int64_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int64_t v = part[i];
            part[i] = run;
            run += v;
        }
        group_prefix[segments] = (int32_t)run;
    }
    __syncthreads();
    int64_t run = part[t];
    for (int64_t e = e0; e < e1; ++e) {
        group_prefix[e] = (int32_t)run;
        run += groups_for(seg_offsets[e + 1] - seg_offsets[e], rows_per_group);
    }
}

// add != 0: the partial is added to the slot's previous value (deferred accumulation over
// token chunks) instead of replacing it.
template <bool BF16, int V>
__device__ __forceinline__ void hess_partial_body(const uint8_t* __restrict__ X, int64_t in,
                                                  int64_t ldx_bytes, const GroupMap& map,
                                                  int64_t n_strips, double* __restrict__ partial,
                                                  int add, int64_t blk,
                                                  double (*red)[XCols<BF16>::kStrip]) {
    constexpr int C = XCols<BF16>::kCols;
    constexpr int SW = XCols<BF16>::kStrip;

    const int64_t strip = blk % n_strips;
    const int64_t grp = blk / n_strips;
    int64_t e, row0, row1, g, count;
    if (!map_group(map, grp, e, row0, row1, g, count)) return;  // uniform per workgroup

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t col = strip * SW + (int64_t)lane * C;
    const bool active = col < in;
    const uint8_t* base = X + col * (BF16 ? 2 : 4);
    const int64_t blocks = (row1 - row0 + V - 1) / V;  // V-row blocks

    double acc[C];
#pragma unroll
    for (int i = 0; i < C; ++i) acc[i] = 0.0;
    for (int64_t j0 = g; j0 < blocks; j0 += count * kLoads) {
        uint4 v[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int64_t j = j0 + (int64_t)k * count;
            const int64_t r = row0 + j * V + wave;
            if (active && j < blocks && r < row1)
                v[k] = load_stream(base + r * ldx_bytes);
            else
                v[k] = make_uint4(0u, 0u, 0u, 0u);
        }
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
    }
#pragma unroll
    for (int i = 0; i < C; ++i) red[wave][lane * C + i] = acc[i];
    __syncthreads();
    for (int t = threadIdx.x; t < SW; t += 64 * V) {
        const int64_t c = strip * SW + t;
        double s = red[0][t];
#pragma unroll
        for (int q = 1; q < V; ++q) s += red[q][t];
        if (c < in) partial[grp * in + c] = add ? partial[grp * in + c] + s : s;
    }
}

template <bool BF16, int V>
__global__ __launch_bounds__(64 * V) void k_hess_partial(const uint8_t* __restrict__ X,
                                                         int64_t in, int64_t ldx_bytes,
                                                         GroupMap map, int64_t n_strips,
                                                         double* __restrict__ partial, int add) {
    __shared__ double red[V][XCols<BF16>::kStrip];
    hess_partial_body<BF16, V>(X, in, ldx_bytes, map, n_strips, partial, add, blockIdx.x, red);
}

// Eight threads per column: thread `sub` adds row groups sub, sub + 8, ... (8 loads in flight
// at a time, so up to 64 groups arrive in one round), then the eight sums are combined in sub
// order.
constexpr int kFinThreads = 256;
constexpr int kFinSubs = 8;
constexpr int kFinCols = kFinThreads / kFinSubs;

__device__ __forceinline__ void hess_finalize_body(const double* __restrict__ partial, int64_t in,
                                                   const GroupMap& map, double* __restrict__ h_acc,
                                                   float* __restrict__ h, int accumulate,
                                                   int64_t blk, int64_t e,
                                                   double (*red)[kFinCols]) {
    const int cl = threadIdx.x % kFinCols, sub = threadIdx.x / kFinCols;
    const int64_t c = blk * kFinCols + cl;
    int64_t first = 0, count = map.single_groups;
    if (map.seg_offsets != nullptr) {
        first = map.group_prefix[e];
        count = map.group_prefix[e + 1] - first;
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
        double total = red[0][cl];
#pragma unroll
        for (int k = 1; k < kFinSubs; ++k) total += red[k][cl];
        const int64_t idx = e * in + c;
        const double a = (accumulate ? h_acc[idx] : 0.0) + total;
        h_acc[idx] = a;
        if (h) h[idx] = (float)a;
    }
}

__global__ __launch_bounds__(kFinThreads) void k_hess_finalize(const double* __restrict__ partial,
                                                               int64_t in, GroupMap map,
                                                               double* __restrict__ h_acc,
                                                               float* __restrict__ h,
                                                               int accumulate) {
    __shared__ double red[kFinSubs][kFinCols];
    hess_finalize_body(partial, in, map, h_acc, h, accumulate, blockIdx.x, blockIdx.y, red);
}

// Several token chunks of one set at separate addresses, in one partial launch: workgroups
// [blk_prefix[c], blk_prefix[c + 1]) run the single-segment partial pass over chunk c into the
// slots [slot_prefix[c], slot_prefix[c + 1]); one finalize then sums every slot.
template <bool BF16, int V>
__global__ __launch_bounds__(64 * V) void k_hess_partial_chunks(ChunkTable ct, int64_t in,
                                                                int64_t ldx_bytes,
                                                                int64_t n_strips,
                                                                double* __restrict__ partial) {
    __shared__ double red[V][XCols<BF16>::kStrip];
    const int32_t blk = (int32_t)blockIdx.x;
    int c = 0;                                   // chunk of this workgroup (uniform)
    while (c + 1 < ct.n && ct.blk_prefix[c + 1] <= blk) ++c;
    const int32_t slot0 = ct.slot_prefix[c];
    GroupMap map{nullptr, nullptr, 1, ct.tokens[c], 0, ct.slot_prefix[c + 1] - slot0};
    hess_partial_body<BF16, V>(ct.x[c], in, ldx_bytes, map, n_strips, partial + (int64_t)slot0 * in,
                               0, blk - ct.blk_prefix[c], red);
}

// Layer statistics, pass 1: the first n_hess workgroups are the h partial pass over X, the rest
// the amax partial pass over W (both streaming, one launch).
template <bool XBF16, int V, bool WBF16>
__global__ __launch_bounds__(64 * V) void k_stats_partial(
    const uint8_t* __restrict__ X, int64_t in, int64_t ldx_bytes, GroupMap map, int64_t n_strips,
    double* __restrict__ partial, int64_t n_hess, const uint8_t* __restrict__ W, int64_t out,
    AmaxPlan ap, int64_t ldw_bytes, uint32_t* __restrict__ amax_partial) {
    __shared__ double red[V][XCols<XBF16>::kStrip];
    if ((int64_t)blockIdx.x < n_hess) {
        hess_partial_body<XBF16, V>(X, in, ldx_bytes, map, n_strips, partial, 0, blockIdx.x, red);
    } else {
        const int64_t blk = blockIdx.x - n_hess;
        const uint32_t m = amax_chunk<WBF16, 64 * V>(W, out, ap.vpr, ldw_bytes, ap.chunk, blk,
                                                     reinterpret_cast<uint32_t*>(&red[0][0]));
        if (threadIdx.x == 0) amax_partial[blk] = m;
    }
}

// Layer statistics, pass 2: the first n_fin workgroups finalize h, the last one computes S.
__global__ __launch_bounds__(kFinThreads) void k_stats_finalize(
    const double* __restrict__ partial, int64_t in, GroupMap map, double* __restrict__ h_acc,
    float* __restrict__ h, int accumulate, int64_t n_fin, const uint32_t* __restrict__ amax_partial,
    int64_t nblk, int rule, float* __restrict__ S) {
    __shared__ double red[kFinSubs][kFinCols];
    if ((int64_t)blockIdx.x < n_fin) {
        hess_finalize_body(partial, in, map, h_acc, h, accumulate, blockIdx.x, 0, red);
    } else {
        const float s = scale_from_amax_partials<kFinThreads>(
            amax_partial, nblk, rule, reinterpret_cast<uint32_t*>(&red[0][0]));
        if (threadIdx.x == 0) S[0] = s;
    }
}

constexpr size_t kAlign = 256;

size_t round_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

int64_t strips_for(int64_t in, bool bf16) {
    const int sw = bf16 ? XCols<true>::kStrip : XCols<false>::kStrip;
    return (in + sw - 1) / sw;
}

// Several segments: rows per row group of every segment, enough groups for about
// kTargetGroups workgroups over all strips and all segments' tokens.
int64_t rows_per_group(int64_t tokens, int64_t in, bool bf16) {
    const int64_t want = (tokens * strips_for(in, bf16) + kTargetGroups - 1) / kTargetGroups;
    const int64_t r = want < 16 ? 16 : want;
    return (r + 7) / 8 * 8;
}

// One segment: one row group per 16 rows, at most enough for about kTargetGroups workgroups
// over all strips. The count never decreases as tokens grow, so in a deferred sequence whose
// first chunk is the longest every later chunk writes only slots the first one initialised,
// and the finalize (given the first chunk's token count) sums every slot that holds data.
int64_t single_groups(int64_t tokens, int64_t in, bool bf16) {
    if (tokens <= 0) return 0;
    const int64_t cap = (kTargetGroups + strips_for(in, bf16) - 1) / strips_for(in, bf16);
    const int64_t g = (tokens + 15) / 16;
    return g < cap ? g : (cap > 0 ? cap : 1);
}

size_t prefix_bytes(int64_t segments) {
    return segments > 1 ? round_up((size_t)(segments + 1) * sizeof(int32_t)) : 0;
}

int64_t max_groups(int64_t tokens, int64_t in, int64_t segments, bool bf16) {
    if (segments <= 1) return single_groups(tokens, in, bf16);
    return groups_for(tokens, rows_per_group(tokens, in, bf16)) + segments;
}

}  // namespace

size_t hessian_workspace_bytes(int64_t tokens, int64_t in, int64_t segments) {
    // sized for the element type with more row groups, so one size serves both
    const int64_t g = max_groups(tokens, in, segments, false) > max_groups(tokens, in, segments, true)
                          ? max_groups(tokens, in, segments, false)
                          : max_groups(tokens, in, segments, true);
    return prefix_bytes(segments) + (size_t)g * (size_t)in * sizeof(double);
}

int64_t hessian_launch_blocks(int64_t tokens, int64_t in, int64_t segments, bool bf16) {
    return strips_for(in, bf16) * max_groups(tokens, in, segments, bf16);
}

hipError_t launch_diag_hessian(const void* X, bool bf16, int64_t tokens, int64_t in, int64_t ldx,
                               const int64_t* seg_offsets, int64_t segments, double* h_acc,
                               float* h, bool accumulate, void* workspace, hipStream_t stream,
                               HessianPass pass) {
    const bool batched = seg_offsets != nullptr;
    const int64_t E = batched ? segments : 1;
    GroupMap map{batched ? seg_offsets : nullptr, nullptr, E, tokens,
                 rows_per_group(tokens, in, bf16), single_groups(tokens, in, bf16)};
    // workspace: [group prefix (batched only) | row-group partials]
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (batched) {
        map.group_prefix = reinterpret_cast<int32_t*>(ws);
        hipLaunchKernelGGL(k_hess_group_prefix, dim3(1), dim3(256), 0, stream, seg_offsets, E,
                           map.rows_per_group, const_cast<int32_t*>(map.group_prefix));
    }
    double* partial = reinterpret_cast<double*>(ws + prefix_bytes(E));
    const int64_t n_strips = strips_for(in, bf16);
    const int64_t blocks = n_strips * max_groups(tokens, in, E, bf16);
    const int64_t ldx_bytes = ldx * (bf16 ? 2 : 4);
    const uint8_t* Xb = static_cast<const uint8_t*>(X);
    // measured on MI355X: 8-wave workgroups stream small X faster, 4-wave ones large X
    const bool wide = tokens * in * (bf16 ? 2 : 4) >= kWideBytes;
    const int add = (pass == HessianPass::kPartial && accumulate) ? 1 : 0;
    if (blocks > 0 && pass != HessianPass::kFinalize) {
        const dim3 grid((uint32_t)blocks);
        if (bf16 && wide)
            hipLaunchKernelGGL((k_hess_partial<true, 4>), grid, dim3(256), 0, stream, Xb, in,
                               ldx_bytes, map, n_strips, partial, add);
        else if (bf16)
            hipLaunchKernelGGL((k_hess_partial<true, 8>), grid, dim3(512), 0, stream, Xb, in,
                               ldx_bytes, map, n_strips, partial, add);
        else if (wide)
            hipLaunchKernelGGL((k_hess_partial<false, 4>), grid, dim3(256), 0, stream, Xb, in,
                               ldx_bytes, map, n_strips, partial, add);
        else
            hipLaunchKernelGGL((k_hess_partial<false, 8>), grid, dim3(512), 0, stream, Xb, in,
                               ldx_bytes, map, n_strips, partial, add);
    }
    if (pass == HessianPass::kPartial) return hipGetLastError();
    const dim3 fgrid((uint32_t)((in + kFinCols - 1) / kFinCols), (uint32_t)E);
    hipLaunchKernelGGL(k_hess_finalize, fgrid, dim3(kFinThreads), 0, stream, partial, in, map,
                       h_acc, h, accumulate ? 1 : 0);
    return hipGetLastError();
}

// Chunks: rows per group chosen over the whole set (about kTargetGroups workgroups in all, as
// for the segments of a batch), each chunk with ceil(tokens / rows_per_group) groups.
static bool plan_chunks(const int64_t* tokens, int64_t n_chunks, int64_t in, bool bf16,
                        ChunkTable* ct, int64_t* slots, int64_t* blocks) {
    int64_t total = 0;
    for (int64_t c = 0; c < n_chunks; ++c) total += tokens[c];
    const int64_t rpg = rows_per_group(total, in, bf16);
    const int64_t strips = strips_for(in, bf16);
    int64_t s = 0;
    for (int64_t c = 0; c < n_chunks; ++c) {
        if (ct) {
            ct->slot_prefix[c] = (int32_t)s;
            ct->blk_prefix[c] = (int32_t)(s * strips);
            ct->tokens[c] = tokens[c];
        }
        s += groups_for(tokens[c], rpg);
        if (s * strips >= ((int64_t)1 << 31)) return false;
    }
    if (ct) {
        ct->slot_prefix[n_chunks] = (int32_t)s;
        ct->blk_prefix[n_chunks] = (int32_t)(s * strips);
        ct->n = (int32_t)n_chunks;
    }
    *slots = s;
    *blocks = s * strips;
    return true;
}

size_t hessian_chunks_workspace_bytes(const int64_t* tokens, int64_t n_chunks, int64_t in) {
    // sized for the element type with more row groups, so one size serves both
    int64_t s32 = 0, s16 = 0, b = 0;
    if (!plan_chunks(tokens, n_chunks, in, false, nullptr, &s32, &b) ||
        !plan_chunks(tokens, n_chunks, in, true, nullptr, &s16, &b))
        return 0;
    return (size_t)(s32 > s16 ? s32 : s16) * (size_t)in * sizeof(double);
}

int64_t hessian_chunks_launch_blocks(const int64_t* tokens, int64_t n_chunks, int64_t in,
                                     bool bf16) {
    int64_t s = 0, b = 0;
    if (!plan_chunks(tokens, n_chunks, in, bf16, nullptr, &s, &b)) return (int64_t)1 << 31;
    return b;
}

hipError_t launch_diag_hessian_chunks(const void* const* X_chunks, bool bf16,
                                      const int64_t* tokens, int64_t n_chunks, int64_t in,
                                      int64_t ldx, double* h_acc, float* h, bool accumulate,
                                      void* workspace, hipStream_t stream) {
    ChunkTable ct{};
    int64_t slots = 0, blocks = 0;
    if (!plan_chunks(tokens, n_chunks, in, bf16, &ct, &slots, &blocks)) return hipErrorInvalidValue;
    for (int64_t c = 0; c < n_chunks; ++c) ct.x[c] = static_cast<const uint8_t*>(X_chunks[c]);
    double* partial = static_cast<double*>(workspace);
    const int64_t n_strips = strips_for(in, bf16);
    const int64_t ldx_bytes = ldx * (bf16 ? 2 : 4);
    int64_t total = 0;
    for (int64_t c = 0; c < n_chunks; ++c) total += tokens[c];
    const bool wide = total * in * (bf16 ? 2 : 4) >= kWideBytes;
    if (blocks > 0) {
        const dim3 grid((uint32_t)blocks);
        if (bf16 && wide)
            hipLaunchKernelGGL((k_hess_partial_chunks<true, 4>), grid, dim3(256), 0, stream, ct,
                               in, ldx_bytes, n_strips, partial);
        else if (bf16)
            hipLaunchKernelGGL((k_hess_partial_chunks<true, 8>), grid, dim3(512), 0, stream, ct,
                               in, ldx_bytes, n_strips, partial);
        else if (wide)
            hipLaunchKernelGGL((k_hess_partial_chunks<false, 4>), grid, dim3(256), 0, stream, ct,
                               in, ldx_bytes, n_strips, partial);
        else
            hipLaunchKernelGGL((k_hess_partial_chunks<false, 8>), grid, dim3(512), 0, stream, ct,
                               in, ldx_bytes, n_strips, partial);
    }
    const GroupMap map{nullptr, nullptr, 1, total, 0, slots};
    const dim3 fgrid((uint32_t)((in + kFinCols - 1) / kFinCols), 1u);
    hipLaunchKernelGGL(k_hess_finalize, fgrid, dim3(kFinThreads), 0, stream, partial, in, map,
                       h_acc, h, accumulate ? 1 : 0);
    return hipGetLastError();
}

size_t layer_statistics_workspace_bytes(int64_t tokens, int64_t in, int64_t out) {
    return round_up(hessian_workspace_bytes(tokens, in, 1)) +
           (size_t)amax_plan(1, out, in, false).nblk * sizeof(uint32_t);
}

hipError_t launch_layer_statistics(const void* X, bool x_bf16, int64_t tokens, int64_t in,
                                   int64_t ldx, double* h_acc, float* h, bool accumulate,
                                   const void* W, bool w_bf16, int64_t out, int64_t ldw, int rule,
                                   float* S, void* workspace, hipStream_t stream) {
    GroupMap map{nullptr, nullptr, 1, tokens, rows_per_group(tokens, in, x_bf16),
                 single_groups(tokens, in, x_bf16)};
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    double* partial = reinterpret_cast<double*>(ws);
    uint32_t* amax_partial =
        reinterpret_cast<uint32_t*>(ws + round_up(hessian_workspace_bytes(tokens, in, 1)));
    const AmaxPlan ap = amax_plan(1, out, in, w_bf16);
    const int64_t n_strips = strips_for(in, x_bf16);
    const int64_t n_hess = n_strips * max_groups(tokens, in, 1, x_bf16);
    const int64_t ldx_bytes = ldx * (x_bf16 ? 2 : 4), ldw_bytes = ldw * (w_bf16 ? 2 : 4);
    const uint8_t* Xb = static_cast<const uint8_t*>(X);
    const uint8_t* Wb = static_cast<const uint8_t*>(W);
    // the workgroup shape follows the h pass (the larger of the two streams)
    const bool wide = tokens * in * (x_bf16 ? 2 : 4) >= kWideBytes;
    const dim3 grid((uint32_t)(n_hess + ap.nblk));
#define NVFP4_STATS(XB, V, WB)                                                                  \
    hipLaunchKernelGGL((k_stats_partial<XB, V, WB>), grid, dim3(64 * V), 0, stream, Xb, in,     \
                       ldx_bytes, map, n_strips, partial, n_hess, Wb, out, ap, ldw_bytes,       \
                       amax_partial)
    if (x_bf16 && wide) {
        if (w_bf16) NVFP4_STATS(true, 4, true); else NVFP4_STATS(true, 4, false);
    } else if (x_bf16) {
        if (w_bf16) NVFP4_STATS(true, 8, true); else NVFP4_STATS(true, 8, false);
    } else if (wide) {
        if (w_bf16) NVFP4_STATS(false, 4, true); else NVFP4_STATS(false, 4, false);
    } else {
        if (w_bf16) NVFP4_STATS(false, 8, true); else NVFP4_STATS(false, 8, false);
    }
#undef NVFP4_STATS
    const int64_t n_fin = (in + kFinCols - 1) / kFinCols;
    hipLaunchKernelGGL(k_stats_finalize, dim3((uint32_t)(n_fin + 1)), dim3(kFinThreads), 0, stream,
                       partial, in, map, h_acc, h, accumulate ? 1 : 0, n_fin, amax_partial,
                       ap.nblk, rule, S);
    return hipGetLastError();
}

}  // namespace nvfp4
