// Global FP32 scale of a weight matrix (or of each matrix of a batch) for gfx950:
// S = amax / 2688 (448 * 6) or S = amax / 1536 (256 * 6), and S = 1 when amax = 0
// (H-Scale §3: the tensor-wide FP32 scale times the per-group E4M3 scale gives the effective
// scale; ScaleSweep §3: the 256 * 6 adjustment of the per-tensor rule).
//
// max |w| is taken on the binary32 bit patterns of non-negative values, which order like
// unsigned integers, so the result is exact and independent of the reduction order.
// Pass 1: about 512 workgroups per launch; each reads one contiguous chunk of the matrix
// (a multiple of 4 KB) with 4 non-temporal 16-byte loads in flight per lane and writes one
// partial maximum. Pass 2: one workgroup per matrix reduces its partials and writes S. The
// kernel boundary makes the partials of every XCD visible to pass 2.
// HBM traffic: W once plus 4 B per workgroup.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 4;
constexpr int kTargetBlocks = 512;          // workgroups per launch, over all matrices
constexpr int64_t kMinChunk = kThreads * kLoads;  // vectors per workgroup at least

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ uint32_t absmax_bits(const uint4 d) {
    if constexpr (BF16) {
        const uint32_t x[4] = {d.x & 0x7FFF7FFFu, d.y & 0x7FFF7FFFu, d.z & 0x7FFF7FFFu,
                               d.w & 0x7FFF7FFFu};
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, max(x[i] << 16, x[i] & 0xFFFF0000u));
        return m;
    } else {
        return max(max(d.x & 0x7FFFFFFFu, d.y & 0x7FFFFFFFu),
                   max(d.z & 0x7FFFFFFFu, d.w & 0x7FFFFFFFu));
    }
}

__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* wmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t r = wmax[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, wmax[i]);
    return r;
}

// Workgroup (x, batch) reduces 16-byte vectors [x * chunk, (x + 1) * chunk) of its matrix,
// numbered row-major over the `in` columns (vpr vectors per row).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_amax_partial(const uint8_t* __restrict__ W,
                                                           int64_t out, int64_t vpr,
                                                           int64_t ldw_bytes,
                                                           int64_t stride_w_bytes, int64_t chunk,
                                                           uint32_t* __restrict__ partial) {
    __shared__ uint32_t wmax[kThreads / 64];
    const int64_t batch = blockIdx.y;
    const uint8_t* base = W + batch * stride_w_bytes;
    const bool dense = ldw_bytes == vpr * 16;
    const int64_t nvec = out * vpr;
    const int64_t v_begin = (int64_t)blockIdx.x * chunk;
    const int64_t v_end = min(nvec, v_begin + chunk);
    uint32_t m = 0u;
    for (int64_t v0 = v_begin + threadIdx.x; v0 < v_end; v0 += kLoads * kThreads) {
        uint4 d[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int64_t v = v0 + k * kThreads;
            d[k] = make_uint4(0u, 0u, 0u, 0u);
            if (v < v_end) {
                const int64_t off = dense ? v * 16 : (v / vpr) * ldw_bytes + (v % vpr) * 16;
                const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
                d[k] = make_uint4(t.x, t.y, t.z, t.w);
            }
        }
#pragma unroll
        for (int k = 0; k < kLoads; ++k) m = max(m, absmax_bits<BF16>(d[k]));
    }
    m = block_max(m, wmax);
    if (threadIdx.x == 0) partial[batch * gridDim.x + blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void k_global_scale_finalize(
    const uint32_t* __restrict__ partial, int64_t nblk, int rule, float* __restrict__ S) {
    __shared__ uint32_t wmax[kThreads / 64];
    const int64_t batch = blockIdx.x;
    uint32_t r = 0u;
    for (int64_t i = threadIdx.x; i < nblk; i += kThreads) r = max(r, partial[batch * nblk + i]);
    r = block_max(r, wmax);
    if (threadIdx.x == 0) {
        const float amax = __uint_as_float(r);
        S[batch] = amax > 0.0f ? __fdiv_rn(amax, rule == 0 ? 2688.0f : 1536.0f) : 1.0f;
    }
}

// Workgroups per matrix: about kTargetBlocks over the batch, each with at least kMinChunk
// vectors (counted for f32, the element type with more vectors, so one workspace size serves
// both types).
int64_t amax_blocks(int64_t batch, int64_t out, int64_t in) {
    const int64_t vec = out * (in / 4);
    const int64_t by_size = (vec + kMinChunk - 1) / kMinChunk;
    const int64_t by_batch = (kTargetBlocks + batch - 1) / batch;
    const int64_t n = by_size < by_batch ? by_size : by_batch;
    return n < 1 ? 1 : n;
}

}  // namespace

size_t global_scale_workspace_bytes(int64_t batch, int64_t out, int64_t in) {
    return (size_t)batch * (size_t)amax_blocks(batch, out, in) * sizeof(uint32_t);
}

int64_t amax_partial_count(int64_t batch, int64_t out, int64_t in) {
    return amax_blocks(batch, out, in);
}

hipError_t launch_amax_partial(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, uint32_t* partial,
                               hipStream_t stream) {
    const int64_t nblk = amax_blocks(batch, out, in);
    const int esz = bf16 ? 2 : 4;
    const int64_t vpr = in / (bf16 ? 8 : 4);
    // chunk: whole 4 KB wave-rows of vectors, so every workgroup starts on a 4 KB boundary of a
    // dense matrix
    int64_t chunk = (out * vpr + nblk - 1) / nblk;
    chunk = (chunk + kThreads - 1) / kThreads * kThreads;
    const dim3 grid((uint32_t)nblk, (uint32_t)batch);
    if (bf16)
        hipLaunchKernelGGL(k_amax_partial<true>, grid, dim3(kThreads), 0, stream,
                           static_cast<const uint8_t*>(W), out, vpr, ldw * esz, stride_w * esz,
                           chunk, partial);
    else
        hipLaunchKernelGGL(k_amax_partial<false>, grid, dim3(kThreads), 0, stream,
                           static_cast<const uint8_t*>(W), out, vpr, ldw * esz, stride_w * esz,
                           chunk, partial);
    return hipGetLastError();
}

hipError_t launch_global_scale(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, int rule, float* S, void* workspace,
                               hipStream_t stream) {
    const int64_t nblk = amax_blocks(batch, out, in);
    uint32_t* partial = static_cast<uint32_t*>(workspace);
    const hipError_t e = launch_amax_partial(W, bf16, batch, out, in, ldw, stride_w, partial, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_global_scale_finalize, dim3((uint32_t)batch), dim3(kThreads), 0, stream,
                       partial, nblk, rule, S);
    return hipGetLastError();
}

}  // namespace nvfp4
