// Global FP32 scale of a weight matrix (or of each matrix of a batch) for gfx950:
// S = amax / 2688 (448 * 6) or S = amax / 1536 (256 * 6), and S = 1 when amax = 0
// (H-Scale §3: the tensor-wide FP32 scale times the per-group E4M3 scale gives the effective
// scale; ScaleSweep Methodology §2: the 256 * 6 adjustment of the per-tensor rule).
//
// max |w| is taken on the binary32 bit patterns of non-negative values, which order like
// unsigned integers, so the result is exact and independent of the reduction order.
// Pass 1: about 512 workgroups per launch; each reads one contiguous chunk of the matrix
// (a multiple of 4 KB) with 4 non-temporal 16-byte loads in flight per lane and writes one
// partial maximum. Pass 2: one workgroup per matrix reduces its partials and writes S. The
// kernel boundary makes the partials of every XCD visible to pass 2.
// HBM traffic: W once plus 4 B per workgroup.
#include <hip/hip_runtime.h>

#include "amax_device.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kTargetBlocks = 512;          // workgroups per launch, over all matrices
constexpr int64_t kMinChunk = kThreads * kAmaxLoads;  // vectors per workgroup at least

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
    const uint32_t m = amax_chunk<BF16, kThreads>(W + batch * stride_w_bytes, out, vpr, ldw_bytes,
                                                  chunk, blockIdx.x, wmax);
    if (threadIdx.x == 0) partial[batch * gridDim.x + blockIdx.x] = m;
}

__global__ __launch_bounds__(kThreads) void k_global_scale_finalize(
    const uint32_t* __restrict__ partial, int64_t nblk, int rule, float* __restrict__ S) {
    __shared__ uint32_t wmax[kThreads / 64];
    const int64_t batch = blockIdx.x;
    const float s = scale_from_amax_partials<kThreads>(partial + batch * nblk, nblk, rule, wmax);
    if (threadIdx.x == 0) S[batch] = s;
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

AmaxPlan amax_plan(int64_t batch, int64_t out, int64_t in, bool bf16) {
    AmaxPlan p;
    p.nblk = amax_blocks(batch, out, in);
    p.vpr = in / (bf16 ? 8 : 4);
    // chunk: whole 4 KB runs of 256 vectors, so every workgroup starts on a 4 KB boundary of a
    // dense matrix
    const int64_t chunk = (out * p.vpr + p.nblk - 1) / p.nblk;
    p.chunk = (chunk + 255) / 256 * 256;
    return p;
}

hipError_t launch_amax_partial(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, uint32_t* partial,
                               hipStream_t stream) {
    const AmaxPlan p = amax_plan(batch, out, in, bf16);
    const int64_t nblk = p.nblk, vpr = p.vpr, chunk = p.chunk;
    const int esz = bf16 ? 2 : 4;
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
