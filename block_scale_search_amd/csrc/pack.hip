// Quantize + pack at given scale bytes for gfx950 (H-Scale App. B: the group is quantized once
// with its chosen scale; round-to-nearest E2M1 at a fixed effective scale).
//
// A wave covers 64 consecutive groups as 16-byte units of W (8 bf16 or 4 f32 elements; U = 2
// or 4 units per group). Lane l converts units l, l + 64, ... of its wave, so every load
// instruction of a wave reads 1 KB of W and every store writes 256 B (bf16) or 128 B (f32) of
// codes, each contiguous when the rows are. The reciprocals r[c] of the matrix's effective
// scales sit in an LDS table. W is read once, with non-temporal loads. HBM traffic: W once,
// 1 B of scale per group, 8 B of codes per group.
#include <hip/hip_runtime.h>

#include "device_formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint8_t* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_pack(
    const uint8_t* __restrict__ W, uint32_t out, uint32_t in, uint64_t gpr_magic,
    uint32_t gpr_shift, int64_t ldw_bytes, int64_t stride_w_bytes,
    const uint8_t* __restrict__ scales, const float* __restrict__ S_arr,
    uint8_t* __restrict__ packed) {
    constexpr int U = BF16 ? 2 : 4;       // 16-byte units per group
    __shared__ float rtab[256];
    const int64_t batch = blockIdx.y;
    const uint32_t gpr = in >> 4;
    const uint32_t G = out * gpr;
    const uint32_t wave_g0 = blockIdx.x * kThreads + (threadIdx.x & ~63u);  // 64 groups per wave
    const int lane = threadIdx.x & 63;

    // issue every load first; the reciprocal table is built while they are in flight
    uint4 a[U];
    int c[U];
    int64_t gidx[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int u = lane + 64 * k;
        const uint32_t gi = wave_g0 + u / U;
        gidx[k] = batch * (int64_t)G + gi;
        a[k] = make_uint4(0u, 0u, 0u, 0u);
        c[k] = 0;
        if (gi < G) {
            const uint32_t row = div_gpr(gi, gpr_magic, gpr_shift);
            const uint32_t g = gi - row * gpr;
            a[k] = load_stream(W + batch * stride_w_bytes + (int64_t)row * ldw_bytes +
                               (int64_t)g * (BF16 ? 32 : 64) + (u % U) * 16);
            c[k] = scales[gidx[k]];
        }
    }
    // r[c] = 1 / (S * dec(c)) for every byte value; bytes outside 1..126 quantize with r = 0,
    // which gives signed zero codes
    static_assert(kThreads == 256, "one table entry per thread");
    {
        const int t = threadIdx.x;
        rtab[t] = (t >= 1 && t <= 126) ? __fdiv_rn(1.0f, S_arr[batch] * e4m3_value(t)) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int u = lane + 64 * k;
        if (wave_g0 + u / U >= G) continue;
        const uint32_t d[4] = {a[k].x, a[k].y, a[k].z, a[k].w};
        const float r = rtab[c[k]];
        uint32_t word = 0u;
        if constexpr (BF16) {
            float w[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[2 * i] = bf16_lo(d[i]);
                w[2 * i + 1] = bf16_hi(d[i]);
            }
            word = e2m1_pack2<0>(word, w[0] * r, w[1] * r);
            word = e2m1_pack2<1>(word, w[2] * r, w[3] * r);
            word = e2m1_pack2<2>(word, w[4] * r, w[5] * r);
            word = e2m1_pack2<3>(word, w[6] * r, w[7] * r);
            reinterpret_cast<uint32_t*>(packed)[gidx[k] * 2 + u % U] = word;
        } else {
            float w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = __uint_as_float(d[i]);
            word = e2m1_pack2<0>(word, w[0] * r, w[1] * r);
            word = e2m1_pack2<1>(word, w[2] * r, w[3] * r);
            reinterpret_cast<uint16_t*>(packed)[gidx[k] * 4 + u % U] = (uint16_t)word;
        }
    }
}

}  // namespace

hipError_t launch_pack(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                       int64_t ldw, int64_t stride_w, const uint8_t* scales, const float* S,
                       uint8_t* packed, hipStream_t stream) {
    const int64_t G = out * (in / 16);
    uint64_t magic;
    uint32_t shift;
    gpr_divisor(in / 16, magic, shift);
    const dim3 grid((uint32_t)((G + kThreads - 1) / kThreads), (uint32_t)batch);
    const int esz = bf16 ? 2 : 4;
    const uint8_t* Wb = static_cast<const uint8_t*>(W);
    uint8_t* P = packed;
    if (bf16)
        hipLaunchKernelGGL(k_pack<true>, grid, dim3(kThreads), 0, stream, Wb, (uint32_t)out,
                           (uint32_t)in, magic, shift, ldw * esz, stride_w * esz, scales, S, P);
    else
        hipLaunchKernelGGL(k_pack<false>, grid, dim3(kThreads), 0, stream, Wb, (uint32_t)out,
                           (uint32_t)in, magic, shift, ldw * esz, stride_w * esz, scales, S, P);
    return hipGetLastError();
}

}  // namespace nvfp4
