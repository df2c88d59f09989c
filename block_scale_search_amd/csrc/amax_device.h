// Device-side pieces of the global-scale reduction for gfx950, shared by the global-scale
// kernels and the fused layer-statistics kernels: max |w| on binary32 bit patterns (exact and
// independent of the reduction order) and the scale rule S = amax / 2688 or amax / 1536, 1 for
// amax = 0 (H-Scale §3: tensor-wide FP32 scale; ScaleSweep Methodology §2: the 256 * 6
// adjustment).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kAmaxLoads = 4;   // 16-byte loads in flight per lane

typedef unsigned int amax_u32x4 __attribute__((ext_vector_type(4)));

// Largest |value| of a 16-byte vector as a binary32 bit pattern (non-negative values order like
// unsigned integers).
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

// Maximum over a workgroup of THREADS threads; wmax holds THREADS / 64 words of LDS.
template <int THREADS>
__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t* wmax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t r = wmax[0];
#pragma unroll
    for (int i = 1; i < THREADS / 64; ++i) r = max(r, wmax[i]);
    return r;
}

// One workgroup's partial maximum: 16-byte vectors [blk * chunk, (blk + 1) * chunk) of a matrix,
// numbered row-major over its columns (vpr vectors per row, rows ldw_bytes apart), read with
// kAmaxLoads non-temporal loads in flight per lane. Thread 0 returns the result.
template <bool BF16, int THREADS>
__device__ __forceinline__ uint32_t amax_chunk(const uint8_t* __restrict__ base, int64_t out,
                                               int64_t vpr, int64_t ldw_bytes, int64_t chunk,
                                               int64_t blk, uint32_t* wmax) {
    const bool dense = ldw_bytes == vpr * 16;
    const int64_t nvec = out * vpr;
    const int64_t v_begin = blk * chunk;
    const int64_t v_end = min(nvec, v_begin + chunk);
    uint32_t m = 0u;
    for (int64_t v0 = v_begin + threadIdx.x; v0 < v_end; v0 += kAmaxLoads * THREADS) {
        uint4 d[kAmaxLoads];
#pragma unroll
        for (int k = 0; k < kAmaxLoads; ++k) {
            const int64_t v = v0 + k * THREADS;
            d[k] = make_uint4(0u, 0u, 0u, 0u);
            if (v < v_end) {
                const int64_t off = dense ? v * 16 : (v / vpr) * ldw_bytes + (v % vpr) * 16;
                const amax_u32x4 t =
                    __builtin_nontemporal_load(reinterpret_cast<const amax_u32x4*>(base + off));
                d[k] = make_uint4(t.x, t.y, t.z, t.w);
            }
        }
#pragma unroll
        for (int k = 0; k < kAmaxLoads; ++k) m = max(m, absmax_bits<BF16>(d[k]));
    }
    return block_max<THREADS>(m, wmax);
}

// S from the partial maxima of one matrix (any number of partials, THREADS threads).
template <int THREADS>
__device__ __forceinline__ float scale_from_amax_partials(const uint32_t* __restrict__ partial,
                                                          int64_t n, int rule, uint32_t* wmax) {
    uint32_t r = 0u;
    for (int64_t i = threadIdx.x; i < n; i += THREADS) r = max(r, partial[i]);
    r = block_max<THREADS>(r, wmax);
    const float amax = __uint_as_float(r);
    return amax > 0.0f ? __fdiv_rn(amax, rule == 0 ? 2688.0f : 1536.0f) : 1.0f;
}

}  // namespace nvfp4
