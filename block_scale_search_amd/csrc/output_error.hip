// Layer-output error of a quantised layer for gfx950 (H-Scale §3: the layer-output
// reconstruction criterion behind the activation-loss comparison of scale rules):
//   err[o] (+)= sum_t (sum_i x_ti (w_oi - w_hat_oi))^2,   w_hat = sign * level * eff[c].
//
// Three kernels:
//   split:  E = fl(w - w_hat) in binary32 per element (w_hat = fl(q * eff) with q from the exact
//           fp4 up-conversion of the packed nibble, eff = fl(S * dec(c))), written as two bf16
//           matrices E_hi = bf16(E) and E_lo = bf16(E - E_hi) (round to nearest even; E - E_hi is
//           exact), so E_hi + E_lo carries 16 significant bits of E.
//   gemm:   Y = X E_hi^T + X E_lo^T on MFMA (v_mfma_f32_32x32x16_bf16, binary32 accumulation).
//           A workgroup of 4 waves owns a 128-token x 128-row tile; each wave a 64 x 64 quarter
//           as 2 x 2 MFMA tiles of 32 x 32. K advances by 32: X and both E tiles are staged
//           through LDS (double-buffered, rows padded to 80 B), the next stage's global loads in
//           flight during the current stage's MFMAs. The epilogue squares Y and sums each
//           column over the tile's 128 tokens (fixed order), writing one binary32 partial per
//           (token tile, row).
//   reduce: one thread per row adds the token-tile partials in order in binary64 (and the
//           running err when accumulating over token chunks).
// No atomics: the result is deterministic.
#include <hip/hip_runtime.h>

#include "device_formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// ---- split --------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// One thread per 8 consecutive weights of a row (one 16-byte half of a group in bf16).
template <bool BF16>
__global__ __launch_bounds__(256) void k_residual_split(
    const uint8_t* __restrict__ W, int64_t out, int64_t in, int64_t ldw_bytes,
    const uint8_t* __restrict__ scales, const uint8_t* __restrict__ packed,
    const float* __restrict__ S_arr, uint16_t* __restrict__ e_hi, uint16_t* __restrict__ e_lo) {
    const int64_t units = out * (in / 8);
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int64_t o = u / (in / 8);
    const int64_t i0 = (u - o * (in / 8)) * 8;
    float w[8];
    if constexpr (BF16) {
        const uint4 a = *reinterpret_cast<const uint4*>(W + o * ldw_bytes + i0 * 2);
        const uint32_t d[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[2 * k] = bf16_lo(d[k]);
            w[2 * k + 1] = bf16_hi(d[k]);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(W + o * ldw_bytes + i0 * 4);
        const float4 b = *reinterpret_cast<const float4*>(W + o * ldw_bytes + i0 * 4 + 16);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
    const int c = scales[o * (in / 16) + i0 / 16];
    const float eff = (c >= 1 && c <= 126) ? S_arr[0] * e4m3_value(c) : 0.0f;
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(packed + o * (in / 2) + i0 / 2);
    float q[8];
    {
        const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
        const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
        const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
        const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
        q[0] = v0[0]; q[1] = v0[1]; q[2] = v1[0]; q[3] = v1[1];
        q[4] = v2[0]; q[5] = v2[1]; q[6] = v3[0]; q[7] = v3[1];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t h2[2], l2[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int j = 2 * k + m;
            const float what = q[j] * eff;
            const float e = w[j] - what;
            const uint32_t hb = bf16_rne_bits(e);
            const float ehi = __uint_as_float(hb << 16);
            h2[m] = hb;
            l2[m] = bf16_rne_bits(e - ehi);
        }
        hi[k] = h2[0] | (h2[1] << 16);
        lo[k] = l2[0] | (l2[1] << 16);
    }
    *reinterpret_cast<uint4*>(e_hi + o * in + i0) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(e_lo + o * in + i0) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ---- gemm + squared-sum epilogue ------------------------------------------------------------

constexpr int BM = 128;      // tokens per tile
constexpr int BN = 128;      // output rows per tile
constexpr int BK = 32;       // reduction step
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements): 80 B

struct Stage {
    uint16_t a[BM][LDK];
    uint16_t bh[BN][LDK];
    uint16_t bl[BN][LDK];
};

__global__ __launch_bounds__(256) void k_output_gemm(
    const uint16_t* __restrict__ X, int64_t T, int64_t in, int64_t ldx,
    const uint16_t* __restrict__ e_hi, const uint16_t* __restrict__ e_lo, int64_t out,
    float* __restrict__ partial) {
    __shared__ Stage st[2];
    __shared__ float red[2][BN];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * BN;   // output-row tile
    const int64_t m0 = (int64_t)blockIdx.y * BM;   // token tile

    // global -> register staging: 512 16-byte chunks per matrix tile, 2 per thread
    uint4 ra[2], rh[2], rl[2];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int id = tid + 256 * r;
            const int row = id >> 2, ch = id & 3;
            const int64_t k = k0 + ch * 8;
            const bool kin = k < in;
            const int64_t t = m0 + row, o = n0 + row;
            ra[r] = (kin && t < T) ? *reinterpret_cast<const uint4*>(X + t * ldx + k)
                                   : make_uint4(0u, 0u, 0u, 0u);
            rh[r] = (kin && o < out) ? *reinterpret_cast<const uint4*>(e_hi + o * in + k)
                                     : make_uint4(0u, 0u, 0u, 0u);
            rl[r] = (kin && o < out) ? *reinterpret_cast<const uint4*>(e_lo + o * in + k)
                                     : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store = [&](Stage& s) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int id = tid + 256 * r;
            const int row = id >> 2, ch = id & 3;
            *reinterpret_cast<uint4*>(&s.a[row][ch * 8]) = ra[r];
            *reinterpret_cast<uint4*>(&s.bh[row][ch * 8]) = rh[r];
            *reinterpret_cast<uint4*>(&s.bl[row][ch * 8]) = rl[r];
        }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    const int64_t nk = (in + BK - 1) / BK;
    load(0);
    store(st[0]);
    __syncthreads();
    const int r32 = lane & 31, kg = (lane >> 5) * 8;
    for (int64_t it = 0; it < nk; ++it) {
        const int cur = (int)(it & 1);
        if (it + 1 < nk) load((it + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 fa[2], fh[2], fl[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                fa[t] = *reinterpret_cast<const bf16x8*>(&st[cur].a[wm * 64 + t * 32 + r32][kk + kg]);
                fh[t] = *reinterpret_cast<const bf16x8*>(&st[cur].bh[wn * 64 + t * 32 + r32][kk + kg]);
                fl[t] = *reinterpret_cast<const bf16x8*>(&st[cur].bl[wn * 64 + t * 32 + r32][kk + kg]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fh[b], acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fl[b], acc[a][b], 0, 0, 0);
                }
        }
        if (it + 1 < nk) store(st[cur ^ 1]);
        __syncthreads();
    }

    // epilogue: lane holds rows i = (e/4)*8 + (lane/32)*4 + e%4 of column j = lane%32 of each
    // 32x32 tile; sum the squares over the lane's rows and tiles, then over the lane pair.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        float s = 0.0f;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 16; ++e) s = __builtin_fmaf(acc[a][b][e], acc[a][b][e], s);
        s += __shfl_xor(s, 32, 64);
        if (lane < 32) red[wm][wn * 64 + b * 32 + lane] = s;
    }
    __syncthreads();
    if (tid < BN) {
        const int64_t o = n0 + tid;
        if (o < out) partial[(int64_t)blockIdx.y * out + o] = red[0][tid] + red[1][tid];
    }
}

// ---- reduce -------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_output_reduce(const float* __restrict__ partial,
                                                       int64_t tiles, int64_t out,
                                                       double* __restrict__ err, int accumulate) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= out) return;
    double s = accumulate ? err[o] : 0.0;
    for (int64_t t = 0; t < tiles; ++t) s += (double)partial[t * out + o];
    err[o] = s;
}

size_t round_up(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t output_error_workspace_bytes(int64_t tokens, int64_t out, int64_t in) {
    const int64_t tiles = (tokens + BM - 1) / BM;
    return 2 * round_up((size_t)out * (size_t)in * 2) + (size_t)tiles * (size_t)out * 4;
}

hipError_t launch_output_error(const void* X, int64_t tokens, int64_t in, int64_t ldx,
                               const void* W, bool w_bf16, int64_t out, int64_t ldw,
                               const uint8_t* scales, const uint8_t* packed, const float* S,
                               double* err, bool accumulate, void* workspace,
                               hipStream_t stream) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* e_hi = reinterpret_cast<uint16_t*>(ws);
    uint16_t* e_lo = reinterpret_cast<uint16_t*>(ws + round_up((size_t)out * (size_t)in * 2));
    float* partial = reinterpret_cast<float*>(ws + 2 * round_up((size_t)out * (size_t)in * 2));
    const int64_t tiles = (tokens + BM - 1) / BM;
    const int64_t units = (tiles > 0) ? out * (in / 8) : 0;
    const dim3 sgrid((uint32_t)((units + 255) / 256));
    if (units > 0) {
        if (w_bf16)
            hipLaunchKernelGGL(k_residual_split<true>, sgrid, dim3(256), 0, stream,
                               static_cast<const uint8_t*>(W), out, in, ldw * 2, scales, packed, S,
                               e_hi, e_lo);
        else
            hipLaunchKernelGGL(k_residual_split<false>, sgrid, dim3(256), 0, stream,
                               static_cast<const uint8_t*>(W), out, in, ldw * 4, scales, packed, S,
                               e_hi, e_lo);
    }
    if (tiles > 0) {
        const dim3 ggrid((uint32_t)((out + BN - 1) / BN), (uint32_t)tiles);
        hipLaunchKernelGGL(k_output_gemm, ggrid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(X), tokens, in, ldx, e_hi, e_lo, out,
                           partial);
    }
    hipLaunchKernelGGL(k_output_reduce, dim3((uint32_t)((out + 255) / 256)), dim3(256), 0, stream,
                       partial, tiles, out, err, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace nvfp4
