// Layer-output error of a quantised layer for gfx950 (H-Scale §3: the layer-output
// reconstruction criterion behind the activation-loss comparison of scale rules):
//   err[o] (+)= sum_t (sum_i x_ti (w_oi - w_hat_oi))^2,   w_hat = sign * level * eff[c].
//
// Three kernels:
//   split:  E = fl(w - w_hat) in binary32 per element (w_hat = fl(q * eff) with q from the exact
//           fp4 up-conversion of the packed nibble, eff = fl(S * dec(c))), written as two bf16
//           matrices E_hi = bf16(E) and E_lo = bf16(E - E_hi) (round to nearest even; E - E_hi is
//           exact), so E_hi + E_lo carries 16 significant bits of E. Both are padded with zeros
//           to whole GEMM tiles.
//   gemm:   Y = X E_hi^T + X E_lo^T on MFMA (v_mfma_f32_32x32x16_bf16, binary32 accumulation).
//           A workgroup of 8 waves owns a 256-token x 256-row tile; each wave a 128 x 64 part
//           as 4 x 2 MFMA tiles of 32 x 32 (16 MFMAs per 8 LDS fragment reads). K advances by
//           32. X and both E tiles go from global memory straight into LDS (LDS-DMA loads, no
//           registers), 16-byte chunks XOR-swizzled per row against bank conflicts, in a ring of
//           3 stages (144 KB, one workgroup per CU): step it + 2 loads while step it computes.
//           The next K slice's fragments are read while the current slice's MFMAs run. Tiles
//           are dealt to the XCDs in groups of 4 x 8 that share K slices in L2. The epilogue
//           squares Y and sums each row over the tile's tokens (fixed order), writing one
//           binary32 partial per (token tile, row).
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

// One thread per 8 consecutive weights of a row (one 16-byte half of a group in bf16). The
// outputs are out_pad x ldE matrices: the padding (rows from `out`, columns from `in`) is
// written as zeros, so the GEMM loads whole tiles without bounds checks.
template <bool BF16>
__global__ __launch_bounds__(256) void k_residual_split(
    const uint8_t* __restrict__ W, int64_t out, int64_t in, int64_t ldw_bytes,
    const uint8_t* __restrict__ scales, const uint8_t* __restrict__ packed,
    const float* __restrict__ S_arr, int64_t out_pad, int64_t ldE, uint16_t* __restrict__ e_hi,
    uint16_t* __restrict__ e_lo) {
    const int64_t units = out_pad * (ldE / 8);
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int64_t o = u / (ldE / 8);
    const int64_t i0 = (u - o * (ldE / 8)) * 8;
    if (o >= out || i0 >= in) {
        *reinterpret_cast<uint4*>(e_hi + o * ldE + i0) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(e_lo + o * ldE + i0) = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
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
    *reinterpret_cast<uint4*>(e_hi + o * ldE + i0) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(e_lo + o * ldE + i0) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ---- gemm + squared-sum epilogue ------------------------------------------------------------

constexpr int BM = 256;      // tokens per tile
constexpr int BN = 256;      // output rows per tile
constexpr int BK = 32;       // reduction step: an LDS row is 64 B = 4 chunks of 16 B
constexpr int kStages = 3;   // LDS ring: step it + 2 loads while step it + 1 waits and it computes
constexpr int kGemmThreads = 512;
constexpr int kXcds = 8;

struct Stage {
    uint16_t a[BM][BK];
    uint16_t bh[BN][BK];
    uint16_t bl[BN][BK];
};
static_assert(kStages * sizeof(Stage) <= 160 * 1024, "the LDS ring exceeds 160 KB");

// 16-byte chunk c of LDS row r sits at chunk position c ^ swz(r). With this XOR pattern the
// MFMA fragment reads (one chunk of 32 consecutive rows per half-wave) touch distinct banks in
// every group of 8 lanes.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Workgroup -> (token tile, row tile). Workgroups are dealt to the 8 XCDs round-robin; when the
// tile count is a multiple of 8, XCD x gets the contiguous tile range [x n/8, (x+1) n/8). Within
// it, tiles come in groups of kGM token tiles x kGN row tiles (32 workgroups, one per CU of the
// XCD) when the tile grid divides evenly, so the workgroups resident on an XCD at one time read
// 4 X tiles and 8 E tiles and advance through K together: each K slice comes into the XCD's L2
// once and is reused there. Otherwise tiles are numbered token-tile-major.
constexpr uint32_t kGM = 4, kGN = 8;

__device__ __forceinline__ void tile_of(uint32_t L, uint32_t ntn, uint32_t ntm, uint32_t nb,
                                        uint32_t& tm, uint32_t& tn) {
    const uint32_t q = (nb % kXcds == 0) ? (L % kXcds) * (nb / kXcds) + L / kXcds : L;
    if (ntn % kGN == 0 && ntm % kGM == 0) {
        const uint32_t g = q / (kGM * kGN), l = q % (kGM * kGN);
        const uint32_t gpr = ntn / kGN;
        tm = (g / gpr) * kGM + l / kGN;
        tn = (g % gpr) * kGN + l % kGN;
    } else {
        tm = q / ntn;
        tn = q - tm * ntn;
    }
}

// waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;   // vmcnt(0)
constexpr int kWaitVm6 = 0x0F76;   // vmcnt(6): one step's six LDS-DMA loads may stay in flight

// One workgroup of 8 waves owns a 256-token x 256-row tile; wave (wm, wn) computes tokens
// wm*128.. and rows wn*64.. as 4 x 2 MFMA tiles of 32 x 32, each fed by E_hi and E_lo.
// E_hi and E_lo are the split kernel's padded copies: ldE columns (a multiple of 32, zero past
// `in`) and rows up to the next multiple of 256 (zero past `out`).
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_output_gemm(
    const uint16_t* __restrict__ X, int64_t T, int64_t in, int64_t ldx,
    const uint16_t* __restrict__ e_hi, const uint16_t* __restrict__ e_lo, int64_t ldE,
    int64_t out, uint32_t ntn, uint32_t ntm, uint32_t nb, float* __restrict__ partial) {
    __shared__ __attribute__((aligned(1024))) Stage st[kStages];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 2, wn = wave & 3;
    uint32_t tm, tn;
    tile_of(blockIdx.x, ntn, ntm, nb, tm, tn);
    const int64_t n0 = (int64_t)tn * BN;
    const int64_t m0 = (int64_t)tm * BM;

    // Staging by LDS DMA (16 bytes per lane, a wave fills 16 consecutive 64-byte LDS rows).
    // The LDS slot of thread chunk id = tid + 512 r is fixed: row id / 4, chunk position id % 4;
    // the lane fetches the logical chunk that the swizzle puts there. Tokens past T read row
    // T - 1 (their products are left out of the sums below); X chunks past `in` read the row's
    // first chunk, which meets the zero padding of E.
    const uint16_t* xp[2];
    const uint16_t* hp[2];
    const uint16_t* lp[2];
    int xk[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int id = tid + kGemmThreads * r, row = id >> 2, lc = (id & 3) ^ swz(row);
        const int64_t t = min(m0 + row, T - 1);
        xp[r] = X + t * ldx;
        xk[r] = lc * 8;
        hp[r] = e_hi + (n0 + row) * ldE + lc * 8;
        lp[r] = e_lo + (n0 + row) * ldE + lc * 8;
    }
    auto dma = [&](Stage& s, int64_t k0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int base = (kGemmThreads * r + 64 * wave) >> 2;   // first LDS row of this wave
            const int64_t k = k0 + xk[r];
            __builtin_amdgcn_global_load_lds(xp[r] + (k < in ? k : 0), &s.a[base][0], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(hp[r] + k0, &s.bh[base][0], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(lp[r] + k0, &s.bl[base][0], 16, 0, 0);
        }
    };

    floatx16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    // MFMA operands of one 16-wide K slice: lane l holds K values (l / 32) * 8 .. + 8 of row
    // l % 32 of each 32-row block
    struct Frag {
        bf16x8 a[4], h[2], l[2];
    };
    const int r32 = lane & 31, kg = (lane >> 5) * 8;
    auto frag = [&](const Stage& s, int kk, Frag& f) {
        const int c = (kk + kg) >> 3;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int row = wm * 128 + t * 32 + r32;
            f.a[t] = *reinterpret_cast<const bf16x8*>(&s.a[row][(c ^ swz(row)) * 8]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = wn * 64 + t * 32 + r32;
            f.h[t] = *reinterpret_cast<const bf16x8*>(&s.bh[row][(c ^ swz(row)) * 8]);
            f.l[t] = *reinterpret_cast<const bf16x8*>(&s.bl[row][(c ^ swz(row)) * 8]);
        }
    };
    auto mfmas = [&](const Frag& f) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[a], f.h[b], acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[a], f.l[b], acc[a][b], 0, 0, 0);
            }
    };

    // Pipeline. Before step it: steps it and it + 1 are loading or loaded, the first K slice of
    // step it is in registers. During step it: read its second slice, multiply the first; wait
    // for step it + 1 and meet at the barrier (after it no wave reads step it - 1's stage any
    // more, so step it + 2 may load into it); read step it + 1's first slice; multiply the
    // second. The barrier is a bare s_barrier: the waits it needs are the explicit ones, and a
    // full __syncthreads would also wait for step it + 2's loads.
    const int64_t nk = (in + BK - 1) / BK;
    if (nk > 0) dma(st[0], 0);
    if (nk > 1) {
        dma(st[1], BK);
        __builtin_amdgcn_s_waitcnt(kWaitVm6);
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    asm volatile("s_barrier" ::: "memory");
    Frag f0, f1;
    frag(st[0], 0, f0);
    int cs = 0;
    for (int64_t it = 0; it < nk; ++it) {
        const int ns = (cs + 1 == kStages) ? 0 : cs + 1;   // stage of step it + 1
        const int ds = (ns + 1 == kStages) ? 0 : ns + 1;   // stage of step it + 2
        frag(st[cs], 16, f1);
        mfmas(f0);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        asm volatile("s_barrier" ::: "memory");
        if (it + 2 < nk) dma(st[ds], (it + 2) * BK);
        frag(st[ns], 0, f0);   // after the last step this reads a stale stage, unused
        mfmas(f1);
        cs = ns;
    }

    // epilogue: a lane holds tokens i = (e/4)*8 + (lane/32)*4 + e%4 of row j = lane%32 of each
    // 32x32 tile; sum the squares over the lane's tokens (those below T) and token tiles, then
    // over the lane pair, then over the two waves of the same rows (fixed order)
    __syncthreads();
    float* red = reinterpret_cast<float*>(&st[0]);   // [2][BN]
    const int64_t tw = m0 + wm * 128 + (lane >> 5) * 4;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        float s = 0.0f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float v = (tw + a * 32 + (e >> 2) * 8 + (e & 3) < T) ? acc[a][b][e] : 0.0f;
                s = __builtin_fmaf(v, v, s);
            }
        s += __shfl_xor(s, 32, 64);
        if (lane < 32) red[wm * BN + wn * 64 + b * 32 + lane] = s;
    }
    __syncthreads();
    if (tid < BN) {
        const int64_t o = n0 + tid;
        if (o < out) partial[(int64_t)tm * out + o] = red[tid] + red[BN + tid];
    }
}

// ---- reduce -------------------------------------------------------------------------------

// One thread per row; the token-tile partials are added in order, 8 loads in flight.
__global__ __launch_bounds__(256) void k_output_reduce(const float* __restrict__ partial,
                                                       int64_t tiles, int64_t out,
                                                       double* __restrict__ err, int accumulate) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= out) return;
    double s = accumulate ? err[o] : 0.0;
    for (int64_t t0 = 0; t0 < tiles; t0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (t0 + k < tiles) ? partial[(t0 + k) * out + o] : 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (t0 + k < tiles) s += (double)v[k];
    }
    err[o] = s;
}

size_t round_up(size_t b) { return (b + 255) / 256 * 256; }

// padded residual matrices: rows to a multiple of BN, columns to a multiple of BK
struct ResidualLayout {
    int64_t out_pad, ldE;
    size_t bytes;   // one matrix, rounded to 256 bytes
};
ResidualLayout residual_layout(int64_t out, int64_t in) {
    ResidualLayout L;
    L.out_pad = (out + BN - 1) / BN * BN;
    L.ldE = (in + BK - 1) / BK * BK;
    L.bytes = round_up((size_t)L.out_pad * (size_t)L.ldE * 2);
    return L;
}

}  // namespace

size_t output_error_workspace_bytes(int64_t tokens, int64_t out, int64_t in) {
    const int64_t tiles = (tokens + BM - 1) / BM;
    return 2 * residual_layout(out, in).bytes + (size_t)tiles * (size_t)out * 4;
}

int64_t output_error_tiles(int64_t tokens, int64_t out) {
    return ((out + BN - 1) / BN) * ((tokens + BM - 1) / BM);
}

hipError_t launch_output_error(const void* X, int64_t tokens, int64_t in, int64_t ldx,
                               const void* W, bool w_bf16, int64_t out, int64_t ldw,
                               const uint8_t* scales, const uint8_t* packed, const float* S,
                               double* err, bool accumulate, void* workspace,
                               hipStream_t stream) {
    const ResidualLayout L = residual_layout(out, in);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* e_hi = reinterpret_cast<uint16_t*>(ws);
    uint16_t* e_lo = reinterpret_cast<uint16_t*>(ws + L.bytes);
    float* partial = reinterpret_cast<float*>(ws + 2 * L.bytes);
    const int64_t tiles = (tokens + BM - 1) / BM;
    const int64_t units = (tiles > 0) ? L.out_pad * (L.ldE / 8) : 0;
    const dim3 sgrid((uint32_t)((units + 255) / 256));
    if (units > 0) {
        if (w_bf16)
            hipLaunchKernelGGL(k_residual_split<true>, sgrid, dim3(256), 0, stream,
                               static_cast<const uint8_t*>(W), out, in, ldw * 2, scales, packed, S,
                               L.out_pad, L.ldE, e_hi, e_lo);
        else
            hipLaunchKernelGGL(k_residual_split<false>, sgrid, dim3(256), 0, stream,
                               static_cast<const uint8_t*>(W), out, in, ldw * 4, scales, packed, S,
                               L.out_pad, L.ldE, e_hi, e_lo);
    }
    if (tiles > 0) {
        const uint32_t ntn = (uint32_t)((out + BN - 1) / BN);
        const uint32_t nb = ntn * (uint32_t)tiles;
        hipLaunchKernelGGL(k_output_gemm, dim3(nb), dim3(kGemmThreads), 0, stream,
                           static_cast<const uint16_t*>(X), tokens, in, ldx, e_hi, e_lo, L.ldE,
                           out, ntn, (uint32_t)tiles, nb, partial);
    }
    hipLaunchKernelGGL(k_output_reduce, dim3((uint32_t)((out + 255) / 256)), dim3(256), 0, stream,
                       partial, tiles, out, err, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace nvfp4
