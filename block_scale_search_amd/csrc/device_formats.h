// Device-side element formats for gfx950: bf16 unpacking, E4M3 codes, E2M1 rounding.
//
// E2M1 rounding uses the CDNA4 conversion pair v_cvt_scalef32_pk_fp4_f32 /
// v_cvt_scalef32_pk_f32_fp4. On gfx950 the down-conversion rounds to nearest, ties to the even
// code, saturates at +-6 and keeps the sign of zero; its scale operand contributes only its
// exponent, dividing exactly by that power of two before rounding. The up-conversion is exact.
// Both facts were checked on an MI355X against a comparison-ladder rounding over every finite
// binary32 input (scale 1 and scale 2), and the library's parity tests recheck them end to end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Value of E4M3 code c in 1..126 (sign 0, 4 exponent bits with bias 7, 3 mantissa bits), exact:
// codes 1..7 are c * 2^-9, normal codes are 2^(e-7) * (1 + m/8) built from their bit fields.
__device__ __forceinline__ float e4m3_value(int c) {
    const int e = c >> 3, m = c & 7;
    if (e == 0) return (float)m * 0x1p-9f;
    return __uint_as_float(((uint32_t)(e + 120) << 23) | ((uint32_t)m << 20));
}

// E4M3 code nearest to s >= 0, ties to the even code, saturating at 448 (code 126).
// Normal range: round the binary32 mantissa to 3 bits with ties-to-even on the bit pattern
// (a carry moves into the exponent field, which is the next code). Below 2^-6 the codes are a
// uniform grid of step 2^-9, so the code is rint(s * 512) (the product is exact).
__device__ __forceinline__ int e4m3_rne_sat(float s) {
    if (!(s < 448.0f)) return 126;
    if (s < 0x1p-6f) return (int)__builtin_rintf(s * 512.0f);
    uint32_t u = __float_as_uint(s);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    const int e = (int)(u >> 23) - 127;
    const int code = ((e + 7) << 3) | (int)((u >> 20) & 7u);
    return code < 126 ? code : 126;
}

// E2M1 round-to-nearest-even of x[0..7] / 2^k, where 2^k is the power of two in `pow2`,
// returned as binary32 values. The eight 4-bit codes go through one dword (bytes 0..3, two
// codes per byte); its previous contents are irrelevant, so the first element's bits seed it.
__device__ __forceinline__ void e2m1_round8(const float (&x)[8], float pow2, float (&q)[8]) {
    uint32_t p = __float_as_uint(x[0]);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[0], x[1], pow2, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[2], x[3], pow2, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[4], x[5], pow2, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[6], x[7], pow2, 3);
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3);
    q[0] = v0[0]; q[1] = v0[1]; q[2] = v1[0]; q[3] = v1[1];
    q[4] = v2[0]; q[5] = v2[1]; q[6] = v3[0]; q[7] = v3[1];
}

// E2M1 codes of x[0..7] / pow2 (round to nearest even) in one dword, two per byte, x[2k] in
// the low nibble of byte k: the down-conversion half of e2m1_round8.
__device__ __forceinline__ uint32_t e2m1_codes8(const float (&x)[8], float pow2) {
    uint32_t p = __float_as_uint(x[0]);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[0], x[1], pow2, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[2], x[3], pow2, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[4], x[5], pow2, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, x[6], x[7], pow2, 3);
    return p;
}

// The levels of the two codes in byte SEL of p, as binary32 values.
template <int SEL>
__device__ __forceinline__ void e2m1_levels2(uint32_t p, float& q0, float& q1) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, SEL);
    q0 = v[0];
    q1 = v[1];
}

// Signed E2M1 codes of (x0, x1) written into byte `sel` of `word` (x0 -> low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t word, float x0, float x1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x0, x1, 1.0f, SEL);
}

// Row of a flat group index, gi / gpr, as (gi * M) >> (32 + L) with L = ceil(log2 gpr) and
// M = ceil(2^(32+L) / gpr) < 2^33: the product stays below 2^64 and the error term, below
// gi / 2^(32+L) < 2^-(L+1) <= 1/(2 gpr), cannot carry the quotient past an integer (gi < 2^31).
__device__ __forceinline__ uint32_t div_gpr(uint32_t gi, uint64_t magic, uint32_t shift) {
    return (uint32_t)(((uint64_t)gi * magic) >> shift);
}

}  // namespace nvfp4
