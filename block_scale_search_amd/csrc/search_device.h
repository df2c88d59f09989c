// Device-side group scale search for gfx950, shared by the fused search + pack kernel and by
// the GPTQ column sweep.
//
// Layout in the fused kernel: one lane owns one group of 16 consecutive weights of a row (32 B of bf16 or 64 B of
// f32, two or four 16-byte loads); consecutive lanes own consecutive groups, so a wave reads
// 2-4 KB of W contiguously and writes 512 B of packed codes and 64 scale bytes contiguously.
// The per-code table (eff[c], r[c]) of the matrix's global scale sits in LDS and each lane reads
// the entries of its own candidates.
//
// The candidate loop is VALU-bound (there is no contraction to put on MFMA). Per element and
// candidate it costs one multiply x = |w| * r, half a down-conversion and half an
// up-conversion (two elements per conversion), the residual fma and, for WMSE, the weighting
// multiply and the accumulating fma. Codes c and c + 8 are exactly one octave apart
// (E4M3 mantissa unchanged, exponent + 1), so r[c + 8] = r[c] / 2 and
// fl(|w| * r[c + 8]) = fl(|w| * r[c]) / 2 exactly; the down-conversion's power-of-two scale
// operand then rounds x / 2 with no second multiply. Waves whose candidate ranges all sit in
// the normal codes use that pairing; other waves (clipped windows, subnormal codes, a global
// scale that breaks the octave identity in binary32) score every code on its own. Both give the
// same bits. The argmin is lexicographic on (loss, code), which equals "first strictly smaller
// loss in ascending code order" and lets the paired loop visit codes out of order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_formats.h"

namespace nvfp4 {

// Loss of one code: the weighted squares summed in a fixed tree. For each quad k = 0..3,
// P_k = u_4k * d_4k, then P_k = fma(u_4k+i, d_4k+i, P_k) for i = 1, 2, 3; the loss is
// (P_0 + P_1) + (P_2 + P_3).
__device__ __forceinline__ float quad_tree(const float (&P)[4]) {
    const float left = P[0] + P[1];
    const float right = P[2] + P[3];
    return left + right;
}

template <bool WMSE>
__device__ __forceinline__ float loss_one(const float (&w)[16], const float (&h)[16], float eff,
                                          float r) {
    float P[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float x[8], q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fabsf(w[8 * half + i]) * r;
        e2m1_round8(x, 1.0f, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = 8 * half + i;
            const float a = fabsf(w[j]);
            const float d = __builtin_fmaf(-q[i], eff, a);
            const float u = WMSE ? h[j] * d : d;
            P[j >> 2] = (j & 3) == 0 ? u * d : __builtin_fmaf(u, d, P[j >> 2]);
        }
    }
    return quad_tree(P);
}

// Losses of codes c and c + 8 from one multiply per element (valid when both are normal codes
// and the table satisfies the octave identity).
template <bool WMSE>
__device__ __forceinline__ void loss_pair(const float (&w)[16], const float (&h)[16], float eff,
                                          float r, float eff_hi, float& L_lo, float& L_hi) {
    float P[4], Q[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        float x[8], q[8], s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fabsf(w[8 * half + i]) * r;
        e2m1_round8(x, 1.0f, q);
        e2m1_round8(x, 2.0f, s);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = 8 * half + i;
            const float a = fabsf(w[j]);
            const float d = __builtin_fmaf(-q[i], eff, a);
            const float e = __builtin_fmaf(-s[i], eff_hi, a);
            const float u = WMSE ? h[j] * d : d;
            const float v = WMSE ? h[j] * e : e;
            P[j >> 2] = (j & 3) == 0 ? u * d : __builtin_fmaf(u, d, P[j >> 2]);
            Q[j >> 2] = (j & 3) == 0 ? v * e : __builtin_fmaf(v, e, Q[j >> 2]);
        }
    }
    L_lo = quad_tree(P);
    L_hi = quad_tree(Q);
}

// Sequence point between candidates: an empty asm that reads and rewrites v, so everything that
// produced v is done before it and everything that uses v comes after it. Without it the compiler
// interleaves the arithmetic of several candidates, which raises the register count and lowers
// the number of waves a SIMD holds.
__device__ __forceinline__ void order_point(float& v) { asm volatile("" : "+v"(v)); }

// Running minimum over candidates visited in ascending code order: a strictly smaller loss
// replaces the best, so the first (lowest) code wins ties.
__device__ __forceinline__ void keep_min(float L, int c, float& best, int& best_c) {
    const bool take = L < best;
    best = take ? L : best;
    best_c = take ? c : best_c;
}

// One block of up to 16 consecutive codes c0 .. c0 + nb - 1 (all normal codes, octave identity
// holding): codes c0 + p and c0 + p + 8 share one multiply. The low codes (p < 8) and the high
// codes (p >= 8) are each scanned in ascending order; every high code follows every low code,
// so the block's first minimum is the low one unless the high one is strictly smaller. The
// block's result then enters the running minimum the same way. NB > 0 fixes the block length
// at compile time (full unroll); NB == 0 reads it from nb.
template <bool WMSE, int NB>
__device__ __forceinline__ void scan_block(const float (&w)[16], const float (&h)[16],
                                           const float2* __restrict__ t0, int c0, int nb,
                                           float& best, int& best_c) {
    const int n = NB > 0 ? NB : nb;
    float bl = __builtin_inff(), bh = __builtin_inff();
    int pl = 0, ph = 8;
#pragma unroll
    for (int p = 0; p < (NB > 0 ? (NB < 8 ? NB : 8) : 8); ++p) {
        if (NB == 0 && p >= n) break;
        float2 er = t0[p];
        order_point(er.x);
        order_point(er.y);
        if (p + 8 < n) {
            float L_lo, L_hi;
            loss_pair<WMSE>(w, h, er.x, er.y, t0[p + 8].x, L_lo, L_hi);
            if (L_lo < bl) { bl = L_lo; pl = p; }
            if (L_hi < bh) { bh = L_hi; ph = p + 8; }
        } else {
            const float L = loss_one<WMSE>(w, h, er.x, er.y);
            if (L < bl) { bl = L; pl = p; }
        }
        order_point(bl);
        order_point(bh);
    }
    keep_min(bl, c0 + pl, best, best_c);
    keep_min(bh, c0 + ph, best, best_c);
}

// Windowed search of one lane: codes first .. first + n - 1 (the window base + lo .. base + hi).
// Fast path for the whole wave when every live lane's codes are normal and unclipped.
template <bool WMSE, int NWIN>
__device__ __forceinline__ void search_window(const float (&w)[16], const float (&h)[16],
                                              const float2* __restrict__ tab, bool octave_ok,
                                              bool live, int first, int n_rt, float& best,
                                              int& best_c) {
    const int n = NWIN > 0 ? NWIN : n_rt;
    // idle lanes score the in-range dummy codes starting at 8
    const bool lane_fast = live ? (first >= 8 && first + n - 1 <= 126) : (n <= 119);
    if (octave_ok && __all(lane_fast)) {
        const int c0 = live ? first : 8;
        if constexpr (NWIN > 0 && NWIN <= 16) {
            scan_block<WMSE, NWIN>(w, h, tab + c0, c0, NWIN, best, best_c);
        } else {
            for (int blk = 0; blk < n; blk += 16)
                scan_block<WMSE, 0>(w, h, tab + c0 + blk, c0 + blk, min(16, n - blk), best,
                                    best_c);
        }
        return;
    }
    // clipped windows, subnormal codes or a table without the octave identity: every code on
    // its own, ascending
    for (int p = 0; p < n; ++p) {
        const int c = first + p;
        if (live && c >= 1 && c <= 126) {
            float2 er = tab[c];
            order_point(er.x);
            order_point(er.y);
            keep_min(loss_one<WMSE>(w, h, er.x, er.y), c, best, best_c);
            order_point(best);
        }
    }
}

// Lexicographic running minimum on (loss, code): the result of a scan that visits codes in any
// order equals the ascending scan's first minimum.
__device__ __forceinline__ void keep_min_lex(float L, int c, float& best, int& best_c) {
    const bool take = L < best || (L == best && c < best_c);
    best = take ? L : best;
    best_c = take ? c : best_c;
}

// Lower bounds of the loss over a whole range of codes, from one code's effective scale eff.
//  - Codes at or below the code of eff (eff' <= eff): an element with a > 6 eff saturates at
//    every such code, so its residual is at least a - 6 eff.
//  - Codes at or above it (eff' >= eff): an element with a < eff / 2 rounds either to 0 (residual
//    a) or to a level of at least eff' / 2 (residual at least eff / 2 - a).
// Both bound sums grow monotonically away from eff, so one test prunes every code beyond.
template <bool WMSE>
__device__ __forceinline__ float bound_below(const float (&w)[16], const float (&h)[16],
                                             float eff) {
    float B = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float t = fmaxf(__builtin_fmaf(-6.0f, eff, fabsf(w[j])), 0.0f);
        B = WMSE ? __builtin_fmaf(h[j] * t, t, B) : __builtin_fmaf(t, t, B);
    }
    return B;
}

template <bool WMSE>
__device__ __forceinline__ float bound_above(const float (&w)[16], const float (&h)[16],
                                             float eff) {
    const float half = 0.5f * eff;
    float B = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float a = fabsf(w[j]);
        const float t = a < half ? fminf(a, half - a) : 0.0f;
        B = WMSE ? __builtin_fmaf(h[j] * t, t, B) : __builtin_fmaf(t, t, B);
    }
    return B;
}

// Eight codes c0 .. c0 + 7 of one lane, each on its own; codes outside 1..126 are skipped.
template <bool WMSE>
__device__ __forceinline__ void scan8(const float (&w)[16], const float (&h)[16],
                                      const float2* __restrict__ tab, int c0, float& best,
                                      int& best_c) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int c = c0 + p;
        const bool in = c >= 1 && c <= 126;
        float2 er = tab[in ? c : 1];
        order_point(er.x);
        order_point(er.y);
        const float L = loss_one<WMSE>(w, h, er.x, er.y);
        if (in) keep_min_lex(L, c, best, best_c);
        order_point(best);
    }
}

// Exhaustive search over all 126 codes, with pruning that provably skips only losers.
// Each lane first scores the 16 codes around its own base code (octave pairs when the table
// allows), then extends upward and downward in blocks of 8 codes while the loss bounds above
// cannot exclude the next code. A bound prunes a direction when it exceeds the best loss by a
// relative margin of 2^-14, which covers the rounding of the binary32 loss tree and of the
// bound itself (each at most about 20 roundings of 2^-24 on sums of non-negative terms). The
// test is used only where that error analysis holds: non-negative finite h, a best loss of at
// least 2^-100 and amax (1 + max h) <= 2^100 best, so that underflowing products (absolute
// error 2^-150 each) stay far below the margin; elsewhere the lane scans every code. The result
// equals the ascending scan of all 126 codes with the first minimum kept.
template <bool WMSE>
__device__ __forceinline__ void search_all(const float (&w)[16], const float (&h)[16],
                                           const float2* __restrict__ tab, bool octave_ok,
                                           bool live, int b, float& best, int& best_c) {
    float amax = 0.0f, hmax = 1.0f;
    bool h_ok = true;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        amax = fmaxf(amax, fabsf(w[j]));
        if (WMSE) {
            hmax = fmaxf(hmax, h[j]);
            h_ok = h_ok && h[j] >= 0.0f && h[j] <= 0x1p100f;
        }
    }
    const float scale_ref = amax * (1.0f + hmax);

    // centre block: 16 codes from c0 (at least 8 and at most 111 so that pairs stay normal)
    const int c0 = live ? min(max(b - 8, 8), 111) : 8;
    if (octave_ok) {
        scan_block<WMSE, 16>(w, h, tab + c0, c0, 16, best, best_c);
    } else {
        scan8<WMSE>(w, h, tab, c0, best, best_c);
        scan8<WMSE>(w, h, tab, c0 + 8, best, best_c);
    }
    int up = c0 + 16, dn = c0 - 1;  // next unscored code in each direction
    bool up_done = !live || up > 126;
    bool dn_done = !live || dn < 1;
    while (true) {
        const bool can_prune = h_ok && best >= 0x1p-100f && scale_ref <= best * 0x1p100f;
        const float thr = __builtin_fmaf(best, 0x1p-14f, best);
        if (!up_done && can_prune) {
            const float B = bound_above<WMSE>(w, h, tab[up].x);
            up_done = B > thr && B <= 0x1.fffffep127f;
        }
        if (up_done && !dn_done && can_prune) {
            const float B = bound_below<WMSE>(w, h, tab[dn].x);
            dn_done = B > thr && B <= 0x1.fffffep127f;
        }
        const bool go_up = !up_done;
        const bool go_dn = up_done && !dn_done;
        if (!__any(go_up || go_dn)) break;
        const int first = go_up ? up : (go_dn ? dn - 7 : 8);
        float bl = best;
        int cl = best_c;
        scan8<WMSE>(w, h, tab, first, bl, cl);
        if (go_up || go_dn) {
            best = bl;
            best_c = cl;
        }
        if (go_up) {
            up += 8;
            up_done = up > 126;
        } else if (go_dn) {
            dn -= 8;
            dn_done = dn < 1;
        }
    }
}

// Per-workgroup code table in LDS: tab[c] = (eff[c], r[c]) for c = 1..126, tab[0] = (0, 0).
// Returns (uniformly) whether every normal pair (c, c + 8) satisfies eff[c+8] == 2 eff[c] and
// r[c+8] == r[c] / 2 with r[c] / 2 a normal number.
__device__ __forceinline__ bool build_table(float S, float2* tab, int* flag) {
    if (threadIdx.x == 0) *flag = 0;
    for (int t = threadIdx.x; t < 128; t += blockDim.x) {
        float eff = 0.0f, r = 0.0f;
        if (t >= 1 && t <= 126) {
            eff = S * e4m3_value(t);
            r = __fdiv_rn(1.0f, eff);
        }
        tab[t] = make_float2(eff, r);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 128; t += blockDim.x) {
        if (t >= 8 && t + 8 <= 126) {
            const float2 a = tab[t], b = tab[t + 8];
            const bool ok = (b.x == 2.0f * a.x) && (b.y == 0.5f * a.y) &&
                            (0.5f * a.y >= 0x1p-126f) && (2.0f * a.x < 0x1p127f);
            if (!ok) atomicOr(flag, 1);
        }
    }
    __syncthreads();
    return *flag == 0;
}

// Base code of a group: E4M3 round-to-nearest-even of (absmax / 6) / S, at least 1; 0 for an
// all-zero group.
__device__ __forceinline__ int base_code(const float (&w)[16], float S) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(w[j]));
    if (!(amax > 0.0f)) return 0;
    const float s_star = __fdiv_rn(__fdiv_rn(amax, 6.0f), S);
    return max(e4m3_rne_sat(s_star), 1);
}

}  // namespace nvfp4
