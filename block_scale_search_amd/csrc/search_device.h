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

// Losses of codes c (lo) and c + 8 (hi) under objective A and, where BLO / BHI, under objective
// B as well: both objectives share the multiply, the conversions and the residuals, and differ
// only in the weighting and the accumulation (each loss keeps the fixed tree order). With equal
// objectives the B losses are the A losses.
template <bool WA, bool WB, bool BLO, bool BHI, int QD, int HALF>
__device__ __forceinline__ void two_quad(const float (&w)[16], const float (&h)[16], uint32_t pq,
                                         uint32_t ps, float eff, float eff_hi, float& PA,
                                         float& QA, float& PB, float& QB) {
    constexpr bool OWN_B = WA != WB;
    float q[4], s[4];
    e2m1_levels2<2 * QD>(pq, q[0], q[1]);
    e2m1_levels2<2 * QD + 1>(pq, q[2], q[3]);
    e2m1_levels2<2 * QD>(ps, s[0], s[1]);
    e2m1_levels2<2 * QD + 1>(ps, s[2], s[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 8 * HALF + 4 * QD + i;
        const float a = fabsf(w[j]);
        const float d = __builtin_fmaf(-q[i], eff, a);
        const float e = __builtin_fmaf(-s[i], eff_hi, a);
        const float u = WA ? h[j] * d : d;
        const float v = WA ? h[j] * e : e;
        PA = i == 0 ? u * d : __builtin_fmaf(u, d, PA);
        QA = i == 0 ? v * e : __builtin_fmaf(v, e, QA);
        if constexpr (OWN_B && BLO) {
            const float ub = WB ? h[j] * d : d;
            PB = i == 0 ? ub * d : __builtin_fmaf(ub, d, PB);
        }
        if constexpr (OWN_B && BHI) {
            const float vb = WB ? h[j] * e : e;
            QB = i == 0 ? vb * e : __builtin_fmaf(vb, e, QB);
        }
    }
}

template <bool WA, bool WB, bool BLO, bool BHI, int HALF>
__device__ __forceinline__ void two_half(const float (&w)[16], const float (&h)[16], float eff,
                                         float r, float eff_hi, float& A_lo, float& A_hi,
                                         float& B_lo, float& B_hi) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fabsf(w[8 * HALF + i]) * r;
    const uint32_t pq = e2m1_codes8(x, 1.0f), ps = e2m1_codes8(x, 2.0f);
    float PA0, QA0, PB0, QB0, PA1, QA1, PB1, QB1;
    two_quad<WA, WB, BLO, BHI, 0, HALF>(w, h, pq, ps, eff, eff_hi, PA0, QA0, PB0, QB0);
    two_quad<WA, WB, BLO, BHI, 1, HALF>(w, h, pq, ps, eff, eff_hi, PA1, QA1, PB1, QB1);
    // the half's two quads: P_0 + P_1 (left) or P_2 + P_3 (right) of the loss tree
    A_lo = PA0 + PA1;
    A_hi = QA0 + QA1;
    if constexpr (WA != WB && BLO) B_lo = PB0 + PB1;
    if constexpr (WA != WB && BHI) B_hi = QB0 + QB1;
}

// Losses of codes c (lo) and c + 8 (hi) under objective A and, where BLO / BHI, under objective
// B as well: both objectives share the multiply, the conversions and the residuals, and differ
// only in the weighting and the accumulation. Each loss is the fixed tree
// (P_0 + P_1) + (P_2 + P_3), its halves summed as soon as they are complete. With equal
// objectives the B losses are the A losses.
template <bool WA, bool WB, bool BLO, bool BHI>
__device__ __forceinline__ void loss_pair_two(const float (&w)[16], const float (&h)[16],
                                              float eff, float r, float eff_hi, float& A_lo,
                                              float& A_hi, float& B_lo, float& B_hi) {
    float la_lo, la_hi, lb_lo = 0.0f, lb_hi = 0.0f, ra_lo, ra_hi, rb_lo = 0.0f, rb_hi = 0.0f;
    two_half<WA, WB, BLO, BHI, 0>(w, h, eff, r, eff_hi, la_lo, la_hi, lb_lo, lb_hi);
    two_half<WA, WB, BLO, BHI, 1>(w, h, eff, r, eff_hi, ra_lo, ra_hi, rb_lo, rb_hi);
    A_lo = la_lo + ra_lo;
    A_hi = la_hi + ra_hi;
    if constexpr (WA != WB) {
        B_lo = lb_lo + rb_lo;
        B_hi = lb_hi + rb_hi;
    } else {
        B_lo = A_lo;
        B_hi = A_hi;
    }
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

// Running minima of a 16-code block scanned for two windows at once: the outer window is the
// block c0 .. c0 + 15 under objective WA, the inner one its codes c0 + OFFB .. c0 + OFFB + NB - 1
// under objective WB. Each keeps the block's split into low codes (p < 8) and high codes
// (p >= 8), both ascending, as scan_block does.
struct TwoMins {
    float blA, bhA, blB, bhB;
    int plA, phA, plB, phB;
};

template <bool WA, bool WB, int OFFB, int NB, int P>
__device__ __forceinline__ void two_step(const float (&w)[16], const float (&h)[16],
                                         const float2* __restrict__ t0, TwoMins& m) {
    constexpr bool BLO = P >= OFFB && P < OFFB + NB;
    constexpr bool BHI = P + 8 >= OFFB && P + 8 < OFFB + NB;
    float2 er = t0[P];
    order_point(er.x);
    order_point(er.y);
    float Alo, Ahi, Blo, Bhi;
    loss_pair_two<WA, WB, BLO, BHI>(w, h, er.x, er.y, t0[P + 8].x, Alo, Ahi, Blo, Bhi);
    if (Alo < m.blA) { m.blA = Alo; m.plA = P; }
    if (Ahi < m.bhA) { m.bhA = Ahi; m.phA = P + 8; }
    if constexpr (BLO) {
        if (Blo < m.blB) { m.blB = Blo; m.plB = P; }
    }
    if constexpr (BHI) {
        if (Bhi < m.bhB) { m.bhB = Bhi; m.phB = P + 8; }
    }
    order_point(m.blA);
    order_point(m.bhA);
    order_point(m.blB);
    order_point(m.bhB);
}

template <bool WA, bool WB, int OFFB, int NB>
__device__ __forceinline__ void scan_block_two(const float (&w)[16], const float (&h)[16],
                                               const float2* __restrict__ t0, int c0,
                                               float& bestA, int& best_cA, float& bestB,
                                               int& best_cB) {
    static_assert(OFFB >= 0 && NB >= 1 && OFFB + NB <= 16, "inner window inside the block");
    TwoMins m{__builtin_inff(), __builtin_inff(), __builtin_inff(), __builtin_inff(),
              0, 8, 0, 8};
    two_step<WA, WB, OFFB, NB, 0>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 1>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 2>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 3>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 4>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 5>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 6>(w, h, t0, m);
    two_step<WA, WB, OFFB, NB, 7>(w, h, t0, m);
    keep_min(m.blA, c0 + m.plA, bestA, best_cA);
    keep_min(m.bhA, c0 + m.phA, bestA, best_cA);
    keep_min(m.blB, c0 + m.plB, bestB, best_cB);
    keep_min(m.bhB, c0 + m.phB, bestB, best_cB);
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
        // a < half: min(a, half - a), both non-negative; a >= half: half - a <= 0, so 0. The
        // median of (a, half - a, 0) is exactly that, in one instruction.
        const float t = __builtin_amdgcn_fmed3f(a, half - a, 0.0f);
        B = WMSE ? __builtin_fmaf(h[j] * t, t, B) : __builtin_fmaf(t, t, B);
    }
    return B;
}

// N codes c0 .. c0 + N - 1 of one lane, each on its own and in ascending order; codes outside
// 1..126 are skipped. The caller starts the running minimum at (+inf, the first code in range)
// and a strictly smaller loss replaces it, so the result is the scan's first minimum, which is
// the lexicographic minimum of (loss, code).
template <bool WMSE, int N>
__device__ __forceinline__ void scan_codes(const float (&w)[16], const float (&h)[16],
                                           const float2* __restrict__ tab, int c0, float& best,
                                           int& best_c) {
#pragma unroll
    for (int p = 0; p < N; ++p) {
        const int c = c0 + p;
        const bool in = c >= 1 && c <= 126;
        float2 er = tab[in ? c : 1];
        order_point(er.x);
        order_point(er.y);
        const float L = loss_one<WMSE>(w, h, er.x, er.y);
        keep_min(in ? L : __builtin_inff(), c, best, best_c);
        order_point(best);
    }
}

// Codes per pending block of the exhaustive search (beyond the 16-code centre).
constexpr int kBlockCodes = 4;

// Exhaustive search over all 126 codes, with pruning that provably skips only losers, in three
// phases per workgroup.
//  1. Each lane scores the 16 codes around its own base code (octave pairs when the table
//     allows) and counts the blocks of kBlockCodes codes it still needs above and below them: a block,
//     and every block beyond it, is skipped when a lower bound on the loss at the block's first
//     code exceeds the lane's best loss by a relative margin of 2^-14. The margin covers the
//     rounding of the binary32 loss tree and of the bound itself (each at most about 20
//     roundings of 2^-24 on sums of non-negative terms). The test is used only where that
//     error analysis holds: every h_j without sign bit and at most 2^100, a best loss of at
//     least 2^-100 and amax (1 + max h) <= 2^100 best, so that underflowing products (absolute
//     error 2^-150 each) stay far below the margin; elsewhere the lane needs every block.
//  2. The workgroup's pending blocks are dealt over its lanes, 64 items per wave and round (a
//     prefix of the per-lane counts in LDS tells each item's owner), so that the workgroup runs
//     ceil(total / 64) wave-rounds of kBlockCodes codes instead of as many rounds as its busiest
//     lane needs in every wave. A lane scoring another lane's block reloads that group's
//     weights and h (recently read, so from the caches). Each block's lowest
//     (loss, code) is merged into its owner's slot with an LDS 64-bit minimum on a key whose
//     unsigned order is the (loss, code) order (loss_key below), so the merged result does not
//     depend on the order of the merges.
//  3. Each lane reads its slot.
// Every skipped code provably has a larger binary32 loss than the best found, so the result is
// the lexicographic minimum of (loss, code) over all 126 codes: the ascending scan's first
// minimum.

// Phase 1 of one lane, first half: the centre block of 16 codes c0 .. c0 + 15 with
// c0 = clamp(b + clo, 8, 111) (at least 8 and at most 111 so that octave pairs stay normal),
// scanned in ascending order from (+inf, c0). Where c0 = b + clo this is exactly the ascending
// scan of the window clo .. clo + 15, so a 16-code window's result comes from the same losses.
// Returns c0.
template <bool WMSE>
__device__ __forceinline__ int centre_scan(const float (&w)[16], const float (&h)[16],
                                           const float2* __restrict__ tab, bool octave_ok,
                                           bool live, int b, int clo, float& best,
                                           int& best_c) {
    const int c0 = live ? min(max(b + clo, 8), 111) : 8;
    best = __builtin_inff();
    best_c = c0;
    if (octave_ok) {
        scan_block<WMSE, 16>(w, h, tab + c0, c0, 16, best, best_c);
    } else {
        scan_codes<WMSE, 16>(w, h, tab, c0, best, best_c);
    }
    return c0;
}

// Blocks needed in one direction from the centre: blocks k = 0 .. all - 1 start at code
// first + kBlockCodes k (UP) or end at code first - kBlockCodes k (down), and block k, with
// every block beyond it, is
// skipped when its bound B_k exceeds thr (and is finite). B_k is nondecreasing in k (the
// effective scale grows, or shrinks, monotonically, and every step of the bound is monotone in
// it), so a pruned block 1 leaves block 0's test to decide between 0 and 1 blocks, and a kept
// block 1 means at least 2: the second test runs at block 0 or block 2 per lane, one pass for
// the whole wave, and only lanes needing 3 blocks or more test further. (Where B_1 overflows
// to +inf, blocks 0 and 1 are both kept: more blocks, never fewer, than the tests allow.)
template <bool WMSE, bool UP>
__device__ __forceinline__ int blocks_needed(const float (&w)[16], const float (&h)[16],
                                             const float2* __restrict__ tab, int first, int all,
                                             float thr) {
    auto needed = [&](int k) {
        const float e = tab[UP ? first + kBlockCodes * k : first - kBlockCodes * k].x;
        const float B = UP ? bound_above<WMSE>(w, h, e) : bound_below<WMSE>(w, h, e);
        return !(B > thr && B <= 0x1.fffffep127f);
    };
    int n = 0;
    if (all > 0) {
        const bool na = needed(min(1, all - 1));
        const int kb = na ? 2 : 0;
        bool nb = false;
        if (all >= 2 && kb < all) nb = needed(kb);
        if (all == 1) {
            n = na ? 1 : 0;
        } else if (!na) {
            n = nb ? 1 : 0;
        } else if (all == 2 || !nb) {
            n = 2;
        } else {
            n = 3;
            while (n < all && needed(n)) ++n;
        }
    }
    return n;
}

// Phase 1, second half: the numbers of kBlockCodes-code blocks needed above the centre block (n_up, from
// code c0 + 16) and below it (n_dn, down from code c0 - 1), given the centre's best loss.
template <bool WMSE>
__device__ __forceinline__ void pending_blocks(const float (&w)[16], const float (&h)[16],
                                               const float2* __restrict__ tab, bool live, int c0,
                                               float best, int& n_up, int& n_dn) {
    n_up = 0;
    n_dn = 0;
    if (!live) return;
    // h on its binary32 bit patterns: every h_j is a non-negative number of at most 2^100
    // (no sign bit, not NaN) exactly when the largest pattern is at most that of 2^100, and the
    // largest pattern is then the largest h_j
    float amax = 0.0f;
    uint32_t hbits = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        amax = fmaxf(amax, fabsf(w[j]));
        if (WMSE) hbits = max(hbits, __float_as_uint(h[j]));
    }
    const bool h_ok = hbits <= 0x71800000u;     // the pattern of 2^100
    const float hmax = fmaxf(1.0f, __uint_as_float(hbits));
    const float scale_ref = amax * (1.0f + hmax);
    const int up = c0 + 16, dn = c0 - 1;
    const int all_up = up <= 126 ? (126 - up) / kBlockCodes + 1 : 0;
    const int all_dn = dn >= 1 ? (dn - 1) / kBlockCodes + 1 : 0;
    const bool can_prune = h_ok && best >= 0x1p-100f && scale_ref <= best * 0x1p100f;
    if (!can_prune) {
        n_up = all_up;
        n_dn = all_dn;
        return;
    }
    const float thr = __builtin_fmaf(best, 0x1p-14f, best);
    n_up = blocks_needed<WMSE, true>(w, h, tab, up, all_up, thr);
    n_dn = blocks_needed<WMSE, false>(w, h, tab, dn, all_dn, thr);
}

// (loss, code) as one 64-bit key whose unsigned order is the lexicographic order of the scan:
// the high word maps the binary32 loss monotonically onto an unsigned value (negative losses,
// possible with a caller's negative h, below positive ones; -0 and +0 onto the same value, as
// they compare equal; NaN above everything, as a strict comparison never takes it), then the
// code, then the loss's sign bit, so that the winner's exact loss (a zero's sign included) can
// be read back.
__device__ __forceinline__ uint64_t loss_key(float L, int c) {
    const uint32_t u = __float_as_uint(L);
    const uint32_t mag = u & 0x7FFFFFFFu;
    const uint32_t ord = (L != L) ? 0xFFFFFFFFu
                         : ((u >> 31) ? 0x80000000u - mag : 0x80000000u + mag);
    return ((uint64_t)ord << 32) | ((uint64_t)(uint32_t)c << 1) | (uint64_t)(u >> 31);
}

__device__ __forceinline__ int key_code(uint64_t k) { return (int)((k >> 1) & 0xFFu); }

__device__ __forceinline__ float key_loss(uint64_t k) {
    const uint32_t ord = (uint32_t)(k >> 32);
    if (ord == 0xFFFFFFFFu) return __uint_as_float(0x7FC00000u);
    const uint32_t sign = (uint32_t)(k & 1u) << 31;
    const uint32_t mag = ord >= 0x80000000u ? ord - 0x80000000u : 0x80000000u - ord;
    return __uint_as_float(sign | mag);
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
