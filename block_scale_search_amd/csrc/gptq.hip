// GPTQ with the per-group scale search as its local quantiser, for gfx950 (H-Scale App. B: the
// search replaces only the local quantisation call; inverse-Cholesky processing and error
// propagation are kept; Replay the Curvature §3: input columns in sequence, one shared Hessian
// factor, output rows independent).
//
// Per output row, binary32, column j = 0..in-1 in order:
//   - at a group's first column its scale code is searched on the row's current values;
//   - the column is quantised at that code, v = fl(q * eff), err = fl(fl(w_j - v) / U[j][j]);
//   - every later column k takes w_k = fma(-err, U[j][k], w_k).
// U is the upper-triangular factor of the damped inverse Hessian (row-major [in, in]).
//
// Columns run in outer blocks of 256, each made of 4 inner blocks of 64.
//   outer:  one kernel per outer block. 16 lanes per row (4 rows per wave) hold the row's 256
//           outer-block columns in registers, 16 per lane: 4 consecutive columns of each inner
//           block, so that lanes 4q..4q+3 hold group q of the inner block being quantised. Per
//           inner block, U's rows of that block (its columns up to the outer block's end; zero
//           at or left of the diagonal) are staged in LDS. At a group's first column the 16
//           lanes gather the group's current values by DPP row broadcasts and score the
//           window's codes side by side (lane i takes candidates i, i + 16, ...); a
//           lexicographic (loss, code) minimum over the 16 lanes picks the code, which equals
//           the ascending scan's first minimum. Per column, the lane holding it quantises and
//           divides and stores the column's final value, error and code; the error goes to the
//           row's 16 lanes by a DPP row broadcast, and every lane takes fma(-err, U[j][k], w_k)
//           on its 16 columns (a zero U entry leaves a value unchanged up to the sign of a
//           zero, and the columns at or before j were stored when they were quantised). The
//           chain through the errors is serial, so this kernel is latency-bound.
//   update: after each outer block every later column takes its 256 updates as one fma chain
//           in column order, acc = fma(-err_j, U[j][k], acc), on 128-, 64- or 32-row x
//           128-column tiles (8, 4 or 2 x 8 per thread, the height chosen so that the tiles
//           fill the resident workgroups evenly) with the errors and U rows
//           staged through LDS. Batching 256 errors per pass over the later columns keeps the
//           pass bound by the fma issue rate rather than by HBM.
// Each element of W sees exactly the sequential algorithm's fma sequence, so the result does
// not depend on the blocking.
#include <hip/hip_runtime.h>

#include <atomic>
#include <utility>

#include "device_formats.h"
#include "internal.h"
#include "search_device.h"

namespace nvfp4 {
namespace {

constexpr int kB = 64;          // columns per block (a multiple of the group size 16)

// W (bf16 or f32, row stride ldw) -> binary32 working copy [out, in].
template <bool BF16>
__global__ __launch_bounds__(256) void k_gptq_load(const uint8_t* __restrict__ W, int64_t out,
                                                   int64_t in, int64_t ldw_bytes,
                                                   float* __restrict__ Wf) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= out * in) return;
    const int64_t o = i / in, c = i - o * in;
    if constexpr (BF16) {
        const uint16_t v = *reinterpret_cast<const uint16_t*>(W + o * ldw_bytes + c * 2);
        Wf[i] = __uint_as_float((uint32_t)v << 16);
    } else {
        Wf[i] = *reinterpret_cast<const float*>(W + o * ldw_bytes + c * 4);
    }
}

// DPP moves within 16-lane rows: lane n of each row to the whole row, and the butterfly steps
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror) of a 16-lane reduction.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return dpp_f<0x150 + N>(x);
}

// Lexicographic (loss, code) minimum over the 16 lanes of a row; every lane gets the result.
template <int CTRL>
__device__ __forceinline__ void lex_step(float& L, int& c) {
    const float oL = dpp_f<CTRL>(L);
    const int oc = dpp_i<CTRL>(c);
    const bool take = oL < L || (oL == L && oc < c);
    L = take ? oL : L;
    c = take ? oc : c;
}
__device__ __forceinline__ int row_argmin(float L, int c) {
    lex_step<0xB1>(L, c);
    lex_step<0x4E>(L, c);
    lex_step<0x141>(L, c);
    lex_step<0x140>(L, c);
    return c;
}

constexpr int kOB = 256;        // columns per outer block
constexpr int kBlockRows = 16;  // rows per block-kernel workgroup (256 threads)

// One lane of the outer-block kernel: 16 of the row's columns in registers, 4 per inner block
// (slot s = inner block i + s, element e = column 64 (i + s) + 4t + e of the outer block). Slot
// 0 is the inner block being quantised; after each inner block the slots shift down by one.
struct OuterLane {
    float w[16];       // current values
    float dg[4];       // slot 0: U[c][c] of the lane's 4 columns
    float wq[4];       // slot 0: each column's value when it was quantised
    float ev[4];       // slot 0: each column's error
    uint32_t nibs;     // slot 0: the 4 columns' E2M1 codes, column 4t + e at bit 4e
    float2 er;         // (eff, r) of the current group's code
    float4 u[4];       // the lane's U entries of the current column, one float4 per slot
    int t;             // lane within the row
    bool valid;
};

// LDS of the outer-block kernel. us[J][s][t] holds U[row J of the inner block][the 4 columns of
// lane t in slot s]; in slot 0 the entries at or left of the diagonal are zero.
struct OuterLds {
    float4 us[kB][4][16];   // 64 KB
    float hb[kOB];
    float ud[kB];
    float2 tab[128];
    int flag;
};

// Column J of the current inner block (J is a compile-time constant so that register indices
// and DPP lane selects are fixed).
template <bool WMSE, int NWIN, int J>
__device__ __forceinline__ void outer_step(OuterLane& s, const OuterLds& L, int bc, int hcol,
                                           float S, int lo, int n, uint8_t* __restrict__ scale_row) {
    // Columns at or after bc (a ragged last inner block) run as padding: zero values, zero U
    // entries and a unit diagonal give code 0 and a +0 error, and fma(-(+0), +0, w) == w
    // exactly, so they change nothing that is kept; only their outputs are skipped.
    if constexpr ((J & 15) == 0) {
        // the group's 16 current values and h in every lane of the row
        constexpr int q4 = J >> 2;
        float wg[16], h[16];
        wg[0] = row_bcast<q4 + 0>(s.w[0]);
        wg[1] = row_bcast<q4 + 0>(s.w[1]);
        wg[2] = row_bcast<q4 + 0>(s.w[2]);
        wg[3] = row_bcast<q4 + 0>(s.w[3]);
        wg[4] = row_bcast<q4 + 1>(s.w[0]);
        wg[5] = row_bcast<q4 + 1>(s.w[1]);
        wg[6] = row_bcast<q4 + 1>(s.w[2]);
        wg[7] = row_bcast<q4 + 1>(s.w[3]);
        wg[8] = row_bcast<q4 + 2>(s.w[0]);
        wg[9] = row_bcast<q4 + 2>(s.w[1]);
        wg[10] = row_bcast<q4 + 2>(s.w[2]);
        wg[11] = row_bcast<q4 + 2>(s.w[3]);
        wg[12] = row_bcast<q4 + 3>(s.w[0]);
        wg[13] = row_bcast<q4 + 3>(s.w[1]);
        wg[14] = row_bcast<q4 + 3>(s.w[2]);
        wg[15] = row_bcast<q4 + 3>(s.w[3]);
#pragma unroll
        for (int e = 0; e < 16; ++e) h[e] = WMSE ? L.hb[hcol + J + e] : 0.0f;
        const int b = base_code(wg, S);
        const bool live = s.valid && b > 0;
        // lane t scores codes first + t, first + t + 16, ...; codes outside 1..126 are skipped
        // and a NaN loss counts as +inf, so the lexicographic minimum equals the ascending
        // scan's first strict minimum started from the lowest in-range code
        float best = __builtin_inff();
        int best_c = 127;
        const int first = b + lo;
#pragma unroll
        for (int p0 = 0; p0 < (NWIN > 0 ? (NWIN + 15) / 16 : 1) * 16; p0 += 16) {
            const int p = p0 + s.t;
            const int c = first + p;
            if (live && p < n && c >= 1 && c <= 126) {
                const float2 ce = L.tab[c];
                float Lc = loss_one<WMSE>(wg, h, ce.x, ce.y);
                Lc = (Lc == Lc) ? Lc : __builtin_inff();
                keep_min_lex(Lc, c, best, best_c);
            }
        }
        if constexpr (NWIN == 0) {
            for (int p = 16 + s.t; p < n; p += 16) {
                const int c = first + p;
                if (live && c >= 1 && c <= 126) {
                    const float2 ce = L.tab[c];
                    float Lc = loss_one<WMSE>(wg, h, ce.x, ce.y);
                    Lc = (Lc == Lc) ? Lc : __builtin_inff();
                    keep_min_lex(Lc, c, best, best_c);
                }
            }
        }
        const int cm = row_argmin(best, best_c);
        const int c = live ? cm : 0;
        s.er = L.tab[c];                         // (0, 0) for code 0: signed zero codes
        if (s.valid && s.t == q4 && J < bc) scale_row[J / 16] = (uint8_t)c;
    }
    // the next column's U entries are read now, so that their LDS latency overlaps this
    // column's chain
    float4 un[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) un[sl] = L.us[J + 1 < kB ? J + 1 : J][sl][s.t];
    // quantise column J (meaningful in the lane that holds it: lane J / 4, element J % 4)
    constexpr int e = J & 3;
    const float wj = s.w[e];
    const uint32_t byte =
        __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, wj * s.er.y, 0.0f, 1.0f, 0);
    const float q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0)[0];
    const float v = q * s.er.x;
    const float err_own = __fdiv_rn(wj - v, s.dg[e]);
    const float err = row_bcast<(J >> 2)>(err_own);
    // the lane holding column J keeps its value, error and code (selects, no branch); they are
    // stored after the inner block
    const bool mine = s.t == (J >> 2);
    s.wq[e] = mine ? wj : s.wq[e];
    s.ev[e] = mine ? err_own : s.ev[e];
    s.nibs = mine ? (s.nibs | ((byte & 15u) << (4 * e))) : s.nibs;
    asm volatile("" : "+v"(s.wq[e]), "+v"(s.ev[e]), "+v"(s.nibs));
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
        const float4 u4 = s.u[sl];
        s.w[4 * sl + 0] = __builtin_fmaf(-err, u4.x, s.w[4 * sl + 0]);
        s.w[4 * sl + 1] = __builtin_fmaf(-err, u4.y, s.w[4 * sl + 1]);
        s.w[4 * sl + 2] = __builtin_fmaf(-err, u4.z, s.w[4 * sl + 2]);
        s.w[4 * sl + 3] = __builtin_fmaf(-err, u4.w, s.w[4 * sl + 3]);
        s.u[sl] = un[sl];
    }
    // Keep each column's instructions together: the compiler would otherwise defer each
    // register's fma updates to that register's next use, keeping the errors and U entries of
    // many columns live at once. The empty asm makes all 16 values due here.
    asm volatile("" : "+v"(s.w[0]), "+v"(s.w[1]), "+v"(s.w[2]), "+v"(s.w[3]), "+v"(s.w[4]),
                 "+v"(s.w[5]), "+v"(s.w[6]), "+v"(s.w[7]), "+v"(s.w[8]), "+v"(s.w[9]),
                 "+v"(s.w[10]), "+v"(s.w[11]), "+v"(s.w[12]), "+v"(s.w[13]), "+v"(s.w[14]),
                 "+v"(s.w[15]));
    __builtin_amdgcn_sched_barrier(0);
}

template <bool WMSE, int NWIN, int... J>
__device__ __forceinline__ void outer_steps(OuterLane& s, const OuterLds& L, int bc, int hcol,
                                            float S, int lo, int n, uint8_t* __restrict__ scale_row,
                                            std::integer_sequence<int, J...>) {
    (outer_step<WMSE, NWIN, J>(s, L, bc, hcol, S, lo, n, scale_row), ...);
}

// One outer block (columns o0 .. o1 - 1, at most 256) of 16 rows per workgroup: its 4 inner
// blocks in order, each followed by its updates of the outer block's later columns (held in
// the lanes' registers). Writes the columns' final values, scale bytes and codes, and the outer
// block's errors E[0 .. o1 - o0)[r] (row stride ldE).
struct OuterArgs {
    float* Wf;
    int64_t out, in, o0;
    int oc;
    const float* U;
    const float* h;
    int lo, hi;
    const float* S;
    uint8_t* scales;
    uint8_t* packed;
    float* E;          // this outer block's errors
    int64_t ldE;
};

template <bool WMSE, int NWIN>
__device__ __forceinline__ void outer_body(OuterLds& L, uint32_t rg, const OuterArgs& a) {
    float* __restrict__ Wf = a.Wf;
    const int64_t out = a.out, in = a.in, o0 = a.o0, ldE = a.ldE;
    const int oc = a.oc, lo = a.lo, hi = a.hi;
    const float* __restrict__ U = a.U;
    const float* __restrict__ hvec = a.h;
    uint8_t* __restrict__ scales = a.scales;
    uint8_t* __restrict__ packed = a.packed;
    float* __restrict__ E = a.E;
    const int tid = threadIdx.x;
    OuterLane s;
    s.t = tid & 15;
    const int64_t r = (int64_t)rg * kBlockRows + (tid >> 4);
    s.valid = r < out;
    const int t = s.t;

    // the row's 16 columns first: their loads overlap the table set-up
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (s.valid && 64 * sl + 4 * t < oc)
            v = *reinterpret_cast<const float4*>(Wf + r * in + o0 + 64 * sl + 4 * t);
        s.w[4 * sl + 0] = v.x;
        s.w[4 * sl + 1] = v.y;
        s.w[4 * sl + 2] = v.z;
        s.w[4 * sl + 3] = v.w;
    }
    for (int i = tid; i < kOB; i += 256) L.hb[i] = (WMSE && i < oc) ? hvec[o0 + i] : 0.0f;
    const float S = a.S[0];
    build_table(S, L.tab, &L.flag);   // its octave test is unused here
    const int n = hi - lo + 1;
    uint8_t* scale_row = scales + (s.valid ? r : 0) * (in / 16) + o0 / 16;

    // U staging of an inner block: thread tid holds the 16 float4 of rows J = tid / 64 + 4q,
    // slot (tid / 16) % 4, lane tid % 16 (q = 0..15). The next inner block's are loaded into
    // registers before this block's columns run, so their latency overlaps the column chain.
    float4 pre[16];
    const int sl_t = (tid >> 4) & 3, tt_t = tid & 15, k_t = 64 * sl_t + 4 * tt_t;
    auto load_u = [&](int ib) {
        const int64_t b0 = o0 + (int64_t)ib * kB;
        const int bc = min(kB, oc - ib * kB), rest = oc - ib * kB;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int J = (tid >> 6) + 4 * q;
            pre[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (J < bc && k_t < rest)
                pre[q] = *reinterpret_cast<const float4*>(U + (b0 + J) * in + b0 + k_t);
        }
    };
    // results of an inner block, kept until they are stored
    float pq[4], pe[4];
    uint32_t pn = 0u;
    auto store_block = [&](int ib) {
        const int bc = min(kB, oc - ib * kB);
        if (!s.valid || 4 * t >= bc) return;
        const int64_t b0 = o0 + (int64_t)ib * kB;
        *reinterpret_cast<float4*>(Wf + r * in + b0 + 4 * t) = make_float4(pq[0], pq[1], pq[2], pq[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) E[(int64_t)(ib * kB + 4 * t + e) * ldE + r] = pe[e];
        // columns 4t .. 4t + 3: two bytes, even column in the low nibble
        *reinterpret_cast<uint16_t*>(packed + r * (in / 2) + (b0 + 4 * t) / 2) = (uint16_t)pn;
    };
    load_u(0);
    for (int ib = 0; ib * kB < oc; ++ib) {
        const int bc = min(kB, oc - ib * kB);
        __syncthreads();                                // the previous inner block's readers
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int J = (tid >> 6) + 4 * q;
            float4 v = pre[q];
            if (sl_t == 0) {
                const int dj = J - k_t;
                const float dv = dj == 0 ? v.x : (dj == 1 ? v.y : (dj == 2 ? v.z : v.w));
                if (dj >= 0 && dj < 4) L.ud[J] = J < bc ? dv : 1.0f;
                v.x = k_t + 0 > J ? v.x : 0.0f;
                v.y = k_t + 1 > J ? v.y : 0.0f;
                v.z = k_t + 2 > J ? v.z : 0.0f;
                v.w = k_t + 3 > J ? v.w : 0.0f;
            }
            L.us[J][sl_t][tt_t] = v;
        }
        __syncthreads();
        // the previous inner block's results, stored only now: a store still in flight at the
        // staging above would have been waited for with the prefetched loads
        if (ib > 0) store_block(ib - 1);
        if ((ib + 1) * kB < oc) load_u(ib + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s.dg[e] = L.ud[4 * t + e];
            s.wq[e] = s.ev[e] = 0.0f;
        }
        s.nibs = 0u;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) s.u[sl] = L.us[0][sl][t];
        outer_steps<WMSE, NWIN>(s, L, bc, ib * kB, S, lo, n, scale_row + ib * (kB / 16),
                                std::make_integer_sequence<int, kB>{});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pq[e] = s.wq[e];
            pe[e] = s.ev[e];
        }
        pn = s.nibs;
        // the next inner block's columns move to slot 0
#pragma unroll
        for (int k = 0; k < 12; ++k) s.w[k] = s.w[k + 4];
    }
    store_block((oc - 1) / kB);
}

template <bool WMSE, int NWIN>
__global__ __launch_bounds__(256) void k_gptq_outer(OuterArgs a) {
    __shared__ OuterLds L;
    outer_body<WMSE, NWIN>(L, blockIdx.x, a);
}

// Columns [k0, k1) of every row take nj updates: acc = fma(-E[jj][r], U[j0 + jj][k], acc) for
// jj = 0..nj-1 in order (E transposed: [kOB][ldE], ldE = out rounded up to a multiple of 4). A workgroup owns a 128 x 128 tile, a thread
// 8 rows x 8 columns (rows 4ty + a and 64 + 4ty + a, columns 4tx + b and 64 + 4tx + b, so that
// each LDS read of a wave covers 256 contiguous bytes); errors and U rows go through LDS
// kUc at a time.
constexpr int kUc = 32;

struct UpdateLds {
    float es[kUc][128];   // [jj][row]
    float us[kUc][128];   // [jj][col]
};

struct UpdateArgs {
    float* Wf;
    int64_t out, in, k0, k1;
    const float* U;
    int64_t j0;
    int nj;
    const float* E;
    int64_t ldE;
    uint32_t gx;          // column tiles
};

// Row of accumulator a of thread row ty in a tile of 16 TR rows: for TR = 8 rows 4ty + a and
// 64 + 4ty + a - 4 (each LDS read of a wave then covers 256 contiguous bytes), for TR = 4 and
// TR = 2 rows TR ty + a.
template <int TR>
__device__ __forceinline__ int tile_row(int ty, int a) {
    if constexpr (TR == 8) return a < 4 ? 4 * ty + a : 64 + 4 * ty + a - 4;
    else return TR * ty + a;
}

// Columns [k0, k1) of every row take nj updates: acc = fma(-E[jj][r], U[j0 + jj][k], acc) for
// jj = 0..nj-1 in order (E transposed: [kOB][ldE], ldE = out rounded up to a multiple of 4).
// A workgroup owns 16 TR rows x 128 columns, a thread TR rows x 8 columns (columns 4tx + b and
// 64 + 4tx + b); errors and U rows go through LDS kUc at a time. TR = 2 gives narrow updates
// (a few column tiles) enough workgroups to fill the chip.
template <int TR>
__device__ __forceinline__ void update_body(UpdateLds& L, uint32_t bx, uint32_t by,
                                            const UpdateArgs& p) {
    constexpr int RT = 16 * TR;
    float* __restrict__ Wf = p.Wf;
    const int64_t out = p.out, in = p.in, k0 = p.k0, k1 = p.k1, j0 = p.j0, ldE = p.ldE;
    const int nj = p.nj;
    const float* __restrict__ U = p.U;
    const float* __restrict__ E = p.E;
    auto& es = L.es;
    auto& us = L.us;
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)by * RT, c0 = k0 + (int64_t)bx * 128;
    const int ty = tid >> 4, tx = tid & 15;
    float acc[TR][8];
#pragma unroll
    for (int a = 0; a < TR; ++a) {
        const int64_t r = r0 + tile_row<TR>(ty, a);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int64_t c = c0 + 64 * hb + 4 * tx;   // k1 - k0 is a multiple of 16
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (r < out && c < k1) v = *reinterpret_cast<const float4*>(Wf + r * in + c);
            acc[a][4 * hb + 0] = v.x;
            acc[a][4 * hb + 1] = v.y;
            acc[a][4 * hb + 2] = v.z;
            acc[a][4 * hb + 3] = v.w;
        }
    }
    constexpr int QE = kUc * RT / 4 / 256, QU = kUc * 128 / 4 / 256;
    float4 pe[QE], pu[QU];
    auto load_chunk = [&](int jc) {
        const int m = min(kUc, nj - jc);
#pragma unroll
        for (int q = 0; q < QE; ++q) {
            const int i = tid + 256 * q;
            const int jj = i / (RT / 4), x4 = (i % (RT / 4)) * 4;
            pe[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (jj < m && r0 + x4 < out)   // rows out .. ldE - 1 are padding
                pe[q] = *reinterpret_cast<const float4*>(E + (jc + jj) * ldE + r0 + x4);
        }
#pragma unroll
        for (int q = 0; q < QU; ++q) {
            const int i = tid + 256 * q;
            const int jj = i >> 5, x4 = (i & 31) * 4;
            pu[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (jj < m && c0 + x4 < k1)
                pu[q] = *reinterpret_cast<const float4*>(U + (j0 + jc + jj) * in + c0 + x4);
        }
    };
    load_chunk(0);
    for (int jc = 0; jc < nj; jc += kUc) {
        const int m = min(kUc, nj - jc);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < QE; ++q) {
            const int i = tid + 256 * q;
            *reinterpret_cast<float4*>(&es[i / (RT / 4)][(i % (RT / 4)) * 4]) = pe[q];
        }
#pragma unroll
        for (int q = 0; q < QU; ++q) {
            const int i = tid + 256 * q;
            *reinterpret_cast<float4*>(&us[i >> 5][(i & 31) * 4]) = pu[q];
        }
        __syncthreads();
        if (jc + kUc < nj) load_chunk(jc + kUc);
        for (int jj = 0; jj < m; ++jj) {
            float e[TR];
            if constexpr (TR == 8) {
                const float4 e0 = *reinterpret_cast<const float4*>(&es[jj][4 * ty]);
                const float4 e1 = *reinterpret_cast<const float4*>(&es[jj][64 + 4 * ty]);
                e[0] = e0.x; e[1] = e0.y; e[2] = e0.z; e[3] = e0.w;
                e[4] = e1.x; e[5] = e1.y; e[6] = e1.z; e[7] = e1.w;
            } else if constexpr (TR == 4) {
                const float4 e0 = *reinterpret_cast<const float4*>(&es[jj][4 * ty]);
                e[0] = e0.x; e[1] = e0.y; e[2] = e0.z; e[3] = e0.w;
            } else {
                const float2 e0 = *reinterpret_cast<const float2*>(&es[jj][2 * ty]);
                e[0] = e0.x; e[1] = e0.y;
            }
            const float4 u0 = *reinterpret_cast<const float4*>(&us[jj][4 * tx]);
            const float4 u1 = *reinterpret_cast<const float4*>(&us[jj][64 + 4 * tx]);
            const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int a = 0; a < TR; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fmaf(-e[a], u[b], acc[a][b]);
        }
    }
#pragma unroll
    for (int a = 0; a < TR; ++a) {
        const int64_t r = r0 + tile_row<TR>(ty, a);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int64_t c = c0 + 64 * hb + 4 * tx;
            if (r < out && c < k1)
                *reinterpret_cast<float4*>(Wf + r * in + c) =
                    make_float4(acc[a][4 * hb + 0], acc[a][4 * hb + 1], acc[a][4 * hb + 2],
                                acc[a][4 * hb + 3]);
        }
    }
}

template <int TR>
__global__ __launch_bounds__(256) void k_gptq_update(UpdateArgs p) {
    __shared__ __attribute__((aligned(16))) UpdateLds L;
    update_body<TR>(L, blockIdx.x, blockIdx.y, p);
}

UpdateArgs update_args(float* Wf, int64_t out, int64_t in, int64_t k0, int64_t k1,
                       const float* U, int64_t j0, int nj, const float* E, int64_t ldE) {
    UpdateArgs p;
    p.Wf = Wf;
    p.out = out;
    p.in = in;
    p.k0 = k0;
    p.k1 = k1;
    p.U = U;
    p.j0 = j0;
    p.nj = nj;
    p.E = E;
    p.ldE = ldE;
    p.gx = (uint32_t)((k1 - k0 + 127) / 128);
    return p;
}

// 128-row tiles where they give at least two workgroups per compute unit, else 32-row tiles
// Resident update workgroups of each tile height on this device (compute units times
// workgroups per compute unit), queried once per device.
struct UpdateCapacity {
    std::atomic<int64_t> cap[3] = {0, 0, 0};   // TR = 8, 4, 2
};
constexpr int kMaxDevices = 64;
UpdateCapacity g_update_cap[kMaxDevices];

template <int TR>
int64_t resident(int cus) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gptq_update<TR>, 256, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return (int64_t)per_cu * cus;
}

// Concurrent first calls may both fill an entry; they write the same values, and cap[0] is
// stored last (release) and read first (acquire), so a reader sees a complete entry.
void update_capacity(int64_t cap[3]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    UpdateCapacity& c = g_update_cap[dev];
    if (c.cap[0].load(std::memory_order_acquire) == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 1;
        c.cap[1].store(resident<4>(cus), std::memory_order_relaxed);
        c.cap[2].store(resident<2>(cus), std::memory_order_relaxed);
        c.cap[0].store(resident<8>(cus), std::memory_order_release);
    }
    cap[0] = c.cap[0].load(std::memory_order_acquire);
    cap[1] = c.cap[1].load(std::memory_order_relaxed);
    cap[2] = c.cap[2].load(std::memory_order_relaxed);
}

// Tile height by how evenly the tiles fill the resident workgroups: a grid of 1.25 rounds takes
// as long as 2. Taller tiles read less LDS per fma, so each shorter height must win clearly
// (weights 1, 0.92, 0.8).
void launch_update(const UpdateArgs& p, hipStream_t stream) {
    if (p.k0 >= p.k1 || p.nj <= 0) return;
    int64_t cap[3];
    update_capacity(cap);
    const int trs[3] = {8, 4, 2};
    const double weight[3] = {1.0, 0.92, 0.8};
    int best = 0;
    double best_score = -1.0;
    for (int i = 0; i < 3; ++i) {
        const int64_t tiles = (int64_t)p.gx * ((p.out + 16 * trs[i] - 1) / (16 * trs[i]));
        const int64_t rounds = (tiles + cap[i] - 1) / cap[i];
        const double score = weight[i] * (double)tiles / (double)(rounds * cap[i]);
        if (score > best_score) {
            best_score = score;
            best = i;
        }
    }
    const dim3 grid(p.gx, (uint32_t)((p.out + 16 * trs[best] - 1) / (16 * trs[best])));
    if (best == 0) hipLaunchKernelGGL(k_gptq_update<8>, grid, dim3(256), 0, stream, p);
    else if (best == 1) hipLaunchKernelGGL(k_gptq_update<4>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(k_gptq_update<2>, grid, dim3(256), 0, stream, p);
}

template <bool WMSE, int NWIN>
void launch_outer(const OuterArgs& a, hipStream_t stream) {
    const uint32_t n_outer = (uint32_t)((a.out + kBlockRows - 1) / kBlockRows);
    hipLaunchKernelGGL((k_gptq_outer<WMSE, NWIN>), dim3(n_outer), dim3(256), 0, stream, a);
}

// Outer blocks in order on one stream, each followed by the update of every later column by
// its errors.
template <bool WMSE>
hipError_t launch_blocks(float* Wf, int64_t out, int64_t in, const float* U, const float* h,
                         int lo, int hi, const float* S, uint8_t* scales, uint8_t* packed,
                         float* E, hipStream_t stream) {
    const int n = hi - lo + 1;
    const int64_t ldE = (out + 3) / 4 * 4;
    for (int64_t o0 = 0; o0 < in; o0 += kOB) {
        const int64_t o1 = o0 + kOB < in ? o0 + kOB : in;
        const int oc = (int)(o1 - o0);
        const OuterArgs a{Wf, out, in, o0, oc, U, h, lo, hi, S, scales, packed, E, ldE};
        if (n == 16) launch_outer<WMSE, 16>(a, stream);
        else if (n == 11) launch_outer<WMSE, 11>(a, stream);
        else launch_outer<WMSE, 0>(a, stream);
        launch_update(update_args(Wf, out, in, o1, in, U, o0, oc, E, ldE), stream);
    }
    return hipGetLastError();
}

}  // namespace

size_t gptq_workspace_bytes(int64_t out, int64_t in) {
    return ((size_t)out * (size_t)in * 4 + 255) / 256 * 256 + (size_t)(out + 3) / 4 * 4 * kOB * 4;
}

hipError_t launch_gptq(const void* W, bool bf16, int64_t out, int64_t in, int64_t ldw,
                       const float* U, const float* h, bool wmse, int lo, int hi, const float* S,
                       uint8_t* scales, uint8_t* packed, float* W_final, void* workspace,
                       hipStream_t stream) {
    float* Wf = W_final ? W_final : static_cast<float*>(workspace);
    float* E = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                        ((size_t)out * (size_t)in * 4 + 255) / 256 * 256);
    const int64_t n = out * in;
    const dim3 lgrid((uint32_t)((n + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(k_gptq_load<true>, lgrid, dim3(256), 0, stream,
                           static_cast<const uint8_t*>(W), out, in, ldw * 2, Wf);
    else
        hipLaunchKernelGGL(k_gptq_load<false>, lgrid, dim3(256), 0, stream,
                           static_cast<const uint8_t*>(W), out, in, ldw * 4, Wf);
    if (wmse) return launch_blocks<true>(Wf, out, in, U, h, lo, hi, S, scales, packed, E, stream);
    return launch_blocks<false>(Wf, out, in, U, h, lo, hi, S, scales, packed, E, stream);
}

}  // namespace nvfp4
