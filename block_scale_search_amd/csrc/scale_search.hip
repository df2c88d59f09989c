// Fused per-group E4M3 scale search + E2M1 quantize + pack for gfx950 (the search itself is in
// search_device.h).
#include <hip/hip_runtime.h>

#include "amax_device.h"
#include "device_formats.h"
#include "internal.h"
#include "search_device.h"

namespace nvfp4 {
namespace {

constexpr int kSearchThreads = 256;

template <bool BF16>
__device__ __forceinline__ void load_group(const uint8_t* __restrict__ p, float (&w)[16]) {
    if constexpr (BF16) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        const uint4 b = reinterpret_cast<const uint4*>(p)[1];
        const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[2 * i] = bf16_lo(d[i]);
            w[2 * i + 1] = bf16_hi(d[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = reinterpret_cast<const float4*>(p)[i];
            w[4 * i] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    }
}

// A group's raw bytes: two (bf16) or four (f32) 16-byte units, and their 16 weights.
template <bool BF16>
constexpr int kGroupUnits = BF16 ? 2 : 4;

template <bool BF16>
__device__ __forceinline__ void unpack_group(const uint4 (&a)[kGroupUnits<BF16>], float (&w)[16]) {
    if constexpr (BF16) {
        const uint32_t d[8] = {a[0].x, a[0].y, a[0].z, a[0].w, a[1].x, a[1].y, a[1].z, a[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[2 * i] = bf16_lo(d[i]);
            w[2 * i + 1] = bf16_hi(d[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[4 * i] = __uint_as_float(a[i].x);
            w[4 * i + 1] = __uint_as_float(a[i].y);
            w[4 * i + 2] = __uint_as_float(a[i].z);
            w[4 * i + 3] = __uint_as_float(a[i].w);
        }
    }
}

// The 16 h values of group g of a row (zeros when not needed or not valid).
template <bool NEED_H>
__device__ __forceinline__ void load_h(const float* __restrict__ hm, bool valid, uint32_t g,
                                       float (&h)[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) h[j] = 0.0f;
    if (NEED_H && valid) {
        const float4* hp = reinterpret_cast<const float4*>(hm + (int64_t)g * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = hp[i];
            h[4 * i] = v.x;
            h[4 * i + 1] = v.y;
            h[4 * i + 2] = v.z;
            h[4 * i + 3] = v.w;
        }
    }
}

// The 16 h values of group g of a row, read by every lane (g must be a group of the row); zeros
// when not needed.
template <bool NEED_H>
__device__ __forceinline__ void load_h_at(const float* __restrict__ hm, uint32_t g,
                                          float (&h)[16]) {
    if constexpr (NEED_H) {
        const float4* hp = reinterpret_cast<const float4*>(hm + (int64_t)g * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = hp[i];
            h[4 * i] = v.x;
            h[4 * i + 1] = v.y;
            h[4 * i + 2] = v.z;
            h[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) h[j] = 0.0f;
    }
}

// One lane's group: its 16 weights and, when a rule needs them, its 16 h values.
template <bool BF16, bool NEED_H>
__device__ __forceinline__ void load_inputs(const uint8_t* __restrict__ Wm, int64_t ldw_bytes,
                                            const float* __restrict__ hm, bool valid,
                                            uint32_t row, uint32_t g, float (&w)[16],
                                            float (&h)[16]) {
    if (valid) {
        load_group<BF16>(Wm + (int64_t)row * ldw_bytes + (int64_t)g * (BF16 ? 32 : 64), w);
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) h[j] = 0.0f;
    if (NEED_H && valid) {
        const float4* hp = reinterpret_cast<const float4*>(hm + (int64_t)g * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = hp[i];
            h[4 * i] = v.x;
            h[4 * i + 1] = v.y;
            h[4 * i + 2] = v.z;
            h[4 * i + 3] = v.w;
        }
    }
}

// Quantize once at the chosen code with the weights' signs (tab[0].r = 0 gives signed zeros
// for an all-zero group), pack two nibbles per byte, even element low, and store the group's
// outputs.
__device__ __forceinline__ void emit_group(const float (&w)[16], const float2* __restrict__ tab,
                                           int best_c, float best, int off, int64_t gidx,
                                           const RuleOut& o) {
    const float r = tab[best_c].y;
    uint32_t p0 = 0u, p1 = 0u;
    p0 = e2m1_pack2<0>(p0, w[0] * r, w[1] * r);
    p0 = e2m1_pack2<1>(p0, w[2] * r, w[3] * r);
    p0 = e2m1_pack2<2>(p0, w[4] * r, w[5] * r);
    p0 = e2m1_pack2<3>(p0, w[6] * r, w[7] * r);
    p1 = e2m1_pack2<0>(p1, w[8] * r, w[9] * r);
    p1 = e2m1_pack2<1>(p1, w[10] * r, w[11] * r);
    p1 = e2m1_pack2<2>(p1, w[12] * r, w[13] * r);
    p1 = e2m1_pack2<3>(p1, w[14] * r, w[15] * r);
    reinterpret_cast<uint2*>(o.packed)[gidx] = make_uint2(p0, p1);
    o.scales[gidx] = (uint8_t)best_c;
    if (o.loss) o.loss[gidx] = best;
    if (o.offset) o.offset[gidx] = (int8_t)off;
}

// PROPOSAL: the window is centred on a per-group proposal code center[] instead of the base
// code, and a valid incoming code incoming[] (if given) is scored as well and kept on ties.
// SFP: S is reduced from amax partials in every workgroup (one matrix; workgroup 0 stores it)
// instead of read from S[].
template <bool BF16, bool WMSE, int NWIN, bool PROPOSAL, bool SFP>
__global__ __launch_bounds__(kSearchThreads) void k_scale_search(
    const uint8_t* __restrict__ W, uint32_t out, uint32_t in, uint64_t gpr_magic,
    uint32_t gpr_shift, int64_t ldw_bytes, int64_t stride_w_bytes, const float* __restrict__ hvec, int64_t stride_h,
    int lo, int hi, ScaleSource src, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ packed, float* __restrict__ loss_out, int8_t* __restrict__ off_out,
    const uint8_t* __restrict__ center, const uint8_t* __restrict__ incoming) {
    __shared__ float2 tab[128];
    __shared__ int flag;
    __shared__ uint32_t wmax[kSearchThreads / 64];
    const int64_t batch = blockIdx.y;

    // the group's weights and h are loaded first: S and the code table, which need a
    // workgroup-wide step, are computed while these loads are in flight
    const uint32_t gpr = in >> 4;
    const uint32_t G = out * gpr;
    const uint32_t gi = blockIdx.x * kSearchThreads + threadIdx.x;
    const bool valid = gi < G;
    const uint32_t row = valid ? div_gpr(gi, gpr_magic, gpr_shift) : 0u;
    const uint32_t g = valid ? gi - row * gpr : 0u;

    float w[16], h[16];
    load_inputs<BF16, WMSE>(W + batch * stride_w_bytes, ldw_bytes, hvec + batch * stride_h, valid,
                            row, g, w, h);

    float S;
    if constexpr (SFP) {
        S = scale_from_amax_partials<kSearchThreads>(src.amax_partial, src.n_partial, src.rule,
                                                     wmax);
        if (blockIdx.x == 0 && threadIdx.x == 0 && src.S_out) src.S_out[0] = S;
    } else {
        S = src.S[batch];
    }
    const bool octave_ok = build_table(S, tab, &flag);

    const int b = base_code(w, S);
    const bool live = valid && b > 0;
    const int64_t gidx = batch * (int64_t)G + gi;

    // window centre: the base code, or the group's proposal code clamped to 1..126
    int cen = b;
    int inc = 0;
    if constexpr (PROPOSAL) {
        cen = valid ? min(max((int)center[gidx], 1), 126) : 1;
        inc = (valid && incoming) ? (int)incoming[gidx] : 0;
    }

    // The running best starts at +inf with the first candidate's code, so a group whose every
    // loss overflows keeps its first candidate, as the ascending scan does.
    float best = __builtin_inff();
    int best_c = min(max(cen + lo, 1), 126);
    search_window<WMSE, NWIN>(w, h, tab, octave_ok, live, cen + lo, hi - lo + 1, best, best_c);
    if constexpr (PROPOSAL) {
        // the incoming code comes first in the scan order, so it wins every tie
        if (live && inc >= 1 && inc <= 126) {
            const float2 er = tab[inc];
            const float L = loss_one<WMSE>(w, h, er.x, er.y);
            if (!(best < L)) {
                best = L;
                best_c = inc;
            }
        }
    }
    if (!live) {
        best = 0.0f;
        best_c = 0;
    }

    if (valid)
        emit_group(w, tab, best_c, best, live ? best_c - cen : 0, gidx,
                   RuleOut{scales, packed, loss_out, off_out});
}

// Exhaustive mode (every code 1..126): the three phases of search_device.h's exhaustive search.
// Phase 1 per lane (centre block, pending block counts), phase 2 the workgroup's pending blocks
// dealt over its lanes, phase 3 each lane's result from its LDS slot, then the output.
// Each lane keeps its group's raw bytes in LDS from phase 1 on, and h is read again from memory
// (a few KB per matrix, always cached), so that phase 2 (another lane's group) and the output
// need no registers held through the kernel (the register count, and the waves per SIMD, stay
// those of the windowed kernel) and W is read from HBM once.
// WIN: a 16-code window wlo .. wlo + 15 under the same objective is searched in the same pass.
// The centre block is then placed on the window (codes b + wlo ..), so wherever the window is
// unclipped and normal its ascending scan is the centre block's, and the window's outputs
// (written to ow) come from losses the exhaustive search computes anyway; a lane whose window
// is clipped or reaches the subnormal codes scans its window codes on their own. Without WIN
// the centre block is codes b - 8 .. b + 7.
template <bool BF16, bool WMSE, bool WIN>
__global__ __launch_bounds__(kSearchThreads) void k_scale_search_exhaustive(
    const uint8_t* __restrict__ W, uint32_t out, uint32_t in, uint64_t gpr_magic,
    uint32_t gpr_shift, int64_t ldw_bytes, int64_t stride_w_bytes, const float* __restrict__ hvec,
    int64_t stride_h, const float* __restrict__ S_arr, RuleOut o, int wlo, RuleOut ow) {
    __shared__ float2 tab[128];
    __shared__ int flag;
    __shared__ int first_item[kSearchThreads];             // exclusive prefix of the counts
    __shared__ int owner_info[kSearchThreads];             // per lane: c0 | n_up << 8
    __shared__ uint32_t owner_g[kSearchThreads];           // per lane: its group's column group
    __shared__ int wave_items[kSearchThreads / 64];        // per wave: its lanes' items
    __shared__ unsigned long long slot[kSearchThreads];    // per lane: min (loss, code) key
    constexpr int U = kGroupUnits<BF16>;
    __shared__ uint4 wraw[kSearchThreads * U];              // per lane: its group's raw bytes
    const int64_t batch = blockIdx.y;
    const uint32_t gpr = in >> 4;
    const uint32_t G = out * gpr;
    const uint32_t wave0 = threadIdx.x & ~63u;
    const int lane = threadIdx.x & 63;
    const uint32_t gi = blockIdx.x * kSearchThreads + threadIdx.x;
    const bool valid = gi < G;
    const uint8_t* Wm = W + batch * stride_w_bytes;
    const float* hm = hvec + batch * stride_h;
    const float S = S_arr[batch];

    // phase 1
    int b, c0 = 8, n_up = 0, n_dn = 0;
    bool live;
    {
        const uint32_t row = valid ? div_gpr(gi, gpr_magic, gpr_shift) : 0u;
        const uint32_t g = valid ? gi - row * gpr : 0u;
        uint4 a[U];
        const uint4* src = reinterpret_cast<const uint4*>(Wm + (int64_t)row * ldw_bytes +
                                                          (int64_t)g * (BF16 ? 32 : 64));
#pragma unroll
        for (int k = 0; k < U; ++k) a[k] = valid ? src[k] : make_uint4(0u, 0u, 0u, 0u);
        float w[16], h[16];
        load_h<WMSE>(hm, valid, g, h);
#pragma unroll
        for (int k = 0; k < U; ++k) wraw[threadIdx.x * U + k] = a[k];
        owner_g[threadIdx.x] = g;
        unpack_group<BF16>(a, w);
        const bool octave_ok = build_table(S, tab, &flag);
        b = base_code(w, S);
        live = valid && b > 0;
        float best = __builtin_inff();
        int best_c = 1;
        if (__any(live)) {
            c0 = centre_scan<WMSE>(w, h, tab, octave_ok, live, b, WIN ? wlo : -8, best, best_c);
            if constexpr (WIN) {
                float wb = best;
                int wc = best_c;
                const bool own = live && c0 != b + wlo;
                if (__any(own)) {
                    // the window's codes clamp(b + wlo + p, 1, 126), p = 0..15, ascending
                    float wb2 = __builtin_inff();
                    int wc2 = min(max(b + wlo, 1), 126);
                    search_window<WMSE, 0>(w, h, tab, false, own, b + wlo, 16, wb2, wc2);
                    wb = own ? wb2 : wb;
                    wc = own ? wc2 : wc;
                }
                if (valid)
                    emit_group(w, tab, live ? wc : 0, live ? wb : 0.0f, live ? wc - b : 0,
                               batch * (int64_t)G + gi, ow);
            }
            pending_blocks<WMSE>(w, h, tab, live, c0, best, n_up, n_dn);
            // +inf with code 1: a group whose every loss overflows keeps code 1, as the
            // ascending scan over all codes does
            if (!(best < __builtin_inff())) best_c = 1;
        } else if constexpr (WIN) {
            if (valid) emit_group(w, tab, 0, 0.0f, 0, batch * (int64_t)G + gi, ow);
        }
        slot[threadIdx.x] = loss_key(best, best_c);
    }

    // phase 2: the workgroup's pending blocks in item order (lane by lane), 64 items per wave
    // and round, the waves taking rounds in turn
    const int n = n_up + n_dn;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wave_items[threadIdx.x >> 6] = incl;
    owner_info[threadIdx.x] = c0 | (n_up << 8);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < kSearchThreads / 64; ++q) {
        const int v = wave_items[q];
        before += q < (int)(threadIdx.x >> 6) ? v : 0;
        total += v;
    }
    first_item[threadIdx.x] = before + incl - n;
    __syncthreads();
    for (int t0 = (int)wave0; t0 < total; t0 += kSearchThreads) {
        const int t = t0 + lane;
        const bool has = t < total;
        // owner: the last lane whose first item is <= t (lanes without items share the next
        // lane's first item and are passed over)
        int j = 0;
#pragma unroll
        for (int step = kSearchThreads / 2; step >= 1; step >>= 1)
            if (first_item[j + step] <= t) j += step;
        const int owner = has ? j : (int)threadIdx.x;
        const int k = t - first_item[owner];
        const int info = owner_info[owner];
        const int o_c0 = info & 255, o_up = info >> 8;
        // block k of the owner: upward from o_c0 + 16, then downward from o_c0 - 1
        const int first = !has ? 8
                               : (k < o_up ? o_c0 + 16 + kBlockCodes * k
                                           : o_c0 - kBlockCodes * (k - o_up + 1));
        const uint32_t og = owner_g[owner];   // 0 for lanes past the last group
        uint4 a[U];
#pragma unroll
        for (int q = 0; q < U; ++q) a[q] = wraw[owner * U + q];
        float w[16], h[16];
        unpack_group<BF16>(a, w);
        load_h_at<WMSE>(hm, og, h);      // idle lanes read their own group's h and use none of it
        // every block holds at least one code in 1..126, the first of them max(first, 1)
        float bl = __builtin_inff();
        int cl = max(first, 1);
        scan_codes<WMSE, kBlockCodes>(w, h, tab, first, bl, cl);
        if (has) atomicMin(&slot[owner], (unsigned long long)loss_key(bl, cl));
    }
    __syncthreads();

    // phase 3
    const uint64_t key = slot[threadIdx.x];
    float best = key_loss(key);
    int best_c = key_code(key);
    if (!live) {
        best = 0.0f;
        best_c = 0;
    }
    if (valid) {
        uint4 a[U];
#pragma unroll
        for (int q = 0; q < U; ++q) a[q] = wraw[threadIdx.x * U + q];
        float w[16];
        unpack_group<BF16>(a, w);
        emit_group(w, tab, best_c, best, live ? best_c - b : 0, batch * (int64_t)G + gi, o);
    }
}

// Work count of the exhaustive search on the same inputs: per group with a nonzero base code,
// the 16 codes of its centre block (centre offset clo) and the codes 1..126 of every pending
// block that its lower bounds keep, summed over the launch and added to *count. It runs the
// exhaustive kernel's phase-1 code, so the decisions are the same.
template <bool BF16, bool WMSE>
__global__ __launch_bounds__(kSearchThreads) void k_exhaustive_scored(
    const uint8_t* __restrict__ W, uint32_t out, uint32_t in, uint64_t gpr_magic,
    uint32_t gpr_shift, int64_t ldw_bytes, int64_t stride_w_bytes, const float* __restrict__ hvec,
    int64_t stride_h, const float* __restrict__ S_arr, int clo,
    unsigned long long* __restrict__ count) {
    __shared__ float2 tab[128];
    __shared__ int flag;
    __shared__ uint32_t wsum[kSearchThreads / 64];
    const int64_t batch = blockIdx.y;
    const uint32_t gpr = in >> 4;
    const uint32_t G = out * gpr;
    const uint32_t gi = blockIdx.x * kSearchThreads + threadIdx.x;
    const bool valid = gi < G;
    const uint32_t row = valid ? div_gpr(gi, gpr_magic, gpr_shift) : 0u;
    const uint32_t g = valid ? gi - row * gpr : 0u;
    float w[16], h[16];
    load_inputs<BF16, WMSE>(W + batch * stride_w_bytes, ldw_bytes, hvec + batch * stride_h, valid,
                            row, g, w, h);
    const float S = S_arr[batch];
    const bool octave_ok = build_table(S, tab, &flag);
    const int b = base_code(w, S);
    const bool live = valid && b > 0;
    uint32_t n = 0;
    if (__any(live)) {
        float best;
        int best_c, n_up, n_dn;
        const int c0 = centre_scan<WMSE>(w, h, tab, octave_ok, live, b, clo, best, best_c);
        pending_blocks<WMSE>(w, h, tab, live, c0, best, n_up, n_dn);
        const int up = c0 + 16, dn = c0 - 1;
        if (live) n = 16 + (min(up + kBlockCodes * n_up, 127) - up) + min(kBlockCodes * n_dn, dn);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = n;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int k = 0; k < kSearchThreads / 64; ++k) t += wsum[k];
        atomicAdd(count, (unsigned long long)t);
    }
}

// Two windowed rules on one read of each group (bf16 W): the weights, h, S, the code table and
// the base code are shared, and each rule's search and outputs are those of k_scale_search.
template <bool WA, int NA, bool WB, int NB>
__global__ __launch_bounds__(kSearchThreads) void k_scale_search_pair(
    const uint8_t* __restrict__ W, uint32_t out, uint32_t in, uint64_t gpr_magic,
    uint32_t gpr_shift, int64_t ldw_bytes, int64_t stride_w_bytes, const float* __restrict__ hvec,
    int64_t stride_h, const float* __restrict__ S_arr, int loA, int loB, RuleOut A, RuleOut B) {
    __shared__ float2 tab[128];
    __shared__ int flag;
    const int64_t batch = blockIdx.y;
    const uint32_t gpr = in >> 4;
    const uint32_t G = out * gpr;
    const uint32_t gi = blockIdx.x * kSearchThreads + threadIdx.x;
    const bool valid = gi < G;
    const uint32_t row = valid ? div_gpr(gi, gpr_magic, gpr_shift) : 0u;
    const uint32_t g = valid ? gi - row * gpr : 0u;
    float w[16], h[16];
    load_inputs<true, WA || WB>(W + batch * stride_w_bytes, ldw_bytes, hvec + batch * stride_h,
                                valid, row, g, w, h);
    const float S = S_arr[batch];
    const bool octave_ok = build_table(S, tab, &flag);
    const int b = base_code(w, S);
    const bool live = valid && b > 0;
    const int64_t gidx = batch * (int64_t)G + gi;
    {
        float best = __builtin_inff();
        int best_c = min(max(b + loA, 1), 126);
        search_window<WA, NA>(w, h, tab, octave_ok, live, b + loA, NA, best, best_c);
        if (valid)
            emit_group(w, tab, live ? best_c : 0, live ? best : 0.0f, live ? best_c - b : 0,
                       gidx, A);
    }
    {
        float best = __builtin_inff();
        int best_c = min(max(b + loB, 1), 126);
        search_window<WB, NB>(w, h, tab, octave_ok, live, b + loB, NB, best, best_c);
        if (valid)
            emit_group(w, tab, live ? best_c : 0, live ? best : 0.0f, live ? best_c - b : 0,
                       gidx, B);
    }
}

// Two windowed rules (bf16 W) where one window of 16 codes (outer, objective WO, offsets
// loO .. loO + 15) contains the other (inner, objective WI, codes base + loO + OFFB ..
// + NB - 1): where every lane's outer window is normal and unclipped, each 16-code block is
// scanned once for both (scan_block_two: shared multiply, conversions and residuals). Other
// waves run the two windows one after the other, as k_scale_search_pair does. Each rule's
// outputs are those of k_scale_search.
template <bool WO, bool WI, int OFFB, int NB>
__global__ __launch_bounds__(kSearchThreads) __attribute__((amdgpu_waves_per_eu(7, 8))) void
k_scale_search_nested(
    const uint8_t* __restrict__ W, uint32_t out, uint32_t in, uint64_t gpr_magic,
    uint32_t gpr_shift, int64_t ldw_bytes, int64_t stride_w_bytes, const float* __restrict__ hvec,
    int64_t stride_h, const float* __restrict__ S_arr, int loO, RuleOut O, RuleOut I) {
    __shared__ float2 tab[128];
    __shared__ int flag;
    const int64_t batch = blockIdx.y;
    const uint32_t gpr = in >> 4;
    const uint32_t G = out * gpr;
    const uint32_t gi = blockIdx.x * kSearchThreads + threadIdx.x;
    const bool valid = gi < G;
    const uint32_t row = valid ? div_gpr(gi, gpr_magic, gpr_shift) : 0u;
    const uint32_t g = valid ? gi - row * gpr : 0u;
    float w[16], h[16];
    load_inputs<true, WO || WI>(W + batch * stride_w_bytes, ldw_bytes, hvec + batch * stride_h,
                                valid, row, g, w, h);
    const float S = S_arr[batch];
    const bool octave_ok = build_table(S, tab, &flag);
    const int b = base_code(w, S);
    const bool live = valid && b > 0;
    const int64_t gidx = batch * (int64_t)G + gi;
    const int loI = loO + OFFB;
    float bestO = __builtin_inff(), bestI = __builtin_inff();
    int cO = min(max(b + loO, 1), 126), cI = min(max(b + loI, 1), 126);
    // idle lanes score the dummy codes 8 .. 23
    const bool lane_fast = !live || (b + loO >= 8 && b + loO + 15 <= 126);
    if (octave_ok && __all(lane_fast)) {
        const int c0 = live ? b + loO : 8;
        scan_block_two<WO, WI, OFFB, NB>(w, h, tab + c0, c0, bestO, cO, bestI, cI);
    } else {
        search_window<WO, 16>(w, h, tab, octave_ok, live, b + loO, 16, bestO, cO);
        search_window<WI, NB>(w, h, tab, octave_ok, live, b + loI, NB, bestI, cI);
    }
    if (valid) {
        emit_group(w, tab, live ? cO : 0, live ? bestO : 0.0f, live ? cO - b : 0, gidx, O);
        emit_group(w, tab, live ? cI : 0, live ? bestI : 0.0f, live ? cI - b : 0, gidx, I);
    }
}

}  // namespace

namespace {

struct SearchArgs {
    const uint8_t* W;
    uint32_t out, in;
    uint64_t magic;
    uint32_t shift;
    int64_t ldw_bytes, stride_w_bytes;
    const float* h;
    int64_t stride_h;
    int lo, hi;
    ScaleSource src;
    uint8_t *scales, *packed;
    float* loss;
    int8_t* offset;
    const uint8_t *center, *incoming;
};

template <bool B, bool M, int N, bool P, bool SFP>
void launch_one(const SearchArgs& a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((k_scale_search<B, M, N, P, SFP>), grid, dim3(kSearchThreads), 0, stream,
                       a.W, a.out, a.in, a.magic, a.shift, a.ldw_bytes, a.stride_w_bytes, a.h,
                       a.stride_h, a.lo, a.hi, a.src, a.scales, a.packed, a.loss,
                       a.offset, a.center, a.incoming);
}

// window length at compile time where it is one of the pages' windows (16 and 11 codes) or a
// half-window of 4 around a proposal (9 codes); 0 = run-time length or exhaustive
template <bool B, bool M>
void launch_modes(const SearchArgs& a, int nwin, bool proposal, bool sfp, dim3 grid,
                  hipStream_t stream) {
    if (proposal) {
        if (nwin == 9) launch_one<B, M, 9, true, false>(a, grid, stream);
        else launch_one<B, M, 0, true, false>(a, grid, stream);
    } else if (sfp) {
        if (nwin == 16) launch_one<B, M, 16, false, true>(a, grid, stream);
        else if (nwin == 11) launch_one<B, M, 11, false, true>(a, grid, stream);
        else launch_one<B, M, 0, false, true>(a, grid, stream);
    } else {
        if (nwin == 16) launch_one<B, M, 16, false, false>(a, grid, stream);
        else if (nwin == 11) launch_one<B, M, 11, false, false>(a, grid, stream);
        else launch_one<B, M, 0, false, false>(a, grid, stream);
    }
}

template <bool WA, int NA, bool WB, int NB>
void launch_pair_t(const SearchArgs& a, const float* S, int loA, int loB, const RuleOut& A,
                   const RuleOut& B, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((k_scale_search_pair<WA, NA, WB, NB>), grid, dim3(kSearchThreads), 0,
                       stream, a.W, a.out, a.in, a.magic, a.shift, a.ldw_bytes, a.stride_w_bytes,
                       a.h, a.stride_h, S, loA, loB, A, B);
}

template <bool WO, bool WI, int OFFB, int NB>
void launch_nested_t(const SearchArgs& a, const float* S, const SearchRule& outer,
                     const SearchRule& inner, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((k_scale_search_nested<WO, WI, OFFB, NB>), grid, dim3(kSearchThreads), 0,
                       stream, a.W, a.out, a.in, a.magic, a.shift, a.ldw_bytes, a.stride_w_bytes,
                       a.h, a.stride_h, S, outer.lo, outer.out, inner.out);
}

// Two windowed rules whose one window of 16 codes holds the other, in one of the compiled
// shapes: the inner window of 11 codes ending where the outer one ends (MSE [-3,7] inside
// [-8,7]), or the same 16 codes. Returns false (nothing launched) for other pairs.
bool launch_nested(const SearchArgs& a, const float* S, const SearchRule& r, const SearchRule& q,
                   dim3 grid, hipStream_t stream) {
    const int nr = r.hi - r.lo + 1, nq = q.hi - q.lo + 1;
    const bool r_outer = nr == 16 && (nq != 16 || !r.wmse || q.wmse);
    const SearchRule& outer = r_outer ? r : q;
    const SearchRule& inner = r_outer ? q : r;
    const int n_in = inner.hi - inner.lo + 1;
    const int off = inner.lo - outer.lo;
    if (outer.hi - outer.lo + 1 != 16) return false;
#define NVFP4_NEST(OFF, N)                                                                     \
    if (off == OFF && n_in == N) {                                                             \
        if (outer.wmse && inner.wmse) launch_nested_t<true, true, OFF, N>(a, S, outer, inner, grid, stream);   \
        else if (outer.wmse) launch_nested_t<true, false, OFF, N>(a, S, outer, inner, grid, stream);           \
        else if (inner.wmse) launch_nested_t<false, true, OFF, N>(a, S, outer, inner, grid, stream);           \
        else launch_nested_t<false, false, OFF, N>(a, S, outer, inner, grid, stream);                          \
        return true;                                                                           \
    }
    NVFP4_NEST(5, 11)
    NVFP4_NEST(0, 16)
#undef NVFP4_NEST
    return false;
}

template <bool WA, int NA>
void launch_pair_b(const SearchArgs& a, const float* S, const SearchRule& ra,
                   const SearchRule& rb, dim3 grid, hipStream_t stream) {
    const int nb = rb.hi - rb.lo + 1;
    if (rb.wmse) {
        if (nb == 16) launch_pair_t<WA, NA, true, 16>(a, S, ra.lo, rb.lo, ra.out, rb.out, grid, stream);
        else launch_pair_t<WA, NA, true, 11>(a, S, ra.lo, rb.lo, ra.out, rb.out, grid, stream);
    } else {
        if (nb == 16) launch_pair_t<WA, NA, false, 16>(a, S, ra.lo, rb.lo, ra.out, rb.out, grid, stream);
        else launch_pair_t<WA, NA, false, 11>(a, S, ra.lo, rb.lo, ra.out, rb.out, grid, stream);
    }
}

// rules with a compiled pair kernel: windows of 11 or 16 codes
bool pairable(const SearchRule& r) {
    const int n = r.hi - r.lo + 1;
    return !r.exhaustive && (n == 11 || n == 16);
}

// a 16-code window and an exhaustive rule of the same objective, in either order: one pass
bool fusable(const SearchRule& r, const SearchRule& q) {
    const SearchRule& win = r.exhaustive ? q : r;
    const SearchRule& exh = r.exhaustive ? r : q;
    return exh.exhaustive && !win.exhaustive && win.hi - win.lo + 1 == 16 && win.wmse == exh.wmse;
}

template <bool B, bool M>
void launch_fused_t(const SearchArgs& a, const float* S, int wlo, const RuleOut& exh,
                    const RuleOut& win, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((k_scale_search_exhaustive<B, M, true>), grid, dim3(kSearchThreads), 0,
                       stream, a.W, a.out, a.in, a.magic, a.shift, a.ldw_bytes, a.stride_w_bytes,
                       a.h, a.stride_h, S, exh, wlo, win);
}

}  // namespace

hipError_t launch_scale_search_rules(const void* W, bool bf16, int64_t batch, int64_t out,
                                     int64_t in, int64_t ldw, int64_t stride_w, const float* h,
                                     int64_t stride_h, const float* S, const SearchRule* rules,
                                     int n_rules, hipStream_t stream) {
    const int64_t gpr = in / 16;
    const int64_t G = out * gpr;
    SearchArgs a{};
    gpr_divisor(gpr, a.magic, a.shift);
    const int esz = bf16 ? 2 : 4;
    a.W = static_cast<const uint8_t*>(W);
    a.out = (uint32_t)out;
    a.in = (uint32_t)in;
    a.ldw_bytes = ldw * esz;
    a.stride_w_bytes = stride_w * esz;
    a.h = h;
    a.stride_h = stride_h;
    const dim3 grid((uint32_t)((G + kSearchThreads - 1) / kSearchThreads), (uint32_t)batch);
    ScaleSource src;
    src.S = S;
    for (int i = 0; i < n_rules;) {
        const SearchRule& r = rules[i];
        if (bf16 && i + 1 < n_rules && pairable(r) && pairable(rules[i + 1])) {
            const SearchRule& q = rules[i + 1];
            if (launch_nested(a, S, r, q, grid, stream)) {
                i += 2;
                continue;
            }
            const int na = r.hi - r.lo + 1;
            if (r.wmse) {
                if (na == 16) launch_pair_b<true, 16>(a, S, r, q, grid, stream);
                else launch_pair_b<true, 11>(a, S, r, q, grid, stream);
            } else {
                if (na == 16) launch_pair_b<false, 16>(a, S, r, q, grid, stream);
                else launch_pair_b<false, 11>(a, S, r, q, grid, stream);
            }
            i += 2;
        } else if (i + 1 < n_rules && fusable(r, rules[i + 1])) {
            const SearchRule& win = r.exhaustive ? rules[i + 1] : r;
            const SearchRule& exh = r.exhaustive ? r : rules[i + 1];
            if (bf16) {
                if (r.wmse) launch_fused_t<true, true>(a, S, win.lo, exh.out, win.out, grid, stream);
                else launch_fused_t<true, false>(a, S, win.lo, exh.out, win.out, grid, stream);
            } else {
                if (r.wmse) launch_fused_t<false, true>(a, S, win.lo, exh.out, win.out, grid, stream);
                else launch_fused_t<false, false>(a, S, win.lo, exh.out, win.out, grid, stream);
            }
            i += 2;
        } else {
            const hipError_t e = launch_scale_search(
                W, bf16, batch, out, in, ldw, stride_w, r.wmse ? h : nullptr, r.wmse ? stride_h : 0,
                r.wmse, r.lo, r.hi, r.exhaustive, src, r.out.scales, r.out.packed, r.out.loss,
                r.out.offset, nullptr, nullptr, stream);
            if (e != hipSuccess) return e;
            i += 1;
        }
    }
    return hipGetLastError();
}

hipError_t launch_scale_search(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, const float* h, int64_t stride_h,
                               bool wmse, int lo, int hi, bool exhaustive, ScaleSource src,
                               uint8_t* scales, uint8_t* packed, float* loss, int8_t* offset,
                               const uint8_t* center, const uint8_t* incoming,
                               hipStream_t stream) {
    const int64_t gpr = in / 16;
    const int64_t G = out * gpr;
    SearchArgs a;
    gpr_divisor(gpr, a.magic, a.shift);
    const int esz = bf16 ? 2 : 4;
    a.W = static_cast<const uint8_t*>(W);
    a.out = (uint32_t)out;
    a.in = (uint32_t)in;
    a.ldw_bytes = ldw * esz;
    a.stride_w_bytes = stride_w * esz;
    a.h = h;
    a.stride_h = stride_h;
    a.lo = lo;
    a.hi = hi;
    a.src = src;
    a.scales = scales;
    a.packed = packed;
    a.loss = loss;
    a.offset = offset;
    a.center = center;
    a.incoming = incoming;
    const dim3 grid((uint32_t)((G + kSearchThreads - 1) / kSearchThreads), (uint32_t)batch);
    const int n = hi - lo + 1;
    const bool proposal = center != nullptr;
    const bool sfp = src.amax_partial != nullptr;
    if (exhaustive) {
        // every code 1..126 around the base code, with S given (no proposal, no fused S)
        if (proposal || sfp || src.S == nullptr) return hipErrorInvalidValue;
        const RuleOut o{scales, packed, loss, offset};
#define NVFP4_EXH(B, M)                                                                        \
        hipLaunchKernelGGL((k_scale_search_exhaustive<B, M, false>), grid, dim3(kSearchThreads), \
                           0, stream, a.W, a.out, a.in, a.magic, a.shift, a.ldw_bytes,         \
                           a.stride_w_bytes, a.h, a.stride_h, src.S, o, 0, RuleOut{})
        if (bf16) {
            if (wmse) NVFP4_EXH(true, true); else NVFP4_EXH(true, false);
        } else {
            if (wmse) NVFP4_EXH(false, true); else NVFP4_EXH(false, false);
        }
#undef NVFP4_EXH
        return hipGetLastError();
    }
    const int nwin = n == 16 || n == 11 || n == 9 ? n : 0;
    if (bf16) {
        if (wmse) launch_modes<true, true>(a, nwin, proposal, sfp, grid, stream);
        else launch_modes<true, false>(a, nwin, proposal, sfp, grid, stream);
    } else {
        if (wmse) launch_modes<false, true>(a, nwin, proposal, sfp, grid, stream);
        else launch_modes<false, false>(a, nwin, proposal, sfp, grid, stream);
    }
    return hipGetLastError();
}

hipError_t launch_exhaustive_scored(const void* W, bool bf16, int64_t batch, int64_t out,
                                   int64_t in, int64_t ldw, int64_t stride_w, const float* h,
                                   int64_t stride_h, bool wmse, int clo, const float* S,
                                   uint64_t* count, hipStream_t stream) {
    const int64_t gpr = in / 16;
    const int64_t G = out * gpr;
    uint64_t magic;
    uint32_t shift;
    gpr_divisor(gpr, magic, shift);
    const int esz = bf16 ? 2 : 4;
    const dim3 grid((uint32_t)((G + kSearchThreads - 1) / kSearchThreads), (uint32_t)batch);
    auto* c = reinterpret_cast<unsigned long long*>(count);
#define NVFP4_SCORED(B, M)                                                                     \
    hipLaunchKernelGGL((k_exhaustive_scored<B, M>), grid, dim3(kSearchThreads), 0, stream,     \
                       static_cast<const uint8_t*>(W), (uint32_t)out, (uint32_t)in, magic,    \
                       shift, ldw * esz, stride_w * esz, h, stride_h, S, clo, c)
    if (bf16) {
        if (wmse) NVFP4_SCORED(true, true); else NVFP4_SCORED(true, false);
    } else {
        if (wmse) NVFP4_SCORED(false, true); else NVFP4_SCORED(false, false);
    }
#undef NVFP4_SCORED
    return hipGetLastError();
}

}  // namespace nvfp4
