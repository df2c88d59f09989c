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
    int lo, int hi, int exhaustive, ScaleSource src, uint8_t* __restrict__ scales,
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
    int best_c = exhaustive ? 1 : min(max(cen + lo, 1), 126);
    if (exhaustive) {
        if (__any(live)) search_all<WMSE>(w, h, tab, octave_ok, live, b, best, best_c);
    } else {
        search_window<WMSE, NWIN>(w, h, tab, octave_ok, live, cen + lo, hi - lo + 1, best, best_c);
    }
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
    int lo, hi, exhaustive;
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
                       a.stride_h, a.lo, a.hi, a.exhaustive, a.src, a.scales, a.packed, a.loss,
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

}  // namespace

hipError_t launch_scale_search_rules(const void* W, bool bf16, int64_t batch, int64_t out,
                                     int64_t in, int64_t ldw, int64_t stride_w, const float* h,
                                     int64_t stride_h, const float* S, const SearchRule* rules,
                                     int n_rules, hipStream_t stream) {
    const int64_t gpr = in / 16;
    const int64_t G = out * gpr;
    SearchArgs a{};
    gpr_divisor(gpr, a.magic, a.shift);
    a.W = static_cast<const uint8_t*>(W);
    a.out = (uint32_t)out;
    a.in = (uint32_t)in;
    a.ldw_bytes = ldw * 2;
    a.stride_w_bytes = stride_w * 2;
    a.h = h;
    a.stride_h = stride_h;
    const dim3 grid((uint32_t)((G + kSearchThreads - 1) / kSearchThreads), (uint32_t)batch);
    ScaleSource src;
    src.S = S;
    for (int i = 0; i < n_rules;) {
        const SearchRule& r = rules[i];
        if (bf16 && i + 1 < n_rules && pairable(r) && pairable(rules[i + 1])) {
            const SearchRule& q = rules[i + 1];
            const int na = r.hi - r.lo + 1;
            if (r.wmse) {
                if (na == 16) launch_pair_b<true, 16>(a, S, r, q, grid, stream);
                else launch_pair_b<true, 11>(a, S, r, q, grid, stream);
            } else {
                if (na == 16) launch_pair_b<false, 16>(a, S, r, q, grid, stream);
                else launch_pair_b<false, 11>(a, S, r, q, grid, stream);
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
    a.exhaustive = exhaustive ? 1 : 0;
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
    const int nwin = exhaustive ? 0 : (n == 16 || n == 11 || n == 9 ? n : 0);
    if (bf16) {
        if (wmse) launch_modes<true, true>(a, nwin, proposal, sfp, grid, stream);
        else launch_modes<true, false>(a, nwin, proposal, sfp, grid, stream);
    } else {
        if (wmse) launch_modes<false, true>(a, nwin, proposal, sfp, grid, stream);
        else launch_modes<false, false>(a, nwin, proposal, sfp, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
