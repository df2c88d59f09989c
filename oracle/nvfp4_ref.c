/*
 * NVFP4 per-group E4M3 block-scale search: plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the independent reference that the GPU library is
 * checked against. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, table or constant generator with the GPU library, and the
 * GPU library never calls it.
 *
 * It is written to be read against the pages, not to be fast: every step is a direct loop,
 * every rounding decision is an explicit comparison. Floating point follows the precisions the
 * method fixes: the FP4 values are E2M1, the local scales are E4M3, the global scale and the
 * reconstruction loss are binary32. The diagonal Hessian is summed in binary64 and rounded once.
 * Build with `-O2 -ffp-contract=off` and without fast-math, so that every float expression below
 * is one IEEE-754 binary32 operation with round-to-nearest-even.
 *
 * Sources (web pages on NVFP4 scale refinement):
 *   [HS] "H-Scale: Hessian-Guided Scale Refinement for NVFP4 Sub-Byte LLM Inference"
 *        (paperlayer.ai summary): §3 Method, §4 Experiments, App. B Implementation Pseudocode.
 *   [SS] "Technical Summary: ScaleSweep" (gist.science): Problem Statement, Methodology §1-§3.
 *   [SR] "Replay the Curvature: Accurate and Scalable NVFP4 Quantization for Large Language
 *        Model Inference" (paperlayer.ai summary): §1, §4.1.1, §4.1.4, App. D.2.
 *
 * Readings where the pages are silent (each one is listed with its reason in the design notes):
 *   - E2M1 levels {0, 0.5, 1, 1.5, 2, 3, 4, 6}; round to nearest, ties to the even code,
 *     values above 6 saturate to 6.
 *   - E4M3 is the variant with 126 positive finite codes (0x01..0x7E, max 448); the base scale
 *     is rounded to nearest-even and saturates at 448; a base that rounds to 0 becomes code 1.
 *   - Global scale S = amax / (6*448) ("AMAX_448") or amax / (6*256) ("AMAX_256", [SS] §2),
 *     or a caller-given S. S = 1 for an all-zero tensor.
 *   - Effective scale eff[c] = fl(S * dec(c)); its reciprocal r[c] = fl(1 / eff[c]); a weight is
 *     normalised as fl(|w| * r[c]).
 *   - Residual d = fma(-q, eff, |w|); the weighted squares are summed in a fixed tree: four
 *     fma chains over the element quads 4k..4k+3, then (P0 + P1) + (P2 + P3); the first
 *     strictly smaller loss wins, so ties go to the lowest offset.
 *   - Nibble = sign(w) << 3 | E2M1 index; two nibbles per byte, low nibble first.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { REF_OK = 0, REF_ERR_ARG = 1, REF_ERR_NONFINITE = 2 };
enum { REF_F32 = 0, REF_BF16 = 1 };
enum { REF_MSE = 0, REF_WMSE = 1 };
enum { REF_GS_AMAX_448 = 0, REF_GS_AMAX_256 = 1, REF_GS_GIVEN = 2 };

/* ------------------------------------------------------------------------------------------ */
/* Element formats.                                                                            */
/* ------------------------------------------------------------------------------------------ */

/* FP4 E2M1 magnitudes, indexed by the 3 low bits of the code ([SS] Problem Statement names
 * E2M1; [SR] §4.1.1: the group quantizer rounds normalised values to the E2M1 levels). */
static const float E2M1_LEVEL[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float ref_e2m1_level(int index) { return E2M1_LEVEL[index & 7]; }

/* Round a non-negative binary32 value to the nearest E2M1 level; a value exactly halfway between
 * two levels goes to the one with the even index; anything above 6 becomes 6.
 * The ladder walks the seven midpoints between neighbouring levels (all exact in binary32). */
int ref_e2m1_index(float x)
{
    int index = 0;
    for (int i = 0; i < 7; ++i) {
        float mid = 0.5f * (E2M1_LEVEL[i] + E2M1_LEVEL[i + 1]);
        int upper_is_even = ((i + 1) % 2) == 0;
        if (x > mid || (x == mid && upper_is_even)) index = i + 1;
    }
    return index;
}

/* Value of an E4M3 code 0..126 (sign 0, 4 exponent bits with bias 7, 3 mantissa bits).
 * Codes 1..7 are subnormal (c * 2^-9); 0x7F is NaN and is never a scale ([SS] §2: 126 positive
 * finite values). Exact in double. */
double ref_e4m3_value(int code)
{
    if (code < 8) return (double)code * ldexp(1.0, -9);
    return (1.0 + (double)(code & 7) / 8.0) * ldexp(1.0, (code >> 3) - 7);
}

/* E4M3 code nearest to s >= 0 ([SS] §2: the base scale is the FP8-rounded block maximum).
 * Ties go to the even code; values at or above 448 saturate to code 126. */
int ref_e4m3_encode(float s)
{
    if (s >= 448.0f) return 126;
    int c = 0; /* largest code with value <= s */
    while (c < 126 && ref_e4m3_value(c + 1) <= (double)s) ++c;
    if (c == 126) return 126;
    double lo = ref_e4m3_value(c), hi = ref_e4m3_value(c + 1);
    double mid = 0.5 * (lo + hi);
    if ((double)s > mid) return c + 1;
    if ((double)s < mid) return c;
    return (c % 2 == 0) ? c : c + 1;
}

static float load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == REF_F32) return ((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16; /* bf16 -> binary32, exact */
    float v;
    memcpy(&v, &bits, sizeof v);
    return v;
}

/* ------------------------------------------------------------------------------------------ */
/* Step 1: diagonal second-order weight.                                                       */
/* h_j = sum_t x_tj^2 ([HS] App. B: h = diag(X^T X); [SR] §3: H = X X^T in its notation).     */
/* Summed in binary64 in token order t = 0, 1, ...; each square of a bf16/binary32 value is   */
/* exact in binary64. `acc` is the running sum (kept across token chunks when accumulate=1).   */
/* ------------------------------------------------------------------------------------------ */
int ref_diag_hessian(const void* X, int dtype, int64_t tokens, int64_t in, int64_t ldx,
                     double* acc, int accumulate, float* h_out, int nthreads)
{
    if (!X && tokens > 0) return REF_ERR_ARG;
    if (!acc || in < 0 || tokens < 0 || ldx < in) return REF_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(| : bad)
    for (int64_t j0 = 0; j0 < in; j0 += 64) {
        int64_t j1 = j0 + 64 < in ? j0 + 64 : in;
        for (int64_t j = j0; j < j1; ++j)
            if (!accumulate) acc[j] = 0.0;
        for (int64_t t = 0; t < tokens; ++t) {
            for (int64_t j = j0; j < j1; ++j) {
                double x = (double)load_elem(X, dtype, t * ldx + j);
                if (!isfinite(x)) bad = 1;
                acc[j] = acc[j] + x * x;
            }
        }
        if (h_out)
            for (int64_t j = j0; j < j1; ++j) h_out[j] = (float)acc[j];
    }
    return bad ? REF_ERR_NONFINITE : REF_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Step 2: global FP32 scale ([HS] §3: tensor-level FP32 global scale; [SS] §2:                */
/* S = max|x| / (256 * 6)).                                                                    */
/* ------------------------------------------------------------------------------------------ */
int ref_global_scale(const void* W, int dtype, int64_t out, int64_t in, int64_t ldw, int rule,
                     float given, float* S)
{
    if (!S || out < 0 || in < 0 || ldw < in || (!W && out * in > 0)) return REF_ERR_ARG;
    if (rule == REF_GS_GIVEN) {
        *S = given;
        return REF_OK;
    }
    if (rule != REF_GS_AMAX_448 && rule != REF_GS_AMAX_256) return REF_ERR_ARG;
    float amax = 0.0f;
    for (int64_t o = 0; o < out; ++o)
        for (int64_t i = 0; i < in; ++i) {
            float a = fabsf(load_elem(W, dtype, o * ldw + i));
            if (!isfinite(a)) return REF_ERR_NONFINITE;
            if (a > amax) amax = a;
        }
    if (amax == 0.0f) {
        *S = 1.0f;
        return REF_OK;
    }
    *S = amax / (rule == REF_GS_AMAX_448 ? 2688.0f : 1536.0f);
    return REF_OK;
}

/* Effective scale of every local code: eff[c] = S * dec(c) ([HS] §3: the effective group scale
 * is the product of the global and local scales), and its binary32 reciprocal. Index 0 unused. */
int ref_scale_tables(float S, float* eff, float* rcp)
{
    eff[0] = 0.0f;
    rcp[0] = 0.0f;
    for (int c = 1; c <= 126; ++c) {
        eff[c] = S * (float)ref_e4m3_value(c);
        rcp[c] = 1.0f / eff[c];
        if (!(eff[c] > 0.0f) || !isfinite(rcp[c])) return REF_ERR_ARG;
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Steps 3-6 for one group of 16 weights.                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Reconstruction loss of the group at one candidate scale ([HS] §3: diagonal-Hessian-weighted
 * reconstruction objective; [SS] §1: MSE and WMSE). For element j:
 *   x_j = fl(|w_j| * r),  q_j = E2M1(x_j),  d_j = fma(-q_j, eff, |w_j|),
 *   u_j = fl(h_j * d_j) (WMSE) or d_j (MSE).
 * The 16 products u_j * d_j are summed in a fixed tree: for each quad k = 0..3,
 * P_k = fl(u_4k * d_4k), then P_k = fma(u_4k+i, d_4k+i, P_k) for i = 1, 2, 3;
 * L = fl(fl(P_0 + P_1) + fl(P_2 + P_3)). */
static float group_loss(const float a[16], const float* h, float eff, float r)
{
    float P[4];
    for (int k = 0; k < 4; ++k) {
        for (int i = 0; i < 4; ++i) {
            int j = 4 * k + i;
            float x = a[j] * r;
            float q = E2M1_LEVEL[ref_e2m1_index(x)];
            float d = fmaf(-q, eff, a[j]);
            float u = h ? h[j] * d : d;
            P[k] = (i == 0) ? u * d : fmaf(u, d, P[k]);
        }
    }
    float left = P[0] + P[1];
    float right = P[2] + P[3];
    return left + right;
}

/* Base code of a group: the E4M3-rounded absmax/6 in units of S ([SS] Problem Statement and §2:
 * AbsMax initialisation, s_base = FP8-rounded maximum magnitude; [HS] §4: max-abs
 * initialisation). Returns 0 for an all-zero group. */
static int base_code(const float a[16], float S)
{
    float amax = 0.0f;
    for (int j = 0; j < 16; ++j)
        if (a[j] > amax) amax = a[j];
    if (amax == 0.0f) return 0;
    float s_star = (amax / 6.0f) / S;
    int b = ref_e4m3_encode(s_star);
    return b == 0 ? 1 : b;
}

/* Candidate code for loop position o: with a window, c = clamp(b + o, 1, 126) for
 * o = lo..hi ([HS] §3: nine smaller and six larger E4M3 steps with endpoint clipping;
 * [SS] §3: offsets [-3, 7] for MSE and [-8, 7] for WMSE, in FP8 bit-pattern space).
 * Exhaustive: c = o for o = 1..126 ([SS] §2: all 126 positive finite FP8 values). */
static int candidate_code(int b, int o, int exhaustive)
{
    if (exhaustive) return o;
    int c = b + o;
    if (c < 1) c = 1;
    if (c > 126) c = 126;
    return c;
}

/* Search one group. Writes its scale byte, 16 nibbles, the chosen loss and offset c* - b. */
static void search_group(const float w[16], const float* h, const float* eff, const float* rcp,
                         float S, int lo, int hi, int exhaustive, uint8_t* scale, uint8_t nib[16],
                         float* loss, int* offset)
{
    float a[16];
    for (int j = 0; j < 16; ++j) a[j] = fabsf(w[j]);
    int b = base_code(a, S);
    if (b == 0) { /* all-zero group: scale byte 0, signed zero codes */
        *scale = 0;
        for (int j = 0; j < 16; ++j) nib[j] = (uint8_t)(signbit(w[j]) ? 8 : 0);
        *loss = 0.0f;
        *offset = 0;
        return;
    }
    int first = exhaustive ? 1 : lo, last = exhaustive ? 126 : hi;
    int best_c = candidate_code(b, first, exhaustive);
    float best = group_loss(a, h, eff[best_c], rcp[best_c]);
    /* Keep the candidate with the smallest loss; the first one met wins ties ([HS] App. B:
     * the selected scale minimises the weighted objective; [SR] App. D.2: ties are
     * deterministic). */
    for (int o = first + 1; o <= last; ++o) {
        int c = candidate_code(b, o, exhaustive);
        float L = group_loss(a, h, eff[c], rcp[c]);
        if (L < best) {
            best = L;
            best_c = c;
        }
    }
    /* Quantize once with the chosen scale ([HS] App. B, HScaleGroupQuantize). */
    *scale = (uint8_t)best_c;
    for (int j = 0; j < 16; ++j) {
        float x = a[j] * rcp[best_c];
        nib[j] = (uint8_t)((signbit(w[j]) ? 8 : 0) | ref_e2m1_index(x));
    }
    *loss = best;
    *offset = best_c - b;
}

/* Whole matrix W[out, in] (row stride ldw), groups of 16 consecutive input columns ([HS] §3:
 * NVFP4 partitions weights into groups of 16; [SR] §4.1.1: 16 consecutive columns).
 * h[in] is the diagonal weight (NULL for MSE). Outputs are dense: scales[out, in/16],
 * packed[out, in/2], loss[out, in/16], offset[out, in/16] (loss/offset may be NULL). */
int ref_scale_search(const void* W, int dtype, int64_t out, int64_t in, int64_t ldw,
                     const float* h, int objective, int lo, int hi, int exhaustive, float S,
                     uint8_t* scales, uint8_t* packed, float* loss, int8_t* offset, int nthreads)
{
    if (in % 16 != 0 || out < 0 || in < 0 || ldw < in) return REF_ERR_ARG;
    if (objective == REF_WMSE && !h) return REF_ERR_ARG;
    if (objective == REF_MSE) h = NULL;
    if (!exhaustive && (lo > 0 || hi < 0 || lo < -125 || hi > 125)) return REF_ERR_ARG;
    if (!isfinite(S) || !(S > 0.0f)) return REF_ERR_ARG;
    float eff[127], rcp[127];
    if (ref_scale_tables(S, eff, rcp) != REF_OK) return REF_ERR_ARG;
    if (h)
        for (int64_t i = 0; i < in; ++i)
            if (!isfinite(h[i])) return REF_ERR_NONFINITE;
    int64_t gpr = in / 16;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4) reduction(| : bad)
    for (int64_t o = 0; o < out; ++o) {
        for (int64_t g = 0; g < gpr; ++g) {
            float w[16];
            for (int j = 0; j < 16; ++j) {
                w[j] = load_elem(W, dtype, o * ldw + g * 16 + j);
                if (!isfinite(w[j])) bad = 1;
            }
            uint8_t nib[16], sc;
            float L;
            int off;
            search_group(w, h ? h + g * 16 : NULL, eff, rcp, S, lo, hi, exhaustive, &sc, nib, &L,
                         &off);
            int64_t gi = o * gpr + g;
            scales[gi] = sc;
            for (int k = 0; k < 8; ++k)
                packed[o * (in / 2) + g * 8 + k] = (uint8_t)(nib[2 * k] | (nib[2 * k + 1] << 4));
            if (loss) loss[gi] = L;
            if (offset) offset[gi] = (int8_t)off;
        }
    }
    return bad ? REF_ERR_NONFINITE : REF_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Proposal-centred search ([SR] §4.1.3-§4.1.4, App. D.2).                                    */
/* ------------------------------------------------------------------------------------------ */

/* Schur Replay takes a per-group proposal code, scores the exportable codes within a half-window
 * around it, and keeps the incoming scale unless a candidate is better (ten candidates in
 * all: a half-window of 4 plus the incoming code; ties are deterministic and the status quo is
 * retained). Here the candidates are scored with this path's loss (group_loss):
 *   1. the incoming code, when it is a valid code 1..126;
 *   2. clamp(center + o, 1, 126) for o = lo..hi ascending, center itself clamped to 1..126.
 * A candidate replaces the best only when its loss is strictly smaller, so the incoming code
 * wins every tie and the window's ties go to its lowest code. Without a valid incoming code the
 * first window candidate starts the scan. An all-zero group gets scale byte 0 as in the plain
 * search. The offset reported is c* - center. */
static void search_group_proposal(const float w[16], const float* h, const float* eff,
                                  const float* rcp, float S, int lo, int hi, int center,
                                  int incoming, uint8_t* scale, uint8_t nib[16], float* loss,
                                  int* offset)
{
    float a[16];
    for (int j = 0; j < 16; ++j) a[j] = fabsf(w[j]);
    if (base_code(a, S) == 0) {
        *scale = 0;
        for (int j = 0; j < 16; ++j) nib[j] = (uint8_t)(signbit(w[j]) ? 8 : 0);
        *loss = 0.0f;
        *offset = 0;
        return;
    }
    int cen = center < 1 ? 1 : (center > 126 ? 126 : center);
    int best_c, o0;
    float best;
    if (incoming >= 1 && incoming <= 126) {
        best_c = incoming;
        best = group_loss(a, h, eff[best_c], rcp[best_c]);
        o0 = lo;
    } else {
        best_c = candidate_code(cen, lo, 0);
        best = group_loss(a, h, eff[best_c], rcp[best_c]);
        o0 = lo + 1;
    }
    for (int o = o0; o <= hi; ++o) {
        int c = candidate_code(cen, o, 0);
        float L = group_loss(a, h, eff[c], rcp[c]);
        if (L < best) {
            best = L;
            best_c = c;
        }
    }
    *scale = (uint8_t)best_c;
    for (int j = 0; j < 16; ++j) {
        float x = a[j] * rcp[best_c];
        nib[j] = (uint8_t)((signbit(w[j]) ? 8 : 0) | ref_e2m1_index(x));
    }
    *loss = best;
    *offset = best_c - cen;
}

/* Whole matrix, as ref_scale_search, with per-group proposal codes center[out, in/16] and
 * incoming codes incoming[out, in/16] (NULL: no incoming candidate). */
int ref_scale_search_proposal(const void* W, int dtype, int64_t out, int64_t in, int64_t ldw,
                              const float* h, int objective, int lo, int hi,
                              const uint8_t* center, const uint8_t* incoming, float S,
                              uint8_t* scales, uint8_t* packed, float* loss, int8_t* offset,
                              int nthreads)
{
    if (in % 16 != 0 || out < 0 || in < 0 || ldw < in || !center) return REF_ERR_ARG;
    if (objective == REF_WMSE && !h) return REF_ERR_ARG;
    if (objective == REF_MSE) h = NULL;
    if (lo > 0 || hi < 0 || lo < -125 || hi > 125) return REF_ERR_ARG;
    if (!isfinite(S) || !(S > 0.0f)) return REF_ERR_ARG;
    float eff[127], rcp[127];
    if (ref_scale_tables(S, eff, rcp) != REF_OK) return REF_ERR_ARG;
    if (h)
        for (int64_t i = 0; i < in; ++i)
            if (!isfinite(h[i])) return REF_ERR_NONFINITE;
    int64_t gpr = in / 16;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 4) reduction(| : bad)
    for (int64_t o = 0; o < out; ++o) {
        for (int64_t g = 0; g < gpr; ++g) {
            float w[16];
            for (int j = 0; j < 16; ++j) {
                w[j] = load_elem(W, dtype, o * ldw + g * 16 + j);
                if (!isfinite(w[j])) bad = 1;
            }
            int64_t gi = o * gpr + g;
            uint8_t nib[16], sc;
            float L;
            int off;
            search_group_proposal(w, h ? h + g * 16 : NULL, eff, rcp, S, lo, hi, center[gi],
                                  incoming ? incoming[gi] : 0, &sc, nib, &L, &off);
            scales[gi] = sc;
            for (int k = 0; k < 8; ++k)
                packed[o * (in / 2) + g * 8 + k] = (uint8_t)(nib[2 * k] | (nib[2 * k + 1] << 4));
            if (loss) loss[gi] = L;
            if (offset) offset[gi] = (int8_t)off;
        }
    }
    return bad ? REF_ERR_NONFINITE : REF_OK;
}

/* Losses of every candidate of one group, in loop order (for checks). Returns the base code;
 * codes[i] / losses[i] for i < count, where count = hi - lo + 1 or 126. */
int ref_group_candidates(const float w[16], const float* h, float S, int lo, int hi,
                         int exhaustive, int* codes, float* losses)
{
    float eff[127], rcp[127];
    if (ref_scale_tables(S, eff, rcp) != REF_OK) return -1;
    float a[16];
    for (int j = 0; j < 16; ++j) a[j] = fabsf(w[j]);
    int b = base_code(a, S);
    if (b == 0) return 0;
    int first = exhaustive ? 1 : lo, last = exhaustive ? 126 : hi;
    for (int o = first; o <= last; ++o) {
        int c = candidate_code(b, o, exhaustive);
        codes[o - first] = c;
        losses[o - first] = group_loss(a, h, eff[c], rcp[c]);
    }
    return b;
}

/* Quantize W at given scale bytes and pack ([HS] App. B: quantize the group once with the
 * chosen scale; round-to-nearest at a fixed scale). Scale byte 0 gives signed zero codes. */
int ref_pack(const void* W, int dtype, int64_t out, int64_t in, int64_t ldw,
             const uint8_t* scales, float S, uint8_t* packed, int nthreads)
{
    if (in % 16 != 0 || out < 0 || in < 0 || ldw < in) return REF_ERR_ARG;
    if (!isfinite(S) || !(S > 0.0f)) return REF_ERR_ARG;
    float eff[127], rcp[127];
    if (ref_scale_tables(S, eff, rcp) != REF_OK) return REF_ERR_ARG;
    int64_t gpr = in / 16;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(| : bad)
    for (int64_t o = 0; o < out; ++o) {
        for (int64_t g = 0; g < gpr; ++g) {
            int c = scales[o * gpr + g];
            if (c > 126) bad = 1;
            uint8_t nib[16];
            for (int j = 0; j < 16; ++j) {
                float w = load_elem(W, dtype, o * ldw + g * 16 + j);
                int idx = (c == 0 || c > 126) ? 0 : ref_e2m1_index(fabsf(w) * rcp[c]);
                nib[j] = (uint8_t)((signbit(w) ? 8 : 0) | idx);
            }
            for (int k = 0; k < 8; ++k)
                packed[o * (in / 2) + g * 8 + k] = (uint8_t)(nib[2 * k] | (nib[2 * k + 1] << 4));
        }
    }
    return bad ? REF_ERR_ARG : REF_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* GPTQ with the scale search as its local quantizer ([HS] App. B: the search replaces only   */
/* the local quantisation call; inverse-Cholesky processing and error propagation are kept;  */
/* [SR] §3: input columns in sequence with one shared Hessian factor, rows independent).      */
/* ------------------------------------------------------------------------------------------ */

/* One output row, all binary32, in this order for column j = 0..in-1:
 *   - at the first column of a 16-column group: the group's scale code c by search_group on
 *     the row's current values of the group's columns (and their h);
 *   - x = fl(|w_j| * r[c]), q = E2M1 index with w_j's sign, the dequantised value
 *     v = fl(level * eff[c]) with the sign, err = fl(fl(w_j - v) / U[j][j]);
 *   - every later column k > j: w_k = fma(-err, U[j][k], w_k).
 * U is the upper-triangular factor of the damped inverse Hessian (row-major [in, in]); the
 * nibble of column j and the group's code are the outputs. w is updated in place. */
static void gptq_row(float* w, int64_t in, const float* U, const float* h, const float* eff,
                     const float* rcp, float S, int lo, int hi, uint8_t* scales, uint8_t* packed)
{
    int c = 0;
    for (int64_t j = 0; j < in; ++j) {
        if (j % 16 == 0) {
            uint8_t nib_unused[16], sc;
            float L;
            int off;
            search_group(w + j, h ? h + j : NULL, eff, rcp, S, lo, hi, 0, &sc, nib_unused, &L,
                         &off);
            c = sc;
            scales[j / 16] = sc;
        }
        float a = fabsf(w[j]);
        int idx = (c == 0) ? 0 : ref_e2m1_index(a * rcp[c]);
        float mag = (c == 0) ? 0.0f : E2M1_LEVEL[idx] * eff[c];
        float v = signbit(w[j]) ? -mag : mag;
        uint8_t nib = (uint8_t)((signbit(w[j]) ? 8 : 0) | idx);
        if (j & 1)
            packed[j / 2] = (uint8_t)(packed[j / 2] | (nib << 4));
        else
            packed[j / 2] = nib;
        float err = (w[j] - v) / U[j * in + j];
        for (int64_t k = j + 1; k < in; ++k) w[k] = fmaf(-err, U[j * in + k], w[k]);
    }
}

/* GPTQ over W[out, in] with the window search as local quantiser. Outputs scales[out, in/16]
 * and packed[out, in/2]; W_final[out, in] (optional) receives the updated binary32 weights. */
int ref_gptq(const void* W, int dtype, int64_t out, int64_t in, int64_t ldw, const float* U,
             const float* h, int objective, int lo, int hi, float S, uint8_t* scales,
             uint8_t* packed, float* W_final, int nthreads)
{
    if (in % 16 != 0 || out < 0 || in < 0 || ldw < in || !U) return REF_ERR_ARG;
    if (objective == REF_WMSE && !h) return REF_ERR_ARG;
    if (objective == REF_MSE) h = NULL;
    if (lo > 0 || hi < 0 || lo < -125 || hi > 125) return REF_ERR_ARG;
    if (!isfinite(S) || !(S > 0.0f)) return REF_ERR_ARG;
    float eff[127], rcp[127];
    if (ref_scale_tables(S, eff, rcp) != REF_OK) return REF_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : bad)
    for (int64_t o = 0; o < out; ++o) {
        float* w = (float*)malloc((size_t)in * sizeof(float));
        if (!w) { bad = 1; continue; }
        for (int64_t i = 0; i < in; ++i) {
            w[i] = load_elem(W, dtype, o * ldw + i);
            if (!isfinite(w[i])) bad = 1;
        }
        gptq_row(w, in, U, h, eff, rcp, S, lo, hi, scales + o * (in / 16), packed + o * (in / 2));
        if (W_final) memcpy(W_final + o * in, w, (size_t)in * sizeof(float));
        free(w);
    }
    return bad ? REF_ERR_NONFINITE : REF_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Layer-output evaluation ([HS] §3: layer-output reconstruction; the activation-loss         */
/* comparison of Min-Max, MSE-guided and Hessian-guided scales).                             */
/* ------------------------------------------------------------------------------------------ */

/* Dequantised weights: w_hat[o, i] = sign * level * eff[c] in binary32 (one rounding of the
 * product level * eff, with eff = fl(S * dec(c))), from packed codes [out, in/2] (element 2k in
 * the low nibble of byte k) and scale bytes [out, in/16]. Scale byte 0 gives signed zeros.
 * Scale bytes above 126 are refused. */
int ref_dequant(const uint8_t* packed, const uint8_t* scales, int64_t out, int64_t in, float S,
                float* w_hat)
{
    if (in % 16 != 0 || out < 0 || in < 0) return REF_ERR_ARG;
    if (!isfinite(S) || !(S > 0.0f)) return REF_ERR_ARG;
    float eff[127], rcp[127];
    if (ref_scale_tables(S, eff, rcp) != REF_OK) return REF_ERR_ARG;
    int64_t gpr = in / 16;
    for (int64_t o = 0; o < out; ++o)
        for (int64_t i = 0; i < in; ++i) {
            int c = scales[o * gpr + i / 16];
            if (c > 126) return REF_ERR_ARG;
            uint8_t byte = packed[o * (in / 2) + i / 2];
            int nib = (i & 1) ? (byte >> 4) : (byte & 15);
            float mag = (c == 0) ? 0.0f : E2M1_LEVEL[nib & 7] * eff[c];
            w_hat[o * in + i] = (nib & 8) ? -mag : mag;
        }
    return REF_OK;
}

/* Batch helper for many scalar E2M1 / E4M3 decisions (used by the format checks). */
void ref_e2m1_index_many(const float* x, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)ref_e2m1_index(x[i]);
}

void ref_e4m3_encode_many(const float* s, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)ref_e4m3_encode(s[i]);
}
