/*
 * nvfp4.h - C ABI of the MI355X (gfx950) NVFP4 per-group E4M3 block-scale search library.
 *
 * The library computes, on one GPU, the data-parallel core shared by the NVFP4 scale-refinement
 * methods described in
 *   [HS] "H-Scale: Hessian-Guided Scale Refinement for NVFP4 Sub-Byte LLM Inference",
 *   [SS] "ScaleSweep" (technical summary), and the scale step of
 *   [SR] "Replay the Curvature: Accurate and Scalable NVFP4 Quantization for LLM Inference":
 *   1. a diagonal second-order weight h_j = sum_t x_tj^2 from calibration activations X;
 *   2. a global FP32 scale S per tensor;
 *   3. for every group of 16 consecutive weights of a row, the E4M3 local scale chosen from a
 *      window of adjacent E4M3 codes around the rounded absmax/6 base (or from all 126 codes)
 *      by E2M1 round-to-nearest-even quantization and the h-weighted (or plain) squared error;
 *   4. the packed 4-bit codes and the E4M3 scale bytes.
 *
 * Conventions shared by every entry point:
 *   - Every pointer named "device" is GPU memory owned by the caller; the library allocates
 *     no memory and keeps no data between calls (only, per device, the compute-unit count and
 *     the occupancy figures it queries once). Host pointers are named as such.
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and is
 *     asynchronous. Argument errors are detected on the host and returned before anything is
 *     enqueued; a failed kernel launch returns NVFP4_ERR_HIP. Nothing is thrown across the ABI.
 *   - Matrices are row-major. Sizes and leading dimensions are in elements. A matrix argument
 *     with a zero dimension is valid and enqueues no work (except where noted). Rows times
 *     leading dimension, and matrices times matrix stride, must each stay within 2^56 elements
 *     (else NVFP4_ERR_SHAPE).
 *   - Inputs must be finite; results for non-finite inputs are unspecified.
 *   - Results are deterministic: identical inputs give byte-identical outputs (no float atomics).
 *   - Calls that overlap on the same output buffers race; the library does not serialise them.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,      /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = 2,     /* negative size, in % 16 != 0, ld < in, size too large, ... */
    NVFP4_ERR_DTYPE = 3,     /* unknown element type */
    NVFP4_ERR_ALIGN = 4,     /* a pointer, stride or leading dimension breaks 16-byte rows */
    NVFP4_ERR_WINDOW = 5,    /* window with lo > 0, hi < 0 or |lo|, |hi| > 125 */
    NVFP4_ERR_ARG = 6,       /* other invalid argument (objective, rule, group size, ...) */
    NVFP4_ERR_WORKSPACE = 7, /* workspace missing or smaller than the *_workspace_size value */
    NVFP4_ERR_HIP = 8        /* a HIP runtime call or kernel launch failed */
} nvfp4_status;

typedef enum nvfp4_dtype { NVFP4_DTYPE_F32 = 0, NVFP4_DTYPE_BF16 = 1 } nvfp4_dtype;

/* [SS] Methodology §1: MSE (plain reconstruction error) and WMSE (weighted by importance
 * scores from activation statistics); [HS] §3: the diagonal-Hessian-weighted objective. */
typedef enum nvfp4_objective { NVFP4_MSE = 0, NVFP4_WMSE = 1 } nvfp4_objective;

/* Global-scale rule. [SS] Methodology §2 fixes S = max|w| / (256 * 6) (NVFP4_GS_AMAX_256).
 * NVFP4_GS_AMAX_448 maps the largest group onto E4M3's largest finite value:
 * S = max|w| / (448 * 6). An all-zero tensor gets S = 1. */
typedef enum nvfp4_gs_rule { NVFP4_GS_AMAX_448 = 0, NVFP4_GS_AMAX_256 = 1 } nvfp4_gs_rule;

/* Human-readable name of a status code (static string, never NULL). */
const char* nvfp4_status_string(int status);

/* Library version string, e.g. "nvfp4-gfx950 1.0". */
const char* nvfp4_version(void);

/* ---------------------------------------------------------------------------------------------
 * Step 1: diagonal second-order weight ([HS] §3 and App. B: h = diag(X^T X) from calibration
 * activations, cross-channel terms dropped; [SS] §1: Gram-matrix diagonals as WMSE importance;
 * [SR] §3: H from the calibration inputs).
 *
 *   h_acc[j] = (accumulate ? h_acc[j] : 0) + sum_{t < tokens} X[t, j]^2     (binary64)
 *   h[j]     = (float) h_acc[j]                                              (round to nearest)
 *
 * X       device, [tokens, in] with row stride ldx, bf16 or f32 (x_dtype), 16-byte aligned.
 * h_acc   device, [in] binary64 running sum; read when accumulate != 0, always written. Keeping
 *         it across calls streams X in token chunks with no intermediate fp32 rounding.
 * h       device, [in] binary32 output; may be NULL.
 * workspace  device scratch of at least nvfp4_diag_hessian_workspace_size(tokens, in, 1) bytes,
 *         16-byte aligned; its contents are overwritten and need no initialisation.
 * Requires in % 8 == 0 and ldx % 8 == 0. tokens == 0 is valid: h_acc is cleared (accumulate
 * == 0) or kept, and h is written from it. Partial sums are combined in a fixed order, so the
 * result does not depend on scheduling.
 *
 * Deferred mode, for token chunks of one calibration set: with h_acc == NULL and h == NULL the
 * call only adds the chunk's binary64 row-group sums into the workspace (replacing them when
 * accumulate == 0), and nvfp4_diag_hessian_finalize later turns the workspace into h_acc and
 * h. One finalize per set instead of one per chunk. Every call of a sequence uses the same
 * workspace, x_dtype and in; the first call has accumulate == 0 and the largest token count
 * of the sequence, which finalize is given as `tokens` (it fixes the workspace layout). The
 * number of workspace slots a call writes never decreases as its token count grows, so every
 * later, shorter chunk adds only into slots that the first call initialised. A later chunk
 * longer than the first is outside this contract: its extra slots are not summed.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_diag_hessian_workspace_size(int64_t tokens, int64_t in, int64_t segments);

nvfp4_status nvfp4_diag_hessian(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                int64_t ldx, double* h_acc, float* h, int accumulate,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Finalize of a deferred sequence of nvfp4_diag_hessian calls: h_acc[j] = (accumulate ?
 * h_acc[j] : 0) + the binary64 sum of the workspace's row-group slots, h[j] = (float) h_acc[j]
 * (h may be NULL). tokens and x_dtype are those of the sequence's first call. */
nvfp4_status nvfp4_diag_hessian_finalize(int x_dtype, int64_t tokens, int64_t in, double* h_acc,
                                         float* h, int accumulate, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Token chunks of one calibration set that are resident together but not contiguous (e.g. the
 * activations of several forward passes), reduced in one partial launch and one finalize
 * instead of one launch per chunk ([HS] §4: the one-time activation pass over the calibration
 * set; App. B: h = diag(X^T X)):
 *   h_acc[j] = (accumulate ? h_acc[j] : 0) + sum_c sum_{t < tokens[c]} X_c[t, j]^2   (binary64)
 *   h[j]     = (float) h_acc[j]
 * X_chunks  host array of n_chunks device pointers (read during the call only); chunk c is
 *           [tokens[c], in] with row stride ldx, bf16 or f32 (x_dtype), 16-byte aligned.
 * tokens    host array of n_chunks token counts (>= 0). 1 <= n_chunks <= 64.
 * h_acc, h, accumulate  as for nvfp4_diag_hessian (h_acc required).
 * workspace at least nvfp4_diag_hessian_chunks_workspace_size(tokens, n_chunks, in) bytes,
 *           16-byte aligned; overwritten, no initialisation needed. The size function returns
 *           0 for invalid arguments.
 * Deterministic. The binary64 partial sums are grouped differently from a sequence of
 * per-chunk calls, so the two agree to binary64 rounding, not always bit for bit. */
size_t nvfp4_diag_hessian_chunks_workspace_size(const int64_t* tokens, int64_t n_chunks,
                                                int64_t in);

nvfp4_status nvfp4_diag_hessian_chunks(const void* const* X_chunks, int x_dtype,
                                       const int64_t* tokens, int64_t n_chunks, int64_t in,
                                       int64_t ldx, double* h_acc, float* h, int accumulate,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Batched form for a mixture-of-experts layer: X holds the routed tokens of `segments` experts
 * back to back; expert e owns rows [seg_offsets[e], seg_offsets[e+1]). Writes h_acc/h as
 * [segments, in] (row e = expert e), with the same accumulate rule per row.
 * seg_offsets  device, int64 [segments + 1], non-decreasing, seg_offsets[0] == 0 and
 *              seg_offsets[segments] == total_tokens (not checked on the device).
 * workspace    at least nvfp4_diag_hessian_workspace_size(total_tokens, in, segments) bytes. */
nvfp4_status nvfp4_diag_hessian_batched(const void* X, int x_dtype, const int64_t* seg_offsets,
                                        int64_t segments, int64_t total_tokens, int64_t in,
                                        int64_t ldx, double* h_acc, float* h, int accumulate,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Step 2: global FP32 scale per tensor ([HS] §3: a tensor-level FP32 global scale, the effective
 * group scale being the product of global and local scales; [SS] §2: S = max|x| / (256 * 6)).
 *
 * W        device, `batch` matrices [out, in], row stride ldw, matrix stride stride_w (elements),
 *          bf16 or f32, 16-byte aligned rows.
 * S        device, float [batch]: S[b] from the max |w| of matrix b by `rule`.
 * workspace  device scratch of nvfp4_global_scale_workspace_size(batch, out, in) bytes,
 *          4-byte aligned; its contents are overwritten and need no initialisation.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_global_scale_workspace_size(int64_t batch, int64_t out, int64_t in);

nvfp4_status nvfp4_global_scale(const void* W, int w_dtype, int64_t batch, int64_t out,
                                int64_t in, int64_t ldw, int64_t stride_w, int rule, float* S,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Steps 1 and 2 together for one layer: h of its calibration activations X and the global scale
 * S of its weight matrix W ([HS] §3 / App. B: h = diag(X^T X) and the tensor-level FP32 scale
 * are the two per-layer inputs of the search; [SS] §2: the 256 * 6 rule).
 *
 * Results are bit-identical to nvfp4_diag_hessian(X, ..., h_acc, h, accumulate) followed by
 * nvfp4_global_scale(W, 1 matrix, ..., rule, S); the two reductions share two launches instead
 * of four, which shortens a layer's chain of dependent launches.
 *
 * X, tokens, in, ldx, h_acc, h, accumulate  as for nvfp4_diag_hessian (one token chunk, h_acc
 *          required).
 * W        device, bf16 or f32 [out, in], row stride ldw, 16-byte aligned rows (the layer's
 *          weights: their `in` is X's).
 * rule     NVFP4_GS_AMAX_448 or NVFP4_GS_AMAX_256; S device float [1].
 * workspace  device, nvfp4_layer_statistics_workspace_size(tokens, in, out) bytes, 16-byte
 *          aligned; overwritten, no initialisation needed.
 * Argument errors are those of the two calls it replaces.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_layer_statistics_workspace_size(int64_t tokens, int64_t in, int64_t out);

nvfp4_status nvfp4_layer_statistics(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                    int64_t ldx, double* h_acc, float* h, int accumulate,
                                    const void* W, int w_dtype, int64_t out, int64_t ldw, int rule,
                                    float* S, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------------------------
 * Steps 3-4: per-group E4M3 scale search, fused with quantize + pack.
 *
 * For group g of 16 consecutive input columns of row o of matrix b ([HS] §3 and [SR] §4.1.1:
 * groups of 16, one E4M3 local scale per group):
 *   eff[c] = fl(S[b] * E4M3(c)), r[c] = fl(1 / eff[c])           for codes c = 1..126
 *   base   = E4M3 round-to-nearest-even of fl(fl(max|w| / 6) / S[b]), saturating at 448, and
 *            raised to code 1 if it rounds to 0 ([SS] Problem Statement and §2: AbsMax start,
 *            s_base = FP8-rounded block maximum; [HS] §4: max-abs initialisation)
 *   codes  = base + lo .. base + hi clipped to [1, 126] ([HS] §3: nine smaller and six larger
 *            E4M3 steps with endpoint clipping; [SS] §3: offsets [-3, 7] for MSE, [-8, 7] for
 *            WMSE in FP8 bit-pattern space), or all codes 1..126 if exhaustive ([SS] §2)
 *   loss(c) = sum_j u_j * d_j, x_j = fl(|w_j| * r[c]), q_j = E2M1_RNE(x_j) (ties to the even
 *            code, saturating at 6), d_j = fma(-q_j, eff[c], |w_j|), u_j = fl(h_j * d_j) for
 *            WMSE or d_j for MSE, summed in binary32 in a fixed tree: per quad k = 0..3,
 *            P_k = u_4k d_4k, then P_k = fma(u_4k+i, d_4k+i, P_k) for i = 1..3;
 *            L = (P_0 + P_1) + (P_2 + P_3)
 *   choice = the code of smallest loss, the lowest code among equal losses ([SR] App. D.2:
 *            ties are deterministic)
 *   output ([HS] App. B: quantize once with the chosen scale, native NVFP4):
 *            scales[b, o, g] = chosen code (0 for an all-zero group)
 *            packed[b, o, 8g + k] = nibble(2k) | nibble(2k+1) << 4, nibble = sign(w) << 3 |
 *            E2M1 index of fl(|w| * r[choice])
 *            loss[b, o, g] = loss(choice) (0 for a zero group), offset[b, o, g] = choice - base
 *
 * W         device, `batch` matrices [out, in] (ldw, stride_w in elements), bf16 or f32,
 *           16-byte aligned rows (ldw, stride_w multiples of 16 bytes).
 * group_size must be 16.
 * h         device, float [batch, in] with row stride stride_h (multiple of 4), 16-byte
 *           aligned; required for WMSE, ignored (may be NULL) for MSE.
 * lo, hi    window offsets, -125 <= lo <= 0 <= hi <= 125; ignored when exhaustive != 0.
 * S         device, float [batch], positive, finite, with every S * E4M3(c) a normal binary32
 *           value whose reciprocal is finite (otherwise results are unspecified).
 * scales    device, uint8 [batch, out, in/16];  packed  device, uint8 [batch, out, in/2].
 * loss      device, float [batch, out, in/16] or NULL; offset device, int8 [...] or NULL.
 * Requires in % 16 == 0 and batch * ... sizes with out * in/16 < 2^31 per matrix.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_scale_search(const void* W, int w_dtype, int64_t batch, int64_t out,
                                int64_t in, int64_t ldw, int64_t stride_w, int32_t group_size,
                                const float* h, int64_t stride_h, int objective, int32_t lo,
                                int32_t hi, int exhaustive, const float* S, uint8_t* scales,
                                uint8_t* packed, float* loss, int8_t* offset, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Steps 3-4 for several rules at once: the same weights searched under several objectives and
 * windows, as when Min-Max, MSE-guided and Hessian-guided scales of one layer are compared
 * ([HS] §4: MSE and Hessian-guided refinement against max-abs scales; [SS] §3: the MSE [-3, 7]
 * and WMSE [-8, 7] windows of one model).
 *
 * rules[k]'s outputs are exactly those of nvfp4_scale_search with that rule's objective, lo, hi,
 * exhaustive and output pointers, and the call's other arguments. Rules are taken in order,
 * two at a time where they fit one launch:
 *   - two consecutive windowed rules of 11 or 16 codes on bf16 W run as one launch that reads
 *     each group once and shares its table and base code between them; where one window has
 *     16 codes and holds the other (11 codes ending where it ends, as MSE [-3, 7] inside
 *     [-8, 7], or the same 16 codes), each code is converted once for both rules and only the
 *     weighting and the sum of squares are done per rule;
 *   - else a windowed rule of 16 codes and an exhaustive rule of the same objective, next to
 *     each other in either order (bf16 or f32 W), run as one launch: the exhaustive search's
 *     first block of 16 codes is placed on the window, so the window's losses are the ones the
 *     exhaustive search computes anyway ([SR] App. D.5: a local window's choice audited
 *     against the exhaustive optimum over every exportable scale);
 *   - every other rule runs as its own launch.
 *
 * rules     host, n_rules entries (1 <= n_rules <= 64), read during the call only. The output
 *           buffers of different rules must not overlap.
 * h         required (with the alignment and stride of nvfp4_scale_search) if any rule is
 *           WMSE; ignored otherwise.
 * Every rule is validated before anything is enqueued; the first invalid rule's status is
 * returned.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    int32_t objective;   /* NVFP4_MSE or NVFP4_WMSE */
    int32_t lo, hi;      /* window offsets, -125 <= lo <= 0 <= hi <= 125 unless exhaustive */
    int32_t exhaustive;  /* nonzero: every code 1..126 */
    uint8_t* scales;     /* device, uint8 [batch, out, in/16] */
    uint8_t* packed;     /* device, uint8 [batch, out, in/2], 8-byte aligned */
    float* loss;         /* device, float [batch, out, in/16], or NULL */
    int8_t* offset;      /* device, int8 [batch, out, in/16], or NULL */
} nvfp4_search_rule;

nvfp4_status nvfp4_scale_search_rules(const void* W, int w_dtype, int64_t batch, int64_t out,
                                      int64_t in, int64_t ldw, int64_t stride_w,
                                      int32_t group_size, const float* h, int64_t stride_h,
                                      const float* S, const nvfp4_search_rule* rules,
                                      int32_t n_rules, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Work count of the exhaustive search (for measurement: the exhaustive mode skips every code
 * whose loss a lower bound proves larger than the best already found, so the codes it scores
 * depend on the data). Adds to *count the number of (group, code) candidates that the
 * exhaustive search over these inputs scores: for every group with a nonzero base code, the 16
 * codes of its first block (codes clamp(base + centre_lo, 8, 111) .. + 15) and the codes 1..126
 * of every further block of 4 that its bounds do not rule out. It runs the search's own first
 * phase, so the count is exact for the same W, h and S.
 *
 * centre_lo  -8 for nvfp4_scale_search's exhaustive mode; for nvfp4_scale_search_rules' fused
 *            window + exhaustive launch, the window rule's lo. -15 <= centre_lo <= 0.
 * count      device, one uint64 (8-byte aligned), added to (not cleared) by the call.
 * Other arguments as nvfp4_scale_search.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_scale_search_scored(const void* W, int w_dtype, int64_t batch, int64_t out,
                                       int64_t in, int64_t ldw, int64_t stride_w,
                                       int32_t group_size, const float* h, int64_t stride_h,
                                       int objective, int32_t centre_lo, const float* S,
                                       uint64_t* count, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Steps 3-4 with a proposal-centred window and the incoming scale kept on ties ([SR] §4.1.3 and
 * §4.1.4: a proposal gives a neighbourhood of exportable scales that is then scored, and keeping
 * the status-quo scale means the local search cannot increase the loss; [SR] App. D.2: a
 * half-window of 4 plus the incoming exportable scale, ten candidates in all; deterministic ties).
 *
 * Same arithmetic, arguments and outputs as nvfp4_scale_search, with these differences:
 *   centre  = center[b, o, g] clamped to 1..126 (replaces the base code as the window centre)
 *   scan    = incoming[b, o, g] first when incoming != NULL and the code is 1..126, then
 *             clamp(centre + o, 1, 126) for o = lo..hi ascending; a candidate replaces the best
 *             only when its loss is strictly smaller, so the incoming code wins every tie and the
 *             window's ties go to its lowest code
 *   offset[b, o, g] = choice - centre
 * An all-zero group still gets scale byte 0, zero codes, loss 0 and offset 0.
 *
 * center    device, uint8 [batch, out, in/16], required.
 * incoming  device, uint8 [batch, out, in/16], or NULL for no incoming candidate; codes outside
 *           1..126 mean "no incoming candidate" for that group.
 * lo, hi    window offsets around the centre, -125 <= lo <= 0 <= hi <= 125 (no exhaustive mode).
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_scale_search_proposal(const void* W, int w_dtype, int64_t batch, int64_t out,
                                         int64_t in, int64_t ldw, int64_t stride_w,
                                         int32_t group_size, const float* h, int64_t stride_h,
                                         int objective, int32_t lo, int32_t hi,
                                         const uint8_t* center, const uint8_t* incoming,
                                         const float* S, uint8_t* scales, uint8_t* packed,
                                         float* loss, int8_t* offset, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Quantize + pack at given scale bytes ([HS] App. B: the group is quantized once with its
 * scale; round-to-nearest at a fixed scale). Same layouts and nibble rule as above; a scale
 * byte of 0 gives signed zero codes. Scale bytes must be 0..126.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_pack(const void* W, int w_dtype, int64_t batch, int64_t out, int64_t in,
                        int64_t ldw, int64_t stride_w, const uint8_t* scales, const float* S,
                        uint8_t* packed, void* stream);

/* ---------------------------------------------------------------------------------------------
 * GPTQ with the scale search as local quantiser ([HS] App. B: the search replaces only GPTQ's
 * local quantisation call, and inverse-Cholesky processing and error propagation are kept;
 * [SR] §3: input columns in sequence with one shared Hessian factor, output rows independent).
 *
 * For every row o and column j = 0..in-1 in order, all in binary32:
 *   - at the first column of each 16-column group the group's scale code is chosen as by
 *     nvfp4_scale_search (window lo..hi around the base code, lowest code on ties), from the
 *     row's current (already updated) values of the group's columns and their h;
 *   - the column is quantised at that code (signed E2M1 code of fl(w_j * r[c])), its
 *     dequantised value v = fl(level * eff[c]) with w_j's sign, err = fl(fl(w_j - v) / U[j][j]);
 *   - every later column k > j takes w_k = fma(-err, U[j][k], w_k), in column order j.
 * Each element receives exactly this sequence of operations whatever the internal blocking, so
 * results are deterministic and reproducible by a sequential implementation.
 *
 * W         device, bf16 or f32 [out, in], row stride ldw (16-byte aligned rows).
 * U         device float [in, in] row-major, 16-byte aligned: the upper-triangular factor of the
 *           damped inverse Hessian, (H + damping)^-1 = U^T U (entries below the diagonal are not
 *           read); computed by the caller, e.g. with a Cholesky routine. Its diagonal must be
 *           positive and finite (as a Cholesky factor's is); otherwise the propagated values are
 *           not finite and the outputs are unspecified.
 * Shapes: in % 16 == 0, out * in < 2^39 and out <= 2,097,120 (else NVFP4_ERR_SHAPE).
 * h         device float [in], the diagonal weights of the search (WMSE), e.g. diag(H); NULL
 *           for MSE.
 * S         device float [1]: the global scale (e.g. from nvfp4_global_scale on W).
 * scales    device uint8 [out, in/16]; packed device uint8 [out, in/2], 8-byte aligned.
 * W_final   device float [out, in] or NULL (16-byte aligned): receives the updated binary32
 *           weights.
 * workspace device, nvfp4_gptq_workspace_size(out, in) bytes, 16-byte aligned, no
 *           initialisation needed.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_gptq_workspace_size(int64_t out, int64_t in);

nvfp4_status nvfp4_gptq(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                        const float* U, const float* h, int objective, int32_t lo, int32_t hi,
                        const float* S, uint8_t* scales, uint8_t* packed, float* W_final,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * On-line activation quantisation ([SS] Experimental Results: the WA, WAKV and WAKVQ settings
 * quantise activations, KV cache and query states with the same sweep; [SS] §2: the per-tensor
 * global scale S = max|x| / (256 * 6)).
 *
 * For one activation tensor X [tokens, in]: S = max|x| / 1536 (rule AMAX_256) or / 2688
 * (AMAX_448), 1 for an all-zero tensor, exactly as nvfp4_global_scale computes it; then the
 * scale search and pack of nvfp4_scale_search with that S (window lo..hi around the base code;
 * ScaleSweep's MSE window is [-3, 7]). Outputs are bit-identical to nvfp4_global_scale followed
 * by nvfp4_scale_search. Up to 2^23 elements (decode and small prefill batches) it runs two
 * kernels instead of three: the search kernel reduces the amax partials itself, which shortens
 * the launch chain of an inference step. Larger tensors take the three-kernel path, which is
 * faster there.
 *
 * X         device, bf16 or f32 [tokens, in], row stride ldx, 16-byte aligned rows.
 * objective NVFP4_MSE, or NVFP4_WMSE with h device float [in] (16-byte aligned).
 * S_out     device float [1] or NULL: receives S.
 * scales    device uint8 [tokens, in/16]; packed device uint8 [tokens, in/2], 8-byte aligned.
 * workspace device, at least nvfp4_quantize_activations_workspace_size(tokens, in) bytes,
 *           16-byte aligned, no initialisation needed.
 * Requires in % 16 == 0 and tokens * in/16 < 2^31.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_quantize_activations_workspace_size(int64_t tokens, int64_t in);

nvfp4_status nvfp4_quantize_activations(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                        int64_t ldx, int objective, const float* h, int32_t lo,
                                        int32_t hi, int rule, float* S_out, uint8_t* scales,
                                        uint8_t* packed, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* ---------------------------------------------------------------------------------------------
 * nvfp4_quantize_activations without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Arguments, outputs and errors are those of
 * nvfp4_quantize_activations (outputs bit-identical), minus the workspace.
 *
 * Scratch: a 4096-byte device array in the library, one copy per GPU, held until the process
 * ends; the call uses the copy of the device current at the call (the device `stream` belongs
 * to must be current). The activation call needs at most 2304 bytes of it (the S slot and at
 * most 512 amax partials), whatever the tensor's size; a need above 4096 bytes would return
 * NVFP4_ERR_WORKSPACE. Every call overwrites the scratch bytes it reads, so nothing needs
 * clearing, but all calls on one GPU share the one array: calls that overlap in time on one GPU
 * (on different streams, or from different threads) race and must be serialised by the caller.
 * The first call on a device looks the array's device address up once (no allocation); it
 * returns NVFP4_ERR_HIP if that fails.
 * ------------------------------------------------------------------------------------------- */
nvfp4_status nvfp4_quantize_activations_noalloc(const void* X, int x_dtype, int64_t tokens,
                                                int64_t in, int64_t ldx, int objective,
                                                const float* h, int32_t lo, int32_t hi, int rule,
                                                float* S_out, uint8_t* scales, uint8_t* packed,
                                                void* stream);

/* ---------------------------------------------------------------------------------------------
 * Evaluation: layer-output error of a quantised layer ([HS] §3: the layer-output reconstruction
 * criterion; the activation-loss comparison of Min-Max, MSE-guided and Hessian-guided scales).
 *
 *   w_hat[o, i] = sign * fl(level * eff[c]) from packed[o, i/2] (element 2k in the low nibble)
 *                 and scales[o, i/16], eff[c] = fl(S[0] * E4M3(c)); scale byte 0 gives zeros
 *   err[o]      = sum_t (sum_i x[t, i] * (w[o, i] - w_hat[o, i]))^2   (+ err[o] if accumulate)
 *
 * Computed on MFMA: E = fl(w - w_hat) in binary32 is split into two bf16 matrices E_hi + E_lo
 * (16 significant bits of E), Y = X E_hi^T + X E_lo^T is accumulated in binary32, and the
 * squares of Y are summed per row, over each 256-token tile in binary32 and over tiles in
 * binary64. Deterministic. Relative to the exact binary64 value, err[o] agrees to about 1e-5
 * for activations and residuals without extreme cancellation (the tests use 1e-4).
 *
 * X         device, bf16 [tokens, in], row stride ldx (multiple of 8), 16-byte aligned.
 * W         device, bf16 or f32 [out, in], row stride ldw (16-byte aligned rows), the weights
 *           that were quantised.
 * scales    device, uint8 [out, in/16], codes 0..126; packed device, uint8 [out, in/2],
 *           4-byte aligned; S device float [1] (the global scale the codes were made with).
 * err       device, double [out], 8-byte aligned; written, or added to when accumulate != 0
 *           (token chunks of one calibration set).
 * workspace device, at least nvfp4_output_error_workspace_size(tokens, out, in) bytes,
 *           16-byte aligned, no initialisation needed (holds E_hi, E_lo and the tile partials).
 * Requires in % 16 == 0 and ceil(out/256) * ceil(tokens/256) < 2^31. tokens == 0 or in == 0
 * only writes err.
 * ------------------------------------------------------------------------------------------- */
size_t nvfp4_output_error_workspace_size(int64_t tokens, int64_t out, int64_t in);

nvfp4_status nvfp4_output_error(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                int64_t ldx, const void* W, int w_dtype, int64_t out, int64_t ldw,
                                const uint8_t* scales, const uint8_t* packed, const float* S,
                                double* err, int accumulate, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
