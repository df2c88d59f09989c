// C ABI (include/nvfp4.h): argument validation on the host, then kernel launches on the
// caller's stream. Every check runs before anything is enqueued, so argument errors never
// leave work behind.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/nvfp4.h"
#include "internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

nvfp4::ScaleSource given_scale(const float* S) {
    nvfp4::ScaleSource src;
    src.S = S;
    return src;
}

int elem_size(int dtype) {
    if (dtype == NVFP4_DTYPE_F32) return 4;
    if (dtype == NVFP4_DTYPE_BF16) return 2;
    return 0;
}

nvfp4_status hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Largest element span an operand may cover (rows x leading dimension, matrices x matrix
// stride): every element offset the kernels form then stays far inside int64.
constexpr int64_t kMaxSpan = (int64_t)1 << 56;
bool span_ok(int64_t rows, int64_t ld) {
    return ld <= kMaxSpan && (rows <= 1 || ld <= kMaxSpan / rows);
}

// Matrix operand [batch, out, in] with row stride ldw and matrix stride stride_w (elements).
nvfp4_status check_weights(const void* W, int dtype, int64_t batch, int64_t out, int64_t in,
                           int64_t ldw, int64_t stride_w) {
    const int esz = elem_size(dtype);
    if (esz == 0) return NVFP4_ERR_DTYPE;
    if (batch < 0 || out < 0 || in < 0) return NVFP4_ERR_SHAPE;
    if (in % 16 != 0) return NVFP4_ERR_SHAPE;
    if (ldw < in) return NVFP4_ERR_SHAPE;
    if (!span_ok(out, ldw) || (batch > 1 && !span_ok(batch, stride_w))) return NVFP4_ERR_SHAPE;
    if (batch > 1 && stride_w < out * ldw) return NVFP4_ERR_SHAPE;
    if (batch > 65535) return NVFP4_ERR_SHAPE;
    if (out * (in / 16) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
    if (batch == 0 || out == 0 || in == 0) return NVFP4_OK;
    if (W == nullptr) return NVFP4_ERR_NULL;
    if (!aligned16(W) || (ldw * esz) % 16 != 0 || (batch > 1 && (stride_w * esz) % 16 != 0))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
    switch (status) {
        case NVFP4_OK: return "NVFP4_OK";
        case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
        case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: invalid size, leading dimension or stride";
        case NVFP4_ERR_DTYPE: return "NVFP4_ERR_DTYPE: unknown element type";
        case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: pointer or stride not 16-byte aligned";
        case NVFP4_ERR_WINDOW: return "NVFP4_ERR_WINDOW: window needs -125 <= lo <= 0 <= hi <= 125";
        case NVFP4_ERR_ARG: return "NVFP4_ERR_ARG: invalid argument";
        case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE: workspace missing or too small";
        case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: HIP runtime error";
        default: return "NVFP4: unknown status";
    }
}

const char* nvfp4_version(void) { return "nvfp4-gfx950 1.0"; }

size_t nvfp4_diag_hessian_workspace_size(int64_t tokens, int64_t in, int64_t segments) {
    if (tokens < 0 || in < 0 || segments < 1) return 0;
    return nvfp4::hessian_workspace_bytes(tokens, in, segments);
}

static nvfp4_status diag_hessian_impl(const void* X, int x_dtype, const int64_t* seg_offsets,
                                      int64_t segments, int64_t tokens, int64_t in, int64_t ldx,
                                      double* h_acc, float* h, int accumulate, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    const int esz = elem_size(x_dtype);
    if (esz == 0) return NVFP4_ERR_DTYPE;
    if (tokens < 0 || in < 0 || segments < 1) return NVFP4_ERR_SHAPE;
    if (in % 8 != 0 || ldx < in || ldx % 8 != 0 || !span_ok(tokens, ldx)) return NVFP4_ERR_SHAPE;
    if (segments > 1 && segments >= ((int64_t)1 << 24)) return NVFP4_ERR_SHAPE;
    if (in == 0) return NVFP4_OK;
    // h_acc == h == NULL on one segment: deferred accumulation into the workspace
    const bool deferred = h_acc == nullptr && h == nullptr && seg_offsets == nullptr;
    if (h_acc == nullptr && !deferred) return NVFP4_ERR_NULL;
    if (tokens > 0 && X == nullptr) return NVFP4_ERR_NULL;
    if (seg_offsets == nullptr && segments > 1) return NVFP4_ERR_NULL;
    if ((X && !aligned16(X)) || (h_acc && !aligned8(h_acc)) ||
        (h && (reinterpret_cast<uintptr_t>(h) & 3u)))
        return NVFP4_ERR_ALIGN;
    if (nvfp4::hessian_launch_blocks(tokens, in, segments, x_dtype == NVFP4_DTYPE_BF16) >=
        ((int64_t)1 << 31))
        return NVFP4_ERR_SHAPE;
    const size_t need = nvfp4::hessian_workspace_bytes(tokens, in, segments);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    if (deferred && tokens > 0 && (workspace == nullptr || need == 0)) return NVFP4_ERR_WORKSPACE;
    return hip_status(nvfp4::launch_diag_hessian(
        X, x_dtype == NVFP4_DTYPE_BF16, tokens, in, ldx, segments > 1 ? seg_offsets : nullptr,
        segments, h_acc, h, accumulate != 0, workspace, static_cast<hipStream_t>(stream),
        deferred ? nvfp4::HessianPass::kPartial : nvfp4::HessianPass::kBoth));
}

nvfp4_status nvfp4_diag_hessian(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                int64_t ldx, double* h_acc, float* h, int accumulate,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return diag_hessian_impl(X, x_dtype, nullptr, 1, tokens, in, ldx, h_acc, h, accumulate,
                             workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_diag_hessian_finalize(int x_dtype, int64_t tokens, int64_t in, double* h_acc,
                                         float* h, int accumulate, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    const int esz = elem_size(x_dtype);
    if (esz == 0) return NVFP4_ERR_DTYPE;
    if (tokens < 0 || in < 0 || in % 8 != 0) return NVFP4_ERR_SHAPE;
    if (in == 0) return NVFP4_OK;
    if (h_acc == nullptr) return NVFP4_ERR_NULL;
    if (!aligned8(h_acc) || (h && (reinterpret_cast<uintptr_t>(h) & 3u))) return NVFP4_ERR_ALIGN;
    const size_t need = nvfp4::hessian_workspace_bytes(tokens, in, 1);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_diag_hessian(
        nullptr, x_dtype == NVFP4_DTYPE_BF16, tokens, in, in, nullptr, 1, h_acc, h,
        accumulate != 0, workspace, static_cast<hipStream_t>(stream),
        nvfp4::HessianPass::kFinalize));
}

nvfp4_status nvfp4_diag_hessian_batched(const void* X, int x_dtype, const int64_t* seg_offsets,
                                        int64_t segments, int64_t total_tokens, int64_t in,
                                        int64_t ldx, double* h_acc, float* h, int accumulate,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    if (segments < 1) return NVFP4_ERR_SHAPE;
    if (seg_offsets == nullptr) return NVFP4_ERR_NULL;
    if (segments == 1) {
        // one segment: its rows are [seg_offsets[0], seg_offsets[1]) = [0, total_tokens)
        return diag_hessian_impl(X, x_dtype, nullptr, 1, total_tokens, in, ldx, h_acc, h,
                                 accumulate, workspace, workspace_bytes, stream);
    }
    return diag_hessian_impl(X, x_dtype, seg_offsets, segments, total_tokens, in, ldx, h_acc, h,
                             accumulate, workspace, workspace_bytes, stream);
}

size_t nvfp4_diag_hessian_chunks_workspace_size(const int64_t* tokens, int64_t n_chunks,
                                                int64_t in) {
    if (tokens == nullptr || n_chunks < 1 || n_chunks > nvfp4::kMaxHessianChunks || in < 0)
        return 0;
    for (int64_t c = 0; c < n_chunks; ++c)
        if (tokens[c] < 0) return 0;
    return nvfp4::hessian_chunks_workspace_bytes(tokens, n_chunks, in);
}

nvfp4_status nvfp4_diag_hessian_chunks(const void* const* X_chunks, int x_dtype,
                                       const int64_t* tokens, int64_t n_chunks, int64_t in,
                                       int64_t ldx, double* h_acc, float* h, int accumulate,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (elem_size(x_dtype) == 0) return NVFP4_ERR_DTYPE;
    if (X_chunks == nullptr || tokens == nullptr) return NVFP4_ERR_NULL;
    if (n_chunks < 1 || n_chunks > nvfp4::kMaxHessianChunks || in < 0) return NVFP4_ERR_SHAPE;
    if (in % 8 != 0 || ldx < in || ldx % 8 != 0) return NVFP4_ERR_SHAPE;
    for (int64_t c = 0; c < n_chunks; ++c) {
        if (tokens[c] < 0 || !span_ok(tokens[c], ldx)) return NVFP4_ERR_SHAPE;
        if (tokens[c] > 0 && in > 0 && X_chunks[c] == nullptr) return NVFP4_ERR_NULL;
        if (X_chunks[c] && !aligned16(X_chunks[c])) return NVFP4_ERR_ALIGN;
    }
    if (in == 0) return NVFP4_OK;
    if (h_acc == nullptr) return NVFP4_ERR_NULL;
    if (!aligned8(h_acc) || (h && (reinterpret_cast<uintptr_t>(h) & 3u))) return NVFP4_ERR_ALIGN;
    const bool bf16 = x_dtype == NVFP4_DTYPE_BF16;
    if (nvfp4::hessian_chunks_launch_blocks(tokens, n_chunks, in, bf16) >= ((int64_t)1 << 31))
        return NVFP4_ERR_SHAPE;
    const size_t need = nvfp4::hessian_chunks_workspace_bytes(tokens, n_chunks, in);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_diag_hessian_chunks(X_chunks, bf16, tokens, n_chunks, in, ldx,
                                                        h_acc, h, accumulate != 0, workspace,
                                                        static_cast<hipStream_t>(stream)));
}

size_t nvfp4_global_scale_workspace_size(int64_t batch, int64_t out, int64_t in) {
    if (batch < 0 || out < 0 || in < 0) return 0;
    return nvfp4::global_scale_workspace_bytes(batch, out, in);
}

nvfp4_status nvfp4_global_scale(const void* W, int w_dtype, int64_t batch, int64_t out,
                                int64_t in, int64_t ldw, int64_t stride_w, int rule, float* S,
                                void* workspace, size_t workspace_bytes, void* stream) {
    nvfp4_status st = check_weights(W, w_dtype, batch, out, in, ldw, stride_w);
    if (st != NVFP4_OK) return st;
    if (rule != NVFP4_GS_AMAX_448 && rule != NVFP4_GS_AMAX_256) return NVFP4_ERR_ARG;
    if (batch == 0) return NVFP4_OK;
    if (S == nullptr) return NVFP4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(S) & 3u) return NVFP4_ERR_ALIGN;
    const size_t need = nvfp4::global_scale_workspace_bytes(batch, out, in);
    if (workspace == nullptr || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 3u) return NVFP4_ERR_ALIGN;
    // Empty matrices reach the kernels too: the reduction sees no element and S = 1.
    return hip_status(nvfp4::launch_global_scale(W, w_dtype == NVFP4_DTYPE_BF16, batch, out, in,
                                                 ldw, stride_w, rule, S, workspace,
                                                 static_cast<hipStream_t>(stream)));
}

size_t nvfp4_layer_statistics_workspace_size(int64_t tokens, int64_t in, int64_t out) {
    if (tokens < 0 || in < 0 || out < 0) return 0;
    return nvfp4::layer_statistics_workspace_bytes(tokens, in, out);
}

nvfp4_status nvfp4_layer_statistics(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                    int64_t ldx, double* h_acc, float* h, int accumulate,
                                    const void* W, int w_dtype, int64_t out, int64_t ldw, int rule,
                                    float* S, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (elem_size(x_dtype) == 0) return NVFP4_ERR_DTYPE;
    if (tokens < 0 || in < 0 || out < 0) return NVFP4_ERR_SHAPE;
    if (in % 8 != 0 || ldx < in || ldx % 8 != 0 || !span_ok(tokens, ldx)) return NVFP4_ERR_SHAPE;
    nvfp4_status st = check_weights(W, w_dtype, 1, out, in, ldw, 0);
    if (st != NVFP4_OK) return st;
    if (rule != NVFP4_GS_AMAX_448 && rule != NVFP4_GS_AMAX_256) return NVFP4_ERR_ARG;
    if (in == 0) return NVFP4_OK;
    if (h_acc == nullptr || S == nullptr) return NVFP4_ERR_NULL;
    if (tokens > 0 && X == nullptr) return NVFP4_ERR_NULL;
    if ((X && !aligned16(X)) || !aligned8(h_acc) || (h && (reinterpret_cast<uintptr_t>(h) & 3u)) ||
        (reinterpret_cast<uintptr_t>(S) & 3u))
        return NVFP4_ERR_ALIGN;
    if (nvfp4::hessian_launch_blocks(tokens, in, 1, x_dtype == NVFP4_DTYPE_BF16) +
            nvfp4::amax_partial_count(1, out, in) >=
        ((int64_t)1 << 31))
        return NVFP4_ERR_SHAPE;
    const size_t need = nvfp4::layer_statistics_workspace_bytes(tokens, in, out);
    if (workspace == nullptr || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_layer_statistics(
        X, x_dtype == NVFP4_DTYPE_BF16, tokens, in, ldx, h_acc, h, accumulate != 0, W,
        w_dtype == NVFP4_DTYPE_BF16, out, ldw, rule, S, workspace,
        static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_scale_search(const void* W, int w_dtype, int64_t batch, int64_t out,
                                int64_t in, int64_t ldw, int64_t stride_w, int32_t group_size,
                                const float* h, int64_t stride_h, int objective, int32_t lo,
                                int32_t hi, int exhaustive, const float* S, uint8_t* scales,
                                uint8_t* packed, float* loss, int8_t* offset, void* stream) {
    if (group_size != 16) return NVFP4_ERR_ARG;
    if (objective != NVFP4_MSE && objective != NVFP4_WMSE) return NVFP4_ERR_ARG;
    if (!exhaustive && (lo > 0 || hi < 0 || lo < -125 || hi > 125)) return NVFP4_ERR_WINDOW;
    nvfp4_status st = check_weights(W, w_dtype, batch, out, in, ldw, stride_w);
    if (st != NVFP4_OK) return st;
    const bool wmse = objective == NVFP4_WMSE;
    if (wmse) {
        if (stride_h < 0 || (batch > 1 && stride_h < in) || stride_h % 4 != 0) return NVFP4_ERR_SHAPE;
    }
    if (batch == 0 || out == 0 || in == 0) return NVFP4_OK;
    if (S == nullptr || scales == nullptr || packed == nullptr) return NVFP4_ERR_NULL;
    if (wmse && h == nullptr) return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(S) & 3u) || !aligned8(packed) ||
        (loss && (reinterpret_cast<uintptr_t>(loss) & 3u)) || (wmse && !aligned16(h)))
        return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_scale_search(
        W, w_dtype == NVFP4_DTYPE_BF16, batch, out, in, ldw, stride_w, wmse ? h : nullptr,
        wmse ? stride_h : 0, wmse, lo, hi, exhaustive != 0, given_scale(S), scales, packed, loss,
        offset, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_scale_search_scored(const void* W, int w_dtype, int64_t batch, int64_t out,
                                       int64_t in, int64_t ldw, int64_t stride_w,
                                       int32_t group_size, const float* h, int64_t stride_h,
                                       int objective, int32_t centre_lo, const float* S,
                                       uint64_t* count, void* stream) {
    if (group_size != 16) return NVFP4_ERR_ARG;
    if (objective != NVFP4_MSE && objective != NVFP4_WMSE) return NVFP4_ERR_ARG;
    if (centre_lo < -15 || centre_lo > 0) return NVFP4_ERR_WINDOW;
    nvfp4_status st = check_weights(W, w_dtype, batch, out, in, ldw, stride_w);
    if (st != NVFP4_OK) return st;
    const bool wmse = objective == NVFP4_WMSE;
    if (wmse) {
        if (stride_h < 0 || (batch > 1 && stride_h < in) || stride_h % 4 != 0) return NVFP4_ERR_SHAPE;
    }
    if (batch == 0 || out == 0 || in == 0) return NVFP4_OK;
    if (S == nullptr || count == nullptr) return NVFP4_ERR_NULL;
    if (wmse && h == nullptr) return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(S) & 3u) || !aligned8(count) || (wmse && !aligned16(h)))
        return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_exhaustive_scored(
        W, w_dtype == NVFP4_DTYPE_BF16, batch, out, in, ldw, stride_w, wmse ? h : nullptr,
        wmse ? stride_h : 0, wmse, centre_lo, S, count, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_scale_search_rules(const void* W, int w_dtype, int64_t batch, int64_t out,
                                      int64_t in, int64_t ldw, int64_t stride_w,
                                      int32_t group_size, const float* h, int64_t stride_h,
                                      const float* S, const nvfp4_search_rule* rules,
                                      int32_t n_rules, void* stream) {
    constexpr int kMaxRules = 64;
    if (group_size != 16) return NVFP4_ERR_ARG;
    if (rules == nullptr) return NVFP4_ERR_NULL;
    if (n_rules < 1 || n_rules > kMaxRules) return NVFP4_ERR_ARG;
    bool any_wmse = false;
    for (int k = 0; k < n_rules; ++k) {
        const nvfp4_search_rule& r = rules[k];
        if (r.objective != NVFP4_MSE && r.objective != NVFP4_WMSE) return NVFP4_ERR_ARG;
        if (!r.exhaustive && (r.lo > 0 || r.hi < 0 || r.lo < -125 || r.hi > 125))
            return NVFP4_ERR_WINDOW;
        any_wmse = any_wmse || r.objective == NVFP4_WMSE;
    }
    nvfp4_status st = check_weights(W, w_dtype, batch, out, in, ldw, stride_w);
    if (st != NVFP4_OK) return st;
    if (any_wmse) {
        if (stride_h < 0 || (batch > 1 && stride_h < in) || stride_h % 4 != 0) return NVFP4_ERR_SHAPE;
    }
    if (batch == 0 || out == 0 || in == 0) return NVFP4_OK;
    if (S == nullptr || (any_wmse && h == nullptr)) return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(S) & 3u) || (any_wmse && !aligned16(h))) return NVFP4_ERR_ALIGN;
    nvfp4::SearchRule rs[kMaxRules];
    for (int k = 0; k < n_rules; ++k) {
        const nvfp4_search_rule& r = rules[k];
        if (r.scales == nullptr || r.packed == nullptr) return NVFP4_ERR_NULL;
        if (!aligned8(r.packed) || (r.loss && (reinterpret_cast<uintptr_t>(r.loss) & 3u)))
            return NVFP4_ERR_ALIGN;
        rs[k] = nvfp4::SearchRule{r.objective == NVFP4_WMSE, r.lo, r.hi, r.exhaustive != 0,
                                  nvfp4::RuleOut{r.scales, r.packed, r.loss, r.offset}};
    }
    return hip_status(nvfp4::launch_scale_search_rules(
        W, w_dtype == NVFP4_DTYPE_BF16, batch, out, in, ldw, stride_w, any_wmse ? h : nullptr,
        any_wmse ? stride_h : 0, S, rs, n_rules, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_scale_search_proposal(const void* W, int w_dtype, int64_t batch, int64_t out,
                                         int64_t in, int64_t ldw, int64_t stride_w,
                                         int32_t group_size, const float* h, int64_t stride_h,
                                         int objective, int32_t lo, int32_t hi,
                                         const uint8_t* center, const uint8_t* incoming,
                                         const float* S, uint8_t* scales, uint8_t* packed,
                                         float* loss, int8_t* offset, void* stream) {
    if (group_size != 16) return NVFP4_ERR_ARG;
    if (objective != NVFP4_MSE && objective != NVFP4_WMSE) return NVFP4_ERR_ARG;
    if (lo > 0 || hi < 0 || lo < -125 || hi > 125) return NVFP4_ERR_WINDOW;
    nvfp4_status st = check_weights(W, w_dtype, batch, out, in, ldw, stride_w);
    if (st != NVFP4_OK) return st;
    const bool wmse = objective == NVFP4_WMSE;
    if (wmse) {
        if (stride_h < 0 || (batch > 1 && stride_h < in) || stride_h % 4 != 0) return NVFP4_ERR_SHAPE;
    }
    if (batch == 0 || out == 0 || in == 0) return NVFP4_OK;
    if (S == nullptr || scales == nullptr || packed == nullptr || center == nullptr)
        return NVFP4_ERR_NULL;
    if (wmse && h == nullptr) return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(S) & 3u) || !aligned8(packed) ||
        (loss && (reinterpret_cast<uintptr_t>(loss) & 3u)) || (wmse && !aligned16(h)))
        return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_scale_search(
        W, w_dtype == NVFP4_DTYPE_BF16, batch, out, in, ldw, stride_w, wmse ? h : nullptr,
        wmse ? stride_h : 0, wmse, lo, hi, false, given_scale(S), scales, packed, loss, offset,
        center, incoming, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_pack(const void* W, int w_dtype, int64_t batch, int64_t out, int64_t in,
                        int64_t ldw, int64_t stride_w, const uint8_t* scales, const float* S,
                        uint8_t* packed, void* stream) {
    nvfp4_status st = check_weights(W, w_dtype, batch, out, in, ldw, stride_w);
    if (st != NVFP4_OK) return st;
    if (batch == 0 || out == 0 || in == 0) return NVFP4_OK;
    if (S == nullptr || scales == nullptr || packed == nullptr) return NVFP4_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(S) & 3u) || !aligned8(packed)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_pack(W, w_dtype == NVFP4_DTYPE_BF16, batch, out, in, ldw,
                                         stride_w, scales, S, packed,
                                         static_cast<hipStream_t>(stream)));
}

// On-line activation quantisation: up to kFusedElems elements the search kernel reduces the
// amax partials itself (two kernels); above, the per-workgroup reduction of the partials costs
// more than the launch it saves (measured on MI355X), so the global scale runs as its own two
// kernels and the search reads S. Both give the same bits.
constexpr int64_t kFusedElems = (int64_t)1 << 23;

size_t nvfp4_quantize_activations_workspace_size(int64_t tokens, int64_t in) {
    if (tokens < 0 || in < 0) return 0;
    // [S slot, 256 B][amax partials]
    return 256 + (size_t)nvfp4::amax_partial_count(1, tokens, in) * sizeof(uint32_t);
}

}  // extern "C"

namespace {

// Validation and launches shared by nvfp4_quantize_activations and its allocation-free variant;
// `workspace` holds [S slot, 256 B][amax partials] of the size
// nvfp4_quantize_activations_workspace_size returns (already checked by the caller).
nvfp4_status check_activations(const void* X, int x_dtype, int64_t tokens, int64_t in,
                               int64_t ldx, int objective, const float* h, int32_t lo, int32_t hi,
                               int rule, const float* S_out, const uint8_t* scales,
                               const uint8_t* packed) {
    if (objective != NVFP4_MSE && objective != NVFP4_WMSE) return NVFP4_ERR_ARG;
    if (rule != NVFP4_GS_AMAX_448 && rule != NVFP4_GS_AMAX_256) return NVFP4_ERR_ARG;
    if (lo > 0 || hi < 0 || lo < -125 || hi > 125) return NVFP4_ERR_WINDOW;
    nvfp4_status st = check_weights(X, x_dtype, 1, tokens, in, ldx, 0);
    if (st != NVFP4_OK) return st;
    if (tokens == 0 || in == 0) return NVFP4_OK;
    const bool wmse = objective == NVFP4_WMSE;
    if (scales == nullptr || packed == nullptr || (wmse && h == nullptr)) return NVFP4_ERR_NULL;
    if (!aligned8(packed) || (S_out && (reinterpret_cast<uintptr_t>(S_out) & 3u)) ||
        (wmse && !aligned16(h)))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

nvfp4_status launch_activations(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                int64_t ldx, int objective, const float* h, int32_t lo,
                                int32_t hi, int rule, float* S_out, uint8_t* scales,
                                uint8_t* packed, void* workspace, void* stream) {
    const bool wmse = objective == NVFP4_WMSE;
    const bool bf16 = x_dtype == NVFP4_DTYPE_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* S_slot = static_cast<float*>(workspace);
    uint32_t* partial = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + 256);
    nvfp4::ScaleSource src;
    if (tokens * in <= kFusedElems) {
        hipError_t e = nvfp4::launch_amax_partial(X, bf16, 1, tokens, in, ldx, tokens * ldx,
                                                  partial, s);
        if (e != hipSuccess) return hip_status(e);
        src.amax_partial = partial;
        src.n_partial = nvfp4::amax_partial_count(1, tokens, in);
        src.rule = rule;
        src.S_out = S_out;
    } else {
        float* S = S_out ? S_out : S_slot;
        hipError_t e = nvfp4::launch_global_scale(X, bf16, 1, tokens, in, ldx, tokens * ldx, rule,
                                                  S, partial, s);
        if (e != hipSuccess) return hip_status(e);
        src.S = S;
    }
    return hip_status(nvfp4::launch_scale_search(X, bf16, 1, tokens, in, ldx, tokens * ldx,
                                                 wmse ? h : nullptr, 0, wmse, lo, hi, false, src,
                                                 scales, packed, nullptr, nullptr, nullptr,
                                                 nullptr, s));
}

// Scratch of nvfp4_quantize_activations_noalloc, one copy per GPU for the life of the process:
// the S slot (256 B) and the amax partials (at most 512 x 4 B), the same layout as the caller's
// workspace of nvfp4_quantize_activations.
constexpr size_t kNoAllocScratchBytes = 4096;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// In host code `scratch` names a host-side stand-in for the symbol, not a device address: the
// address of each GPU's copy is looked up once per device, with that device current, and kept.
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_status[kMaxScratchDevices];

hipError_t current_device_scratch(void** ptr) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_ptr[dev] != nullptr ? g_scratch_status[dev] : hipErrorInvalidSymbol;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize_activations(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                        int64_t ldx, int objective, const float* h, int32_t lo,
                                        int32_t hi, int rule, float* S_out, uint8_t* scales,
                                        uint8_t* packed, void* workspace, size_t workspace_bytes,
                                        void* stream) {
    const nvfp4_status st = check_activations(X, x_dtype, tokens, in, ldx, objective, h, lo, hi,
                                              rule, S_out, scales, packed);
    if (st != NVFP4_OK || tokens == 0 || in == 0) return st;
    const size_t need = nvfp4_quantize_activations_workspace_size(tokens, in);
    if (workspace == nullptr || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    return launch_activations(X, x_dtype, tokens, in, ldx, objective, h, lo, hi, rule, S_out,
                              scales, packed, workspace, stream);
}

nvfp4_status nvfp4_quantize_activations_noalloc(const void* X, int x_dtype, int64_t tokens,
                                                int64_t in, int64_t ldx, int objective,
                                                const float* h, int32_t lo, int32_t hi, int rule,
                                                float* S_out, uint8_t* scales, uint8_t* packed,
                                                void* stream) {
    const nvfp4_status st = check_activations(X, x_dtype, tokens, in, ldx, objective, h, lo, hi,
                                              rule, S_out, scales, packed);
    if (st != NVFP4_OK || tokens == 0 || in == 0) return st;
    if (nvfp4_quantize_activations_workspace_size(tokens, in) > kNoAllocScratchBytes)
        return NVFP4_ERR_WORKSPACE;
    void* ws = nullptr;
    if (current_device_scratch(&ws) != hipSuccess) return NVFP4_ERR_HIP;
    return launch_activations(X, x_dtype, tokens, in, ldx, objective, h, lo, hi, rule, S_out,
                              scales, packed, ws, stream);
}

size_t nvfp4_gptq_workspace_size(int64_t out, int64_t in) {
    if (out < 0 || in < 0) return 0;
    return nvfp4::gptq_workspace_bytes(out, in);
}

nvfp4_status nvfp4_gptq(const void* W, int w_dtype, int64_t out, int64_t in, int64_t ldw,
                        const float* U, const float* h, int objective, int32_t lo, int32_t hi,
                        const float* S, uint8_t* scales, uint8_t* packed, float* W_final,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (objective != NVFP4_MSE && objective != NVFP4_WMSE) return NVFP4_ERR_ARG;
    if (lo > 0 || hi < 0 || lo < -125 || hi > 125) return NVFP4_ERR_WINDOW;
    nvfp4_status st = check_weights(W, w_dtype, 1, out, in, ldw, 0);
    if (st != NVFP4_OK) return st;
    if (out * in >= ((int64_t)1 << 39)) return NVFP4_ERR_SHAPE;
    if ((out + 31) / 32 > 65535) return NVFP4_ERR_SHAPE;   // row tiles of the update grid
    if (out == 0 || in == 0) return NVFP4_OK;
    const bool wmse = objective == NVFP4_WMSE;
    if (U == nullptr || S == nullptr || scales == nullptr || packed == nullptr ||
        (wmse && h == nullptr))
        return NVFP4_ERR_NULL;
    if (!aligned16(U) || (reinterpret_cast<uintptr_t>(S) & 3u) || !aligned8(packed) ||
        (h && (reinterpret_cast<uintptr_t>(h) & 3u)) || (W_final && !aligned16(W_final)))
        return NVFP4_ERR_ALIGN;
    const size_t need = nvfp4::gptq_workspace_bytes(out, in);
    if (workspace == nullptr || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_gptq(W, w_dtype == NVFP4_DTYPE_BF16, out, in, ldw, U,
                                         wmse ? h : nullptr, wmse, lo, hi, S, scales, packed,
                                         W_final, workspace, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_output_error_workspace_size(int64_t tokens, int64_t out, int64_t in) {
    if (tokens < 0 || out < 0 || in < 0) return 0;
    return nvfp4::output_error_workspace_bytes(tokens, out, in);
}

nvfp4_status nvfp4_output_error(const void* X, int x_dtype, int64_t tokens, int64_t in,
                                int64_t ldx, const void* W, int w_dtype, int64_t out, int64_t ldw,
                                const uint8_t* scales, const uint8_t* packed, const float* S,
                                double* err, int accumulate, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (x_dtype != NVFP4_DTYPE_BF16) return NVFP4_ERR_DTYPE;
    nvfp4_status st = check_weights(W, w_dtype, 1, out, in, ldw, 0);
    if (st != NVFP4_OK) return st;
    if (tokens < 0 || ldx < in || ldx % 8 != 0 || !span_ok(tokens, ldx)) return NVFP4_ERR_SHAPE;
    if (nvfp4::output_error_tiles(tokens, out) >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
    if (out == 0) return NVFP4_OK;
    if (err == nullptr) return NVFP4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(err) & 7u) return NVFP4_ERR_ALIGN;
    // with no tokens or no columns there are no terms: the kernels then only write err
    // (0, or its old value when accumulating) and read nothing else
    if (tokens > 0 && in > 0) {
        if (X == nullptr || scales == nullptr || packed == nullptr || S == nullptr)
            return NVFP4_ERR_NULL;
        if (!aligned16(X) || (reinterpret_cast<uintptr_t>(packed) & 3u) ||
            (reinterpret_cast<uintptr_t>(S) & 3u))
            return NVFP4_ERR_ALIGN;
    }
    const size_t need = nvfp4::output_error_workspace_bytes(tokens, out, in);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    return hip_status(nvfp4::launch_output_error(X, tokens, in, ldx, W,
                                                 w_dtype == NVFP4_DTYPE_BF16, out, ldw, scales,
                                                 packed, S, err, accumulate != 0, workspace,
                                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
