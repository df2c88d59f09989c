// Launchers shared between the C-ABI layer and the kernel files. Arguments are validated by
// the caller (api.hip); launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// Magic multiplier and shift for div_gpr (device_formats.h): gi / gpr for 0 <= gi < 2^31.
inline void gpr_divisor(int64_t gpr, uint64_t& magic, uint32_t& shift) {
    uint32_t L = 0;
    while (((int64_t)1 << L) < gpr) ++L;
    magic = (((uint64_t)1 << (32 + L)) + (uint64_t)gpr - 1) / (uint64_t)gpr;
    shift = 32 + L;
}

// Diagonal Hessian: workspace bytes and the partial kernel's workgroup count.
size_t hessian_workspace_bytes(int64_t tokens, int64_t in, int64_t segments);
int64_t hessian_launch_blocks(int64_t tokens, int64_t in, int64_t segments, bool bf16);

// kBoth: partial pass then finalize. kPartial: partial pass only, its sums replacing
// (accumulate false) or added to (accumulate true) the workspace slots. kFinalize: finalize of
// the slots only (tokens gives the slot layout of the chunks that filled them).
enum class HessianPass { kBoth, kPartial, kFinalize };

hipError_t launch_diag_hessian(const void* X, bool bf16, int64_t tokens, int64_t in, int64_t ldx,
                               const int64_t* seg_offsets, int64_t segments, double* h_acc,
                               float* h, bool accumulate, void* workspace, hipStream_t stream,
                               HessianPass pass = HessianPass::kBoth);

// Token chunks of one set at separate addresses: one partial launch over all of them, then
// one finalize. Workspace bytes (0 if the plan does not fit) and partial workgroup count.
constexpr int kMaxHessianChunks = 64;
size_t hessian_chunks_workspace_bytes(const int64_t* tokens, int64_t n_chunks, int64_t in);
int64_t hessian_chunks_launch_blocks(const int64_t* tokens, int64_t n_chunks, int64_t in,
                                     bool bf16);
hipError_t launch_diag_hessian_chunks(const void* const* X_chunks, bool bf16,
                                      const int64_t* tokens, int64_t n_chunks, int64_t in,
                                      int64_t ldx, double* h_acc, float* h, bool accumulate,
                                      void* workspace, hipStream_t stream);

size_t global_scale_workspace_bytes(int64_t batch, int64_t out, int64_t in);
hipError_t launch_global_scale(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, int rule, float* S, void* workspace,
                               hipStream_t stream);

// Pass 1 of the global scale alone (per-workgroup partial maxima, amax_partial_count of them
// per matrix), for callers that reduce the partials themselves.
int64_t amax_partial_count(int64_t batch, int64_t out, int64_t in);
hipError_t launch_amax_partial(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, uint32_t* partial,
                               hipStream_t stream);

// How the global-scale pass splits a matrix: nblk workgroups per matrix, each over `chunk`
// 16-byte vectors (vpr per row).
struct AmaxPlan {
    int64_t nblk, chunk, vpr;
};
AmaxPlan amax_plan(int64_t batch, int64_t out, int64_t in, bool bf16);

// Layer statistics: h of X and S of W (one matrix, one token chunk) in two launches, each
// result bit-identical to launch_diag_hessian and launch_global_scale.
size_t layer_statistics_workspace_bytes(int64_t tokens, int64_t in, int64_t out);
hipError_t launch_layer_statistics(const void* X, bool x_bf16, int64_t tokens, int64_t in,
                                   int64_t ldx, double* h_acc, float* h, bool accumulate,
                                   const void* W, bool w_bf16, int64_t out, int64_t ldw, int rule,
                                   float* S, void* workspace, hipStream_t stream);

// Where the search takes S from: S[batch] as given, or (one matrix) reduced in every
// workgroup from the amax partials with the rule, workgroup 0 also writing it to S_out.
struct ScaleSource {
    const float* S = nullptr;
    const uint32_t* amax_partial = nullptr;
    int64_t n_partial = 0;
    int rule = 0;
    float* S_out = nullptr;
};

// center == NULL: plain window (around the base code) or exhaustive search. center != NULL:
// window around center[] with the optional incoming[] code kept on ties (exhaustive false).
hipError_t launch_scale_search(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                               int64_t ldw, int64_t stride_w, const float* h, int64_t stride_h,
                               bool wmse, int lo, int hi, bool exhaustive, ScaleSource src,
                               uint8_t* scales, uint8_t* packed, float* loss, int8_t* offset,
                               const uint8_t* center, const uint8_t* incoming,
                               hipStream_t stream);

// Several search rules over one set of weights: each rule's outputs equal launch_scale_search's
// for that rule alone. Consecutive windowed rules of 11 or 16 codes on bf16 W run in pairs, one
// launch per pair sharing each group's loads, table and base code; the rest run one launch each.
struct RuleOut {
    uint8_t* scales;   // [batch, out, in/16]
    uint8_t* packed;   // [batch, out, in/2]
    float* loss;       // [batch, out, in/16] or null
    int8_t* offset;    // [batch, out, in/16] or null
};
struct SearchRule {
    bool wmse;
    int lo, hi;
    bool exhaustive;
    RuleOut out;
};
hipError_t launch_scale_search_rules(const void* W, bool bf16, int64_t batch, int64_t out,
                                     int64_t in, int64_t ldw, int64_t stride_w, const float* h,
                                     int64_t stride_h, const float* S, const SearchRule* rules,
                                     int n_rules, hipStream_t stream);

// Work count of the exhaustive search (candidates scored), added to *count.
hipError_t launch_exhaustive_scored(const void* W, bool bf16, int64_t batch, int64_t out,
                                   int64_t in, int64_t ldw, int64_t stride_w, const float* h,
                                   int64_t stride_h, bool wmse, int clo, const float* S,
                                   uint64_t* count, hipStream_t stream);

// Layer-output error: workspace bytes (residual halves + token-tile partials) and launch.
size_t output_error_workspace_bytes(int64_t tokens, int64_t out, int64_t in);
int64_t output_error_tiles(int64_t tokens, int64_t out);   // GEMM workgroups
hipError_t launch_output_error(const void* X, int64_t tokens, int64_t in, int64_t ldx,
                               const void* W, bool w_bf16, int64_t out, int64_t ldw,
                               const uint8_t* scales, const uint8_t* packed, const float* S,
                               double* err, bool accumulate, void* workspace, hipStream_t stream);

// GPTQ with the window search as local quantiser: workspace bytes and launch (W_final may be
// NULL; the binary32 working copy then lives in the workspace).
size_t gptq_workspace_bytes(int64_t out, int64_t in);
hipError_t launch_gptq(const void* W, bool bf16, int64_t out, int64_t in, int64_t ldw,
                       const float* U, const float* h, bool wmse, int lo, int hi, const float* S,
                       uint8_t* scales, uint8_t* packed, float* W_final, void* workspace,
                       hipStream_t stream);

hipError_t launch_pack(const void* W, bool bf16, int64_t batch, int64_t out, int64_t in,
                       int64_t ldw, int64_t stride_w, const uint8_t* scales, const float* S,
                       uint8_t* packed, hipStream_t stream);

}  // namespace nvfp4
