// Host-side interface between the C-ABI layer (uno_api.cpp) and the kernel
// translation units.  Every function here assumes its arguments were already
// validated by the C-ABI layer and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace uno {

constexpr size_t kWorkspaceAlign = 256;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- Philox uniforms -------------------------------------------------------
hipError_t philox_uniforms_launch(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n,
                                  float* out, hipStream_t stream);

// ---- verification and draft sampling -----------------------------------------
struct VerifyProblem {
    const void* target;      // rows (s, i) at s * t_stride + i * V
    const void* draft;       // rows (s, i) at s * d_stride + i * V (may be null: draft sampling)
    int64_t t_stride;
    int64_t d_stride;
    const int32_t* tokens;   // [B, L] (verify only)
    const float* uniforms;   // verify: [B, L+1]; draft sampling: [B, L]
    int64_t B;
    int32_t L;
    int64_t V;
    int32_t has_bonus;
    float temperature;
    bool bf16;               // logits dtype
    int32_t* n_accepted;     // verify outputs
    int32_t* out_tokens;
    int32_t* n_emitted;
    int32_t* sampled;        // draft sampling output [B, L]
};

size_t verify_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus);
size_t verify_early_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus);
size_t draft_sample_workspace_size(int64_t B, int32_t L, int64_t V);
// chunk = 0: one pass over every row; chunk > 0: early exit in chunks of positions
hipError_t block_verify_launch(const VerifyProblem& p, void* ws, hipStream_t stream, int32_t chunk = 0);
hipError_t draft_sample_launch(const VerifyProblem& p, void* ws, hipStream_t stream);
// Scratch of the verifier's no-allocation entry point: its size, and its
// device address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

// ---- gated-LoRA projection ----------------------------------------------------
struct GemmProblem {
    const void* x;        // [M, K]
    const void* w;        // [N, K]
    const void* a;        // [r, K]
    const void* b;        // [N, r]
    const uint8_t* gate;  // [M]
    void* y;              // [M, N]
    int64_t M, N, K;
    int32_t r;
    float scale;
    bool bf16;
};

size_t gated_lora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, bool bf16);
hipError_t gated_lora_launch(const GemmProblem& p, void* ws, size_t ws_bytes, hipStream_t stream);

// The three steps of the bf16 projection, exported separately.
size_t row_plan_bytes(int64_t M);
// byte offset in a row plan of int32 {rows with an invalid gate byte, first such row or -1}
size_t row_plan_gate_error_offset();
hipError_t segment_rows_launch(const uint8_t* gate, int64_t M, void* plan, hipStream_t stream);
size_t lora_t_bytes(int64_t M, int32_t r);
size_t lora_down_workspace_size(int64_t M, int64_t K, int32_t r);
hipError_t lora_down_launch(const void* x, const void* lora_a, const void* plan, void* t, int64_t M, int64_t K,
                            int32_t r, float scale, void* ws, hipStream_t stream);
// Output column groups: n_groups in [1, 4], group_n[g] >= 1, every group but
// the last a multiple of 128 columns.
// epi: 0 store, 1 accumulate into y, 2 SwiGLU over 128-column gate / up
// blocks (one group of 2 * N_half interleaved columns; y is [M, N_half]).
bool gated_gemm_groups_ok(const int64_t* group_n, int32_t n_groups);
size_t gated_gemm_workspace_size(int64_t M, int64_t K, const int64_t* group_n, int32_t n_groups, int32_t epi = 0);
hipError_t gated_gemm_launch(const void* x, const void* w, const void* t, const void* lora_b, const void* plan,
                             void* const* ys, const int64_t* group_n, int32_t n_groups, int64_t M, int64_t K,
                             int32_t r, void* ws, hipStream_t stream, int32_t epi = 0);
// Interleave W_gate / W_up [N_half, K] into [2 N_half, K] in 128-row blocks and
// B_gate / B_up [N_half, r] into the block-diagonal [2 N_half, 2 r].
hipError_t swiglu_pack_launch(const void* w_gate, const void* w_up, const void* b_gate, const void* b_up,
                              int64_t N_half, int64_t K, int32_t r, void* w_out, void* b_out, hipStream_t stream);

// ---- tree verification ----------------------------------------------------------
struct TreeProblem {
    const void* logits;      // node (s, n) row at s * seq_stride + n * V
    int64_t seq_stride;
    const int32_t* parents;  // [B, N]
    const int32_t* tokens;   // [B, N]
    const float* uniforms;   // [B, N]: the draw at depth d uses slot d
    int64_t B;
    int32_t N;
    int64_t V;
    float temperature;
    bool bf16;
    int32_t* n_accepted;
    int32_t* out_tokens;     // [B, N]
    int32_t* n_emitted;
    int32_t* last_node;
};
size_t tree_verify_workspace_size(int64_t B, int32_t N, int64_t V);
hipError_t tree_verify_launch(const TreeProblem& p, void* ws, hipStream_t stream);

// ---- LM head fused with the verification statistics ----------------------------
// Row plan, statistics map and gathered tokens of the stacked hidden rows, and
// the (empty) plan of the 2 B redraw rows.
int32_t* row_plan_perm(void* plan);
hipError_t lm_rows_launch(int64_t B, int32_t L, int32_t nb, const int32_t* tokens, void* plan, int32_t* stat_map,
                          int32_t* row_token, void* rc_plan, hipStream_t stream);
// Chunks per row of the statistics (one per 256 columns of the head).
int64_t lm_head_stat_chunks(int64_t V);
// y = x W^T over the M rows of the plan (x holds x_rows rows), bf16 (y may be
// null with stats); with stats (ChunkStat [rows][chunks]) the statistics
// epilogue; out_compact: the output row is the plan position.
hipError_t lm_head_gemm_launch(const void* x, int64_t x_rows, const void* w, const void* plan, int64_t M, int64_t V,
                               int64_t K, void* y, int32_t out_compact, void* stats, const int32_t* stat_map,
                               const int32_t* row_token, float* gathered, float c2, hipStream_t stream);

struct LmHeadProblem {
    const void* hidden;      // bf16 [B (L + nb) + B L, K]: target rows, then draft rows
    const void* w;           // bf16 [V, K]
    int64_t B;
    int32_t L;
    int64_t V, K;
    int32_t has_bonus;
    float temperature;
    const int32_t* tokens;   // [B, L]
    const float* uniforms;   // [B, L + 1]
    int32_t* n_accepted;
    int32_t* out_tokens;
    int32_t* n_emitted;
    void* logits;            // bf16 [rows, V] or null (redraw rows recomputed)
};
size_t lm_head_verify_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus);
hipError_t lm_head_verify_launch(const LmHeadProblem& p, void* ws, hipStream_t stream);

// ---- layer glue ----------------------------------------------------------------
hipError_t rmsnorm_launch(const void* x, void* y, int64_t M, int64_t K, float eps,
                          hipStream_t stream);
hipError_t silu_mul_launch(const void* gate, const void* up, void* out, int64_t n,
                           hipStream_t stream);
hipError_t residual_add_launch(const void* a, const void* b, void* out, int64_t n,
                               hipStream_t stream);
hipError_t residual_rmsnorm_launch(const void* x, const void* y, void* s_out, void* h, int64_t M, int64_t K,
                                  float eps, hipStream_t stream);

}  // namespace uno
