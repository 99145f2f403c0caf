// C ABI of libuno: argument validation, workspace checks and dispatch to the
// kernel launchers.  Every check runs on the host before anything is
// enqueued, so a rejected call leaves the stream untouched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/uno.h"
#include "uno_internal.h"

namespace {

thread_local std::string g_last_error;

uno_status fail(uno_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

uno_status ok() {
    g_last_error.clear();
    return UNO_OK;
}

uno_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(UNO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

constexpr int64_t kMaxGridX = 2147483647LL;

uno_status check_workspace(void* ws, size_t have, size_t need) {
    if (need == 0) return UNO_OK;
    if (ws == nullptr) return fail(UNO_ERR_WORKSPACE, "workspace is null but %zu bytes are required", need);
    if (!aligned256(ws)) return fail(UNO_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (have < need) return fail(UNO_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", have, need);
    return UNO_OK;
}

}  // namespace

extern "C" {

int32_t uno_abi_version(void) { return UNO_ABI_VERSION; }

const char* uno_status_string(int32_t status) {
    switch (status) {
        case UNO_OK: return "UNO_OK";
        case UNO_ERR_INVALID_ARG: return "UNO_ERR_INVALID_ARG";
        case UNO_ERR_UNSUPPORTED: return "UNO_ERR_UNSUPPORTED";
        case UNO_ERR_WORKSPACE: return "UNO_ERR_WORKSPACE";
        case UNO_ERR_HIP: return "UNO_ERR_HIP";
        default: return "UNO_ERR_UNKNOWN";
    }
}

const char* uno_last_error_message(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ Philox
uno_status uno_philox_uniforms(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n, float* out,
                               hipStream_t stream) {
    if (n < 0) return fail(UNO_ERR_INVALID_ARG, "n must be >= 0 (got %lld)", static_cast<long long>(n));
    if (n == 0) return ok();
    if (out == nullptr) return fail(UNO_ERR_INVALID_ARG, "out is null");
    if (static_cast<uint64_t>(n) - 1u > ~offset) return fail(UNO_ERR_INVALID_ARG, "offset + n exceeds 2^64");
    const uint64_t blocks4 = ((offset + static_cast<uint64_t>(n) - 1u) >> 2) - (offset >> 2) + 1u;
    if ((blocks4 + 255u) / 256u > static_cast<uint64_t>(kMaxGridX))
        return fail(UNO_ERR_UNSUPPORTED, "n too large for one launch");
    return from_hip(uno::philox_uniforms_launch(seed, stream_id, offset, n, out, stream), "philox launch");
}

// ------------------------------------------------------------------ gated LoRA
static uno_status check_gemm(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dtype) {
    if (dtype != UNO_BF16 && dtype != UNO_F32) return fail(UNO_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (M < 0 || N < 1 || K < 1) return fail(UNO_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1");
    if (M > 2147483647LL - 64 || N > 2147483647LL || K > 2147483647LL)
        return fail(UNO_ERR_UNSUPPORTED, "sizes must fit in 31 bits");
    if (r < 1 || r > 256) return fail(UNO_ERR_UNSUPPORTED, "rank r must be in [1, 256] (got %d)", r);
    if (dtype == UNO_BF16) {
        if (K % 8 != 0) return fail(UNO_ERR_UNSUPPORTED, "bf16 path needs K %% 8 == 0 (got %lld)", static_cast<long long>(K));
        if (r % 8 != 0) return fail(UNO_ERR_UNSUPPORTED, "bf16 path needs r %% 8 == 0 (got %d)", r);
        const int64_t rows_cap = (M + 31) / 32 * 32 + 32;
        if (M * K >= (1LL << 30) || N * K >= (1LL << 30) || rows_cap * r >= (1LL << 30))
            return fail(UNO_ERR_UNSUPPORTED, "bf16 operands must stay under 2^30 elements each");
        // byte offsets of the rows one tile reads past N (or past r) stay
        // under 2^32, where the copy engine's range check still sees them
        if ((N + 256) * K >= (1LL << 31) || (r + 256) * K >= (1LL << 31) || (N + 256) * r >= (1LL << 31))
            return fail(UNO_ERR_UNSUPPORTED, "operand rows past a tile edge would overflow 32-bit offsets");
        if (((rows_cap + 63) / 64) * ((N + 127) / 128) > kMaxGridX)
            return fail(UNO_ERR_UNSUPPORTED, "problem too large for the tile grid");
    } else {
        if (M * N > kMaxGridX * 256 || M * r > kMaxGridX * 256) return fail(UNO_ERR_UNSUPPORTED, "problem too large for the fp32 path");
    }
    return UNO_OK;
}

size_t uno_gated_lora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dtype) {
    if (check_gemm(M, N, K, r, dtype) != UNO_OK) return 0;
    ok();
    return uno::gated_lora_workspace_size(M, N, K, r, dtype == UNO_BF16);
}

uno_status uno_gated_lora_fwd(const void* x, const void* w, const void* lora_a, const void* lora_b,
                              const uint8_t* gate, void* y, int64_t M, int64_t N, int64_t K, int32_t r,
                              float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    uno_status st = check_gemm(M, N, K, r, dtype);
    if (st != UNO_OK) return st;
    if (!std::isfinite(scale)) return fail(UNO_ERR_INVALID_ARG, "scale must be finite");
    if (M == 0) return ok();
    if (!x || !w || !lora_a || !lora_b || !gate || !y) return fail(UNO_ERR_INVALID_ARG, "null tensor pointer");
    if (dtype == UNO_BF16) {
        if (!aligned16(x) || !aligned16(w) || !aligned16(lora_a) || !aligned16(lora_b))
            return fail(UNO_ERR_INVALID_ARG, "bf16 inputs must be 16-byte aligned");
        if (!aligned16(y)) return fail(UNO_ERR_INVALID_ARG, "y must be 16-byte aligned");
    } else {
        if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(lora_a) |
             reinterpret_cast<uintptr_t>(lora_b) | reinterpret_cast<uintptr_t>(y)) & 3u)
            return fail(UNO_ERR_INVALID_ARG, "fp32 tensors must be 4-byte aligned");
    }
    const size_t need = uno::gated_lora_workspace_size(M, N, K, r, dtype == UNO_BF16);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st != UNO_OK) return st;
    uno::GemmProblem p{x, w, lora_a, lora_b, gate, y, M, N, K, r, scale, dtype == UNO_BF16};
    return from_hip(uno::gated_lora_launch(p, workspace, workspace_bytes, stream), "gated lora launch");
}

// ------------------------------------------------------------------ split projection steps
size_t uno_row_plan_size(int64_t M) {
    if (M < 0 || M > 2147483647LL - 64) return 0;
    ok();
    return uno::row_plan_bytes(M);
}

uno_status uno_segment_rows(const uint8_t* gate, int64_t M, void* row_plan, size_t row_plan_bytes,
                            hipStream_t stream) {
    if (M < 0 || M > 2147483647LL - 64) return fail(UNO_ERR_INVALID_ARG, "M must be in [0, 2^31 - 64)");
    if (row_plan == nullptr) return fail(UNO_ERR_INVALID_ARG, "row_plan is null");
    if (!aligned256(row_plan)) return fail(UNO_ERR_INVALID_ARG, "row_plan must be 256-byte aligned");
    if (row_plan_bytes < uno::row_plan_bytes(M))
        return fail(UNO_ERR_WORKSPACE, "row_plan has %zu bytes, %zu required", row_plan_bytes, uno::row_plan_bytes(M));
    if (M > 0 && gate == nullptr) return fail(UNO_ERR_INVALID_ARG, "gate is null");
    return from_hip(uno::segment_rows_launch(gate, M, row_plan, stream), "segment rows launch");
}

uno_status uno_row_plan_gate_errors(const void* row_plan, int32_t* out, hipStream_t stream) {
    if (row_plan == nullptr || out == nullptr) return fail(UNO_ERR_INVALID_ARG, "row_plan and out must not be null");
    if (!aligned256(row_plan)) return fail(UNO_ERR_INVALID_ARG, "row_plan must be 256-byte aligned");
    if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0) return fail(UNO_ERR_INVALID_ARG, "out must be 4-byte aligned");
    const char* src = static_cast<const char*>(row_plan) + uno::row_plan_gate_error_offset();
    return from_hip(hipMemcpyAsync(out, src, 2 * sizeof(int32_t), hipMemcpyDeviceToDevice, stream),
                    "gate error copy");
}

// T may hold several adapters side by side (their A rows stacked): its width
// is the sum of their ranks.
static uno_status check_lora_t(int64_t M, int64_t K, int32_t rt) {
    if (rt < 8 || rt > 1024 || rt % 8 != 0)
        return fail(UNO_ERR_UNSUPPORTED, "T width must be a multiple of 8 in [8, 1024] (got %d)", rt);
    const uno_status st = check_gemm(M, rt, K, 8, UNO_BF16);
    if (st != UNO_OK) return st;
    if (((M + 31) / 32 * 32 + 32) * rt >= (1LL << 30))
        return fail(UNO_ERR_UNSUPPORTED, "T must stay under 2^30 elements");
    return UNO_OK;
}

size_t uno_lora_t_size(int64_t M, int32_t r) {
    if (check_lora_t(M, 8, r) != UNO_OK) return 0;
    ok();
    return uno::lora_t_bytes(M, r);
}

size_t uno_lora_down_workspace_size(int64_t M, int64_t K, int32_t r) {
    if (check_lora_t(M, K, r) != UNO_OK) return 0;
    ok();
    return uno::lora_down_workspace_size(M, K, r);
}

uno_status uno_lora_down(const void* x, const void* lora_a, const void* row_plan, void* t, int64_t M, int64_t K,
                         int32_t r, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    uno_status st = check_lora_t(M, K, r);
    if (st != UNO_OK) return st;
    if (!std::isfinite(scale)) return fail(UNO_ERR_INVALID_ARG, "scale must be finite");
    if (M == 0) return ok();
    if (!x || !lora_a || !row_plan || !t) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(lora_a) || !aligned16(t) || !aligned256(row_plan))
        return fail(UNO_ERR_INVALID_ARG, "x, lora_a and t must be 16-byte aligned, row_plan 256-byte aligned");
    st = check_workspace(workspace, workspace_bytes, uno::lora_down_workspace_size(M, K, r));
    if (st != UNO_OK) return st;
    return from_hip(uno::lora_down_launch(x, lora_a, row_plan, t, M, K, r, scale, workspace, stream),
                    "lora down launch");
}

size_t uno_gated_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (check_gemm(M, N, K, r, UNO_BF16) != UNO_OK) return 0;
    ok();
    return uno::gated_gemm_workspace_size(M, K, &N, 1);
}

uno_status uno_gated_gemm(const void* x, const void* w, const void* t, const void* lora_b, const void* row_plan,
                          void* y, int64_t M, int64_t N, int64_t K, int32_t r, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    return uno_gated_gemm_grouped(x, w, t, lora_b, row_plan, &y, &N, 1, M, K, r, workspace, workspace_bytes, stream);
}

size_t uno_gated_gemm_residual_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (check_gemm(M, N, K, r, UNO_BF16) != UNO_OK) return 0;
    ok();
    return uno::gated_gemm_workspace_size(M, K, &N, 1, 1);
}

uno_status uno_gated_gemm_residual(const void* x, const void* w, const void* t, const void* lora_b,
                                   const void* row_plan, void* y, int64_t M, int64_t N, int64_t K, int32_t r,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    uno_status st = check_gemm(M, N, K, r, UNO_BF16);
    if (st != UNO_OK) return st;
    if (M == 0) return ok();
    if (!x || !w || !t || !lora_b || !row_plan || !y) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(w) || !aligned16(t) || !aligned16(lora_b) || !aligned16(y) ||
        !aligned256(row_plan))
        return fail(UNO_ERR_INVALID_ARG, "tensors must be 16-byte aligned, row_plan 256-byte aligned");
    st = check_workspace(workspace, workspace_bytes, uno::gated_gemm_workspace_size(M, K, &N, 1, 1));
    if (st != UNO_OK) return st;
    void* ys[1] = {y};
    return from_hip(uno::gated_gemm_launch(x, w, t, lora_b, row_plan, ys, &N, 1, M, K, r, workspace, stream, 1),
                    "gated gemm (residual) launch");
}

static uno_status check_swiglu(int64_t M, int64_t N_half, int64_t K, int32_t rt) {
    if (N_half < 128 || N_half % 128 != 0)
        return fail(UNO_ERR_UNSUPPORTED, "N_half must be a positive multiple of 128 (got %lld)",
                    static_cast<long long>(N_half));
    if (N_half > (1LL << 30)) return fail(UNO_ERR_UNSUPPORTED, "N_half too large");
    uno_status st = check_gemm(M, 2 * N_half, K, rt, UNO_BF16);
    if (st != UNO_OK) return st;
    return check_lora_t(M, K, rt);
}

size_t uno_gated_gemm_swiglu_workspace_size(int64_t M, int64_t N_half, int64_t K, int32_t rt) {
    if (check_swiglu(M, N_half, K, rt) != UNO_OK) return 0;
    ok();
    const int64_t N = 2 * N_half;
    return uno::gated_gemm_workspace_size(M, K, &N, 1, 2);
}

uno_status uno_gated_gemm_swiglu(const void* x, const void* w_packed, const void* t, const void* b_packed,
                                 const void* row_plan, void* act, int64_t M, int64_t N_half, int64_t K, int32_t rt,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    uno_status st = check_swiglu(M, N_half, K, rt);
    if (st != UNO_OK) return st;
    if (M == 0) return ok();
    if (!x || !w_packed || !t || !b_packed || !row_plan || !act)
        return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(w_packed) || !aligned16(t) || !aligned16(b_packed) || !aligned16(act) ||
        !aligned256(row_plan))
        return fail(UNO_ERR_INVALID_ARG, "tensors must be 16-byte aligned, row_plan 256-byte aligned");
    int64_t N = 2 * N_half;
    st = check_workspace(workspace, workspace_bytes, uno::gated_gemm_workspace_size(M, K, &N, 1, 2));
    if (st != UNO_OK) return st;
    void* ys[1] = {act};
    return from_hip(uno::gated_gemm_launch(x, w_packed, t, b_packed, row_plan, ys, &N, 1, M, K, rt, workspace,
                                           stream, 2),
                    "gated gemm (SwiGLU) launch");
}

uno_status uno_swiglu_pack(const void* w_gate, const void* w_up, const void* b_gate, const void* b_up,
                           int64_t N_half, int64_t K, int32_t r, void* w_packed, void* b_packed, hipStream_t stream) {
    if (N_half < 128 || N_half % 128 != 0)
        return fail(UNO_ERR_UNSUPPORTED, "N_half must be a positive multiple of 128");
    if (K < 8 || K % 8 != 0 || r < 8 || r % 8 != 0 || r > 512)
        return fail(UNO_ERR_UNSUPPORTED, "need K and r multiples of 8, r in [8, 512]");
    if (N_half > (1LL << 30) || K > (1LL << 30)) return fail(UNO_ERR_UNSUPPORTED, "sizes too large");
    if (!w_gate || !w_up || !b_gate || !b_up || !w_packed || !b_packed)
        return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(b_gate) || !aligned16(b_up) || !aligned16(w_packed) ||
        !aligned16(b_packed))
        return fail(UNO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    return from_hip(uno::swiglu_pack_launch(w_gate, w_up, b_gate, b_up, N_half, K, r, w_packed, b_packed, stream),
                    "swiglu pack launch");
}

static uno_status check_groups(const int64_t* group_n, int32_t n_groups, int64_t M, int64_t K, int32_t r,
                               int64_t* N_out) {
    if (group_n == nullptr) return fail(UNO_ERR_INVALID_ARG, "group_n is null");
    if (n_groups < 1 || n_groups > 4) return fail(UNO_ERR_UNSUPPORTED, "n_groups must be in [1, 4] (got %d)", n_groups);
    int64_t N = 0;
    for (int32_t g = 0; g < n_groups; ++g) {
        if (group_n[g] < 1 || group_n[g] > 2147483647LL) return fail(UNO_ERR_INVALID_ARG, "group %d has %lld columns", g,
                                                                    static_cast<long long>(group_n[g]));
        N += group_n[g];
    }
    if (!uno::gated_gemm_groups_ok(group_n, n_groups))
        return fail(UNO_ERR_UNSUPPORTED, "every group but the last must have a multiple of 128 columns");
    uno_status st = check_gemm(M, N, K, r, UNO_BF16);
    if (st != UNO_OK) return st;
    if (n_groups > 1) {
        st = check_lora_t(M, K, r * n_groups);
        if (st != UNO_OK) return st;
    }
    *N_out = N;
    return UNO_OK;
}

size_t uno_gated_gemm_grouped_workspace_size(int64_t M, int64_t K, int32_t r, const int64_t* group_n,
                                             int32_t n_groups) {
    int64_t N = 0;
    if (check_groups(group_n, n_groups, M, K, r, &N) != UNO_OK) return 0;
    ok();
    return uno::gated_gemm_workspace_size(M, K, group_n, n_groups);
}

uno_status uno_gated_gemm_grouped(const void* x, const void* w, const void* t, const void* lora_b,
                                  const void* row_plan, void* const* y, const int64_t* group_n, int32_t n_groups,
                                  int64_t M, int64_t K, int32_t r, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    int64_t N = 0;
    uno_status st = check_groups(group_n, n_groups, M, K, r, &N);
    if (st != UNO_OK) return st;
    if (M == 0) return ok();
    if (!x || !w || !t || !lora_b || !row_plan || !y) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(w) || !aligned16(t) || !aligned16(lora_b) || !aligned256(row_plan))
        return fail(UNO_ERR_INVALID_ARG, "tensors must be 16-byte aligned, row_plan 256-byte aligned");
    for (int32_t g = 0; g < n_groups; ++g) {
        if (y[g] == nullptr) return fail(UNO_ERR_INVALID_ARG, "output %d is null", g);
        if (!aligned16(y[g])) return fail(UNO_ERR_INVALID_ARG, "output %d must be 16-byte aligned", g);
    }
    st = check_workspace(workspace, workspace_bytes, uno::gated_gemm_workspace_size(M, K, group_n, n_groups));
    if (st != UNO_OK) return st;
    return from_hip(uno::gated_gemm_launch(x, w, t, lora_b, row_plan, y, group_n, n_groups, M, K, r, workspace,
                                           stream),
                    "gated gemm launch");
}

// ------------------------------------------------------------------ verification
static uno_status check_logits(int64_t B, int32_t L, int64_t V, float T, int32_t dtype) {
    if (dtype != UNO_BF16 && dtype != UNO_F32) return fail(UNO_ERR_INVALID_ARG, "unknown logits dtype %d", dtype);
    if (B < 0) return fail(UNO_ERR_INVALID_ARG, "B must be >= 0");
    if (L < 1) return fail(UNO_ERR_INVALID_ARG, "L must be >= 1");
    if (V < 1 || V > 2147483647LL) return fail(UNO_ERR_INVALID_ARG, "V must be in [1, 2^31)");
    if (!(T > 0.0f) || !std::isfinite(T)) return fail(UNO_ERR_UNSUPPORTED, "temperature must be positive and finite");
    return UNO_OK;
}

size_t uno_block_verify_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus) {
    if (B < 0 || L < 1 || L > 64 || V < 1) return 0;
    ok();
    return uno::verify_workspace_size(B, L, V, has_bonus ? 1 : 0);
}

// noalloc: the workspace is the library's own per-device scratch array (the
// caller passes none); sizes past it are rejected before anything runs.
static uno_status block_verify_common(const void* target_logits, const void* draft_logits, int64_t target_seq_stride,
                                      int64_t draft_seq_stride, const int32_t* draft_tokens, const float* uniforms,
                                      int64_t B, int32_t L, int64_t V, int32_t has_bonus, float temperature,
                                      int32_t logits_dtype, int32_t* n_accepted, int32_t* out_tokens,
                                      int32_t* n_emitted, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, int32_t chunk, bool noalloc = false) {
    uno_status st = check_logits(B, L, V, temperature, logits_dtype);
    if (st != UNO_OK) return st;
    if (has_bonus != 0 && has_bonus != 1) return fail(UNO_ERR_INVALID_ARG, "has_bonus must be 0 or 1");
    if (L > 64 || (has_bonus && L > 63))
        return fail(UNO_ERR_UNSUPPORTED, "block length must be <= 64 (<= 63 with a bonus row)");
    if (target_seq_stride < 0 || draft_seq_stride < 0) return fail(UNO_ERR_INVALID_ARG, "strides must be >= 0");
    if (B == 0) return ok();
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !n_accepted || !out_tokens || !n_emitted)
        return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    const size_t esz = logits_dtype == UNO_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(target_logits) | reinterpret_cast<uintptr_t>(draft_logits)) % esz)
        return fail(UNO_ERR_INVALID_ARG, "logits must be aligned to their element size");
    const int64_t rows = B * (L + has_bonus);
    const int64_t max_chunks = (V + 2047) / 2048;
    if (rows * max_chunks > kMaxGridX || B > kMaxGridX) return fail(UNO_ERR_UNSUPPORTED, "problem too large for one launch");
    const size_t need = chunk > 0 ? uno::verify_early_workspace_size(B, L, V, has_bonus)
                                  : uno::verify_workspace_size(B, L, V, has_bonus);
    if (noalloc) {
        if (need > uno::noalloc_scratch_bytes())
            return fail(UNO_ERR_UNSUPPORTED,
                        "B = %lld, L = %d, V = %lld needs %zu bytes of scratch; the no-allocation entry point "
                        "holds %zu (use uno_block_verify with a workspace)",
                        static_cast<long long>(B), L, static_cast<long long>(V), need, uno::noalloc_scratch_bytes());
        const hipError_t e = uno::noalloc_scratch(&workspace);
        if (e != hipSuccess) return from_hip(e, "scratch symbol address");
        workspace_bytes = uno::noalloc_scratch_bytes();
    }
    st = check_workspace(workspace, workspace_bytes, need);
    if (st != UNO_OK) return st;
    uno::VerifyProblem p{};
    p.target = target_logits;
    p.draft = draft_logits;
    p.t_stride = target_seq_stride;
    p.d_stride = draft_seq_stride;
    p.tokens = draft_tokens;
    p.uniforms = uniforms;
    p.B = B;
    p.L = L;
    p.V = V;
    p.has_bonus = has_bonus;
    p.temperature = temperature;
    p.bf16 = logits_dtype == UNO_BF16;
    p.n_accepted = n_accepted;
    p.out_tokens = out_tokens;
    p.n_emitted = n_emitted;
    return from_hip(uno::block_verify_launch(p, workspace, stream, chunk), "block verify launch");
}

uno_status uno_block_verify(const void* target_logits, const void* draft_logits, int64_t target_seq_stride,
                            int64_t draft_seq_stride, const int32_t* draft_tokens, const float* uniforms, int64_t B,
                            int32_t L, int64_t V, int32_t has_bonus, float temperature, int32_t logits_dtype,
                            int32_t* n_accepted, int32_t* out_tokens, int32_t* n_emitted, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    return block_verify_common(target_logits, draft_logits, target_seq_stride, draft_seq_stride, draft_tokens,
                               uniforms, B, L, V, has_bonus, temperature, logits_dtype, n_accepted, out_tokens,
                               n_emitted, workspace, workspace_bytes, stream, 0);
}

uno_status uno_block_verify_noalloc(const void* target_logits, const void* draft_logits, int64_t target_seq_stride,
                                    int64_t draft_seq_stride, const int32_t* draft_tokens, const float* uniforms,
                                    int64_t B, int32_t L, int64_t V, int32_t has_bonus, float temperature,
                                    int32_t logits_dtype, int32_t* n_accepted, int32_t* out_tokens,
                                    int32_t* n_emitted, hipStream_t stream) {
    return block_verify_common(target_logits, draft_logits, target_seq_stride, draft_seq_stride, draft_tokens,
                               uniforms, B, L, V, has_bonus, temperature, logits_dtype, n_accepted, out_tokens,
                               n_emitted, nullptr, 0, stream, 0, true);
}

size_t uno_block_verify_noalloc_max_bytes(void) { return uno::noalloc_scratch_bytes(); }

size_t uno_block_verify_early_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus) {
    if (B < 0 || L < 1 || L > 64 || V < 1) return 0;
    ok();
    return uno::verify_early_workspace_size(B, L, V, has_bonus ? 1 : 0);
}

uno_status uno_block_verify_early(const void* target_logits, const void* draft_logits, int64_t target_seq_stride,
                                  int64_t draft_seq_stride, const int32_t* draft_tokens, const float* uniforms,
                                  int64_t B, int32_t L, int64_t V, int32_t has_bonus, float temperature,
                                  int32_t logits_dtype, int32_t chunk, int32_t* n_accepted, int32_t* out_tokens,
                                  int32_t* n_emitted, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (chunk < 1 || chunk > 64) return fail(UNO_ERR_INVALID_ARG, "chunk must be in [1, 64] (got %d)", chunk);
    return block_verify_common(target_logits, draft_logits, target_seq_stride, draft_seq_stride, draft_tokens,
                               uniforms, B, L, V, has_bonus, temperature, logits_dtype, n_accepted, out_tokens,
                               n_emitted, workspace, workspace_bytes, stream, chunk);
}

size_t uno_draft_sample_workspace_size(int64_t B, int32_t L, int64_t V) {
    if (B < 0 || L < 1 || V < 1) return 0;
    ok();
    return uno::draft_sample_workspace_size(B, L, V);
}

uno_status uno_draft_sample(const void* draft_logits, int64_t seq_stride, const float* uniforms, int64_t B, int32_t L,
                            int64_t V, float temperature, int32_t logits_dtype, int32_t* tokens, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    uno_status st = check_logits(B, L, V, temperature, logits_dtype);
    if (st != UNO_OK) return st;
    if (seq_stride < 0) return fail(UNO_ERR_INVALID_ARG, "seq_stride must be >= 0");
    if (B == 0) return ok();
    if (!draft_logits || !uniforms || !tokens) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    const size_t esz = logits_dtype == UNO_BF16 ? 2 : 4;
    if (reinterpret_cast<uintptr_t>(draft_logits) % esz)
        return fail(UNO_ERR_INVALID_ARG, "logits must be aligned to their element size");
    const int64_t rows = B * L;
    const int64_t max_chunks = (V + 2047) / 2048;
    if (rows * max_chunks > kMaxGridX) return fail(UNO_ERR_UNSUPPORTED, "problem too large for one launch");
    const size_t need = uno::draft_sample_workspace_size(B, L, V);
    st = check_workspace(workspace, workspace_bytes, need);
    if (st != UNO_OK) return st;
    uno::VerifyProblem p{};
    p.draft = draft_logits;
    p.d_stride = seq_stride;
    p.uniforms = uniforms;
    p.B = B;
    p.L = L;
    p.V = V;
    p.temperature = temperature;
    p.bf16 = logits_dtype == UNO_BF16;
    p.sampled = tokens;
    return from_hip(uno::draft_sample_launch(p, workspace, stream), "draft sample launch");
}

// ------------------------------------------------------------------ tree verification
static uno_status check_tree(int64_t B, int32_t N, int64_t V, float temperature, int32_t dtype) {
    uno_status st = check_logits(B, 1, V, temperature, dtype);
    if (st != UNO_OK) return st;
    if (N < 1 || N > 4096) return fail(UNO_ERR_UNSUPPORTED, "nodes per tree must be in [1, 4096] (got %d)", N);
    const int64_t max_chunks = (V + 2047) / 2048;
    if (B * N * max_chunks > kMaxGridX || B * N > kMaxGridX)
        return fail(UNO_ERR_UNSUPPORTED, "problem too large for one launch");
    return UNO_OK;
}

size_t uno_tree_verify_workspace_size(int64_t B, int32_t N, int64_t V) {
    if (B < 0 || N < 1 || N > 4096 || V < 1) return 0;
    ok();
    return uno::tree_verify_workspace_size(B, N, V);
}

uno_status uno_tree_verify(const void* node_logits, int64_t seq_stride, const int32_t* parents,
                           const int32_t* tokens, const float* uniforms, int64_t B, int32_t N, int64_t V,
                           float temperature, int32_t logits_dtype, int32_t* n_accepted, int32_t* out_tokens,
                           int32_t* n_emitted, int32_t* last_node, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    uno_status st = check_tree(B, N, V, temperature, logits_dtype);
    if (st != UNO_OK) return st;
    if (seq_stride < 0) return fail(UNO_ERR_INVALID_ARG, "seq_stride must be >= 0");
    if (B == 0) return ok();
    if (!node_logits || !parents || !tokens || !uniforms || !n_accepted || !out_tokens || !n_emitted || !last_node)
        return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    const size_t esz = logits_dtype == UNO_BF16 ? 2 : 4;
    if (reinterpret_cast<uintptr_t>(node_logits) % esz)
        return fail(UNO_ERR_INVALID_ARG, "logits must be aligned to their element size");
    st = check_workspace(workspace, workspace_bytes, uno::tree_verify_workspace_size(B, N, V));
    if (st != UNO_OK) return st;
    uno::TreeProblem p{};
    p.logits = node_logits;
    p.seq_stride = seq_stride;
    p.parents = parents;
    p.tokens = tokens;
    p.uniforms = uniforms;
    p.B = B;
    p.N = N;
    p.V = V;
    p.temperature = temperature;
    p.bf16 = logits_dtype == UNO_BF16;
    p.n_accepted = n_accepted;
    p.out_tokens = out_tokens;
    p.n_emitted = n_emitted;
    p.last_node = last_node;
    return from_hip(uno::tree_verify_launch(p, workspace, stream), "tree verify launch");
}

// ------------------------------------------------------------------ LM head + verification
static uno_status check_lm_head(int64_t B, int32_t L, int64_t V, int64_t K, int32_t has_bonus, float temperature) {
    uno_status st = check_logits(B, L, V, temperature, UNO_BF16);
    if (st != UNO_OK) return st;
    if (has_bonus != 0 && has_bonus != 1) return fail(UNO_ERR_INVALID_ARG, "has_bonus must be 0 or 1");
    if (L > 64 || (has_bonus && L > 63))
        return fail(UNO_ERR_UNSUPPORTED, "block length must be <= 64 (<= 63 with a bonus row)");
    if (K < 1) return fail(UNO_ERR_INVALID_ARG, "K must be >= 1");
    if (B > (1LL << 24)) return fail(UNO_ERR_UNSUPPORTED, "too many sequences");
    const int64_t rows = B * (L + has_bonus) + B * L;
    return check_gemm(rows, V, K, 8, UNO_BF16);
}

size_t uno_lm_head_verify_workspace_size(int64_t B, int32_t L, int64_t V, int64_t K, int32_t has_bonus) {
    if (check_lm_head(B, L, V, K, has_bonus, 1.0f) != UNO_OK) return 0;
    ok();
    return uno::lm_head_verify_workspace_size(B, L, V, has_bonus);
}

uno_status uno_lm_head_verify(const void* hidden, const void* w_lm, int64_t B, int32_t L, int64_t V, int64_t K,
                              int32_t has_bonus, float temperature, const int32_t* draft_tokens,
                              const float* uniforms, int32_t* n_accepted, int32_t* out_tokens, int32_t* n_emitted,
                              void* logits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    uno_status st = check_lm_head(B, L, V, K, has_bonus, temperature);
    if (st != UNO_OK) return st;
    if (B == 0) return ok();
    if (!hidden || !w_lm || !draft_tokens || !uniforms || !n_accepted || !out_tokens || !n_emitted)
        return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(hidden) || !aligned16(w_lm) || (logits != nullptr && !aligned16(logits)))
        return fail(UNO_ERR_INVALID_ARG, "hidden, w_lm and logits must be 16-byte aligned");
    st = check_workspace(workspace, workspace_bytes, uno::lm_head_verify_workspace_size(B, L, V, has_bonus));
    if (st != UNO_OK) return st;
    uno::LmHeadProblem p{};
    p.hidden = hidden;
    p.w = w_lm;
    p.B = B;
    p.L = L;
    p.V = V;
    p.K = K;
    p.has_bonus = has_bonus;
    p.temperature = temperature;
    p.tokens = draft_tokens;
    p.uniforms = uniforms;
    p.n_accepted = n_accepted;
    p.out_tokens = out_tokens;
    p.n_emitted = n_emitted;
    p.logits = logits;
    return from_hip(uno::lm_head_verify_launch(p, workspace, stream), "LM head verify launch");
}

// ------------------------------------------------------------------ glue
uno_status uno_rmsnorm(const void* x, void* y, int64_t M, int64_t K, float eps, int32_t dtype, hipStream_t stream) {
    if (dtype != UNO_BF16) return fail(UNO_ERR_UNSUPPORTED, "rmsnorm supports bf16 only");
    if (M < 0 || K < 0) return fail(UNO_ERR_INVALID_ARG, "sizes must be >= 0");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(UNO_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (M == 0 || K == 0) return ok();
    if (K % 8 != 0 || K > 65536) return fail(UNO_ERR_UNSUPPORTED, "rmsnorm needs K %% 8 == 0 and K <= 65536");
    if (M > kMaxGridX) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
    if (!x || !y) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(y)) return fail(UNO_ERR_INVALID_ARG, "rmsnorm tensors must be 16-byte aligned");
    return from_hip(uno::rmsnorm_launch(x, y, M, K, eps, stream), "rmsnorm launch");
}

uno_status uno_residual_rmsnorm(const void* x, const void* y, void* s_out, void* h, int64_t M, int64_t K, float eps,
                                int32_t dtype, hipStream_t stream) {
    if (dtype != UNO_BF16) return fail(UNO_ERR_UNSUPPORTED, "residual_rmsnorm supports bf16 only");
    if (M < 0 || K < 0) return fail(UNO_ERR_INVALID_ARG, "sizes must be >= 0");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(UNO_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (M == 0 || K == 0) return ok();
    if (K % 8 != 0 || K > 65536)
        return fail(UNO_ERR_UNSUPPORTED, "residual_rmsnorm needs K %% 8 == 0 and K <= 65536");
    if (M > kMaxGridX) return fail(UNO_ERR_UNSUPPORTED, "too many rows");
    if (!x || !y || !s_out || !h) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(x) || !aligned16(y) || !aligned16(s_out) || !aligned16(h))
        return fail(UNO_ERR_INVALID_ARG, "residual_rmsnorm tensors must be 16-byte aligned");
    return from_hip(uno::residual_rmsnorm_launch(x, y, s_out, h, M, K, eps, stream), "residual_rmsnorm launch");
}

static uno_status check_eltwise(const void* a, const void* b, void* out, int64_t n, int32_t dtype) {
    if (dtype != UNO_BF16) return fail(UNO_ERR_UNSUPPORTED, "elementwise glue supports bf16 only");
    if (n < 0) return fail(UNO_ERR_INVALID_ARG, "n must be >= 0");
    if (n == 0) return UNO_OK;
    if (!a || !b || !out) return fail(UNO_ERR_INVALID_ARG, "null pointer argument");
    if (!aligned16(a) || !aligned16(b) || !aligned16(out))
        return fail(UNO_ERR_INVALID_ARG, "elementwise tensors must be 16-byte aligned");
    return UNO_OK;
}

uno_status uno_silu_mul(const void* gate, const void* up, void* out, int64_t n, int32_t dtype, hipStream_t stream) {
    const uno_status st = check_eltwise(gate, up, out, n, dtype);
    if (st != UNO_OK) return st;
    return from_hip(uno::silu_mul_launch(gate, up, out, n, stream), "silu_mul launch");
}

uno_status uno_residual_add(const void* a, const void* b, void* out, int64_t n, int32_t dtype, hipStream_t stream) {
    const uno_status st = check_eltwise(a, b, out, n, dtype);
    if (st != UNO_OK) return st;
    return from_hip(uno::residual_add_launch(a, b, out, n, stream), "residual_add launch");
}

}  // extern "C"
