/*
 * uno.h -- C ABI of the Uno hot-path library (libuno.so, gfx950 / MI355X).
 *
 * The method ("Uno", from the pages about "Unlocking Lossless Speedups in LLMs
 * via Discrete Diffusion") adds a rank-128, alpha-256 LoRA pathway to every
 * projection of an autoregressive transformer; draft tokens run the AR
 * weights plus the adapter and verification tokens run the AR weights alone,
 * and a sampler accepts the longest drafted prefix that speculative-style
 * rejection sampling against the AR model allows, keeping the AR output
 * distribution exact.  This library provides the two data-parallel pieces of
 * one draft+verify step -- the gated-LoRA projection and block verification --
 * plus the counter-based uniform generator they consume.
 *
 * Conventions shared by every call
 *  - Pointers named as device memory are caller-owned device allocations; the
 *    library never allocates, frees or retains them.  Scalars are passed by
 *    value.  Work that needs scratch space takes a caller-provided device
 *    workspace whose minimum size comes from the matching *_workspace_size().
 *  - All work is enqueued asynchronously on `stream` (0 = the null stream).
 *    No call synchronises the host.
 *  - Argument errors (null pointers, sizes, dtypes, alignment, workspace) are
 *    detected on the host before anything is launched and returned as a
 *    status; uno_last_error_message() then describes the problem.  A failed
 *    launch returns UNO_ERR_HIP.  Faults inside a kernel surface at the
 *    caller's next synchronisation, as for any HIP kernel.
 *  - Device-side precondition failures never trap: they are reported through
 *    sentinel values documented per call.
 *  - Two calls that share a workspace must not overlap in time.
 */
#ifndef UNO_H_
#define UNO_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum uno_status {
    UNO_OK = 0,
    UNO_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, bad alignment */
    UNO_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported domain            */
    UNO_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size()    */
    UNO_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed               */
} uno_status;

typedef enum uno_dtype {
    UNO_BF16 = 0, /* bfloat16, round-to-nearest-even on output */
    UNO_F32 = 1   /* IEEE binary32                             */
} uno_dtype;

/* ABI revision of this header; bumped on any incompatible change. */
#define UNO_ABI_VERSION 1
int32_t uno_abi_version(void);

/* Static text for a status code (never NULL). */
const char* uno_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling host thread
 * (empty string if none).  The pointer stays valid until the next call. */
const char* uno_last_error_message(void);

/* ------------------------------------------------------------------------
 * Counter-based uniforms (Philox4x32-10; Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11).  The rejection sampler of the pages
 * ("The Psi-Spec Sampler" on the aifromscratch.in page) needs one uniform per
 * acceptance test and one per redraw; they are generated here and passed to
 * uno_block_verify / uno_draft_sample as plain inputs.
 *
 *   out[j] = (w >> 8) * 2^-24,  j in [0, n),
 *   w = word ((offset + j) % 4) of Philox4x32-10 with
 *       key     = (seed mod 2^32, seed >> 32),
 *       counter = (b mod 2^32, b >> 32, stream_id mod 2^32, stream_id >> 32),
 *       b       = (offset + j) / 4.
 * Every value lies in [0, 1 - 2^-24] and is exact in binary32.  One call over
 * [0, n) equals two calls over [0, k) and [k, n).
 *
 * out : device float[n].  n = 0 is a no-op.  offset + n must not exceed 2^64.
 * ------------------------------------------------------------------------ */
uno_status uno_philox_uniforms(uint64_t seed, uint64_t stream_id, uint64_t offset, int64_t n,
                               float* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gated-LoRA projection ("Two Decoupled Weight Sets" on the aifromscratch.in
 * page; "How Uno works" on the cctest.ai page): frozen AR weights W_AR plus a
 * LoRA adapter (A, B) of rank r, applied only on draft rows:
 *
 *   y[m, :] = x[m, :] W_AR + gate[m] * scale * (x[m, :] A) B
 *
 * with scale = alpha / r (2.0 for r = 128, alpha = 256).  Storage follows the
 * nn.Linear convention, all row-major:
 *   x      [M, K]   activations (dtype)
 *   w      [N, K]   W_AR transposed (dtype)
 *   lora_a [r, K]   A transposed (dtype)
 *   lora_b [N, r]   B transposed (dtype)
 *   gate   [M]      uint8, 1 = draft row, 0 = verify row
 *   y      [M, N]   output (dtype); must not alias any input
 * Arithmetic: products accumulate in fp32.  For UNO_BF16 the adapter's
 * intermediate scale * (x A) is rounded once to bf16, and y is rounded to
 * bf16 (nearest even).  UNO_F32 keeps every intermediate in fp32.
 * Rows with gate 0 run exactly the instruction sequence of a call whose gates
 * are all 0, so they are bitwise identical to it.
 *
 * Domain: M >= 0 (M = 0 is a no-op), N >= 1, K >= 1, 1 <= r <= 256 and scale
 * finite.  UNO_BF16 additionally needs K and r multiples of 8, 16-byte
 * aligned tensors, and every operand under 2 GiB (M*K, N*K < 2^30 elements).
 * Gate bytes other than 0 and 1 are a caller error that never passes
 * silently: such a row runs neither pathway, its output row is written as
 * NaN (every column), and the row plan at the start of the workspace counts
 * it -- uno_row_plan_gate_errors(workspace, ...) reports the count and the
 * first such row.
 * workspace: device memory of at least uno_gated_lora_workspace_size() bytes
 * (256-byte aligned); it begins with the call's row plan (both dtypes).
 *
 * For UNO_BF16 the call runs three steps, also exported below so that many
 * projections over the same rows (a layer stack) can plan the rows once:
 *   uno_segment_rows   rows -> a row plan (stable partition by gate into
 *                      [verify | draft], each part padded to 32 rows)
 *   uno_lora_down      T = scale * (x A) on the draft rows (bf16, plan order)
 *   uno_gated_gemm     y = x W_AR, plus T B on the draft rows
 * ------------------------------------------------------------------------ */
size_t uno_gated_lora_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r, int32_t dtype);
uno_status uno_gated_lora_fwd(const void* x, const void* w, const void* lora_a,
                              const void* lora_b, const uint8_t* gate, void* y,
                              int64_t M, int64_t N, int64_t K, int32_t r, float scale,
                              int32_t dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Row plan: opaque device buffer of uno_row_plan_size(M) bytes (256-byte
 * aligned) written by uno_segment_rows from gate [M] (device uint8).  It stays
 * valid while the gate values are unchanged.  Rows whose gate byte is neither
 * 0 nor 1 are kept out of both pathways and counted in the plan; every gated
 * GEMM launched with the plan writes NaN into their output rows. */
size_t uno_row_plan_size(int64_t M);
uno_status uno_segment_rows(const uint8_t* gate, int64_t M, void* row_plan, size_t row_plan_bytes,
                            hipStream_t stream);

/* Gate check of a row plan ("Two Decoupled Weight Sets" on the
 * aifromscratch.in page: a token runs the draft pathway or the verification
 * pathway, nothing else).  Enqueues on `stream` a copy into out (device
 * int32[2]) of {number of rows whose gate byte was neither 0 nor 1, the first
 * such row or -1}, as seen by the uno_segment_rows (or uno_gated_lora_fwd,
 * whose workspace starts with its plan) that last wrote row_plan with M >= 1.
 * row_plan 256-byte aligned, out 4-byte aligned; null pointers are
 * UNO_ERR_INVALID_ARG. */
uno_status uno_row_plan_gate_errors(const void* row_plan, int32_t* out, hipStream_t stream);

/* LoRA down-projection on draft rows (bf16): t receives scale * (x A) for the
 * draft rows in plan order, zero rows for padding; t is a device buffer of
 * uno_lora_t_size(M, r) bytes.  x [M, K], lora_a [r, K].  Same domain as
 * uno_gated_lora_fwd with UNO_BF16, except that r here is the width of T: a
 * multiple of 8 up to 1024, so that the A matrices of several projections
 * that read the same x can be stacked ([A_q; A_k; A_v]) and their T computed
 * in one call, side by side. */
size_t uno_lora_t_size(int64_t M, int32_t r);
size_t uno_lora_down_workspace_size(int64_t M, int64_t K, int32_t r);
uno_status uno_lora_down(const void* x, const void* lora_a, const void* row_plan, void* t, int64_t M,
                         int64_t K, int32_t r, float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Gated GEMM (bf16): y = x W_AR for every row plus T B for the draft rows of
 * the plan, T from uno_lora_down with the same plan and rank.  x [M, K],
 * w [N, K], lora_b [N, r], y [M, N] (must not alias inputs). */
size_t uno_gated_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r);
uno_status uno_gated_gemm(const void* x, const void* w, const void* t, const void* lora_b,
                          const void* row_plan, void* y, int64_t M, int64_t N, int64_t K, int32_t r,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Grouped gated GEMM (bf16): several projections that read the same x (q, k
 * and v of a layer; its gate and up) in one launch, each with its own LoRA
 * adapter.  Group g has group_n[g] output columns; w [N, K] and lora_b [N, r]
 * hold the groups' rows one after another (N = sum of group_n); t is the
 * output of uno_lora_down over the stacked A matrices (width n_groups * r),
 * whose columns [g*r, (g+1)*r) belong to group g; y is a host array of
 * n_groups device pointers, y[g] a row-major [M, group_n[g]] output.  The
 * result is that of uno_gated_gemm on each group alone up to the order of the
 * fp32 sums (the launch plan depends on the total width: it may split K, or
 * use a tile whose two wavefront groups sum alternate K steps apart); with
 * the same plan it is bitwise the same.
 * Domain: as uno_gated_gemm, with 1 <= n_groups <= 4 and every group but
 * the last a multiple of 128 columns (UNO_ERR_UNSUPPORTED otherwise).
 * group_n and y are read before the call returns. */
size_t uno_gated_gemm_grouped_workspace_size(int64_t M, int64_t K, int32_t r, const int64_t* group_n,
                                             int32_t n_groups);
uno_status uno_gated_gemm_grouped(const void* x, const void* w, const void* t, const void* lora_b,
                                  const void* row_plan, void* const* y, const int64_t* group_n,
                                  int32_t n_groups, int64_t M, int64_t K, int32_t r, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Gated GEMM with the residual add in its epilogue: y <- y + P, P the
 * uno_gated_gemm result, for a projection that feeds the residual stream of
 * its layer (the pages put the LoRA pathway into each transformer layer --
 * "How It Works: The 'Uno' Architecture" on the aifromscratch.in page).  P is
 * rounded to bf16 first and the sum is rounded again, so y is bitwise
 * uno_residual_add(y, P).  y [M, N] is read and written in place (it must
 * not alias x, w, t or lora_b); other arguments and the domain as
 * uno_gated_gemm. */
size_t uno_gated_gemm_residual_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r);
uno_status uno_gated_gemm_residual(const void* x, const void* w, const void* t, const void* lora_b,
                                   const void* row_plan, void* y, int64_t M, int64_t N, int64_t K, int32_t r,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gate and up projections of a layer with silu(g) * u in the epilogue (the
 * layer structure as for uno_gated_gemm_residual).  The weights come
 * interleaved by uno_swiglu_pack: w_packed [2 N_half, K] holds 128-row blocks
 * of W_gate and W_up in turn, b_packed [2 N_half, rt] the block-diagonal
 * LoRA B (gate rows use T columns [0, rt/2), up rows [rt/2, rt)); t is
 * uno_lora_down over the stacked [A_gate; A_up] (width rt = 2 r).  Output
 * act [M, N_half] = bf16(silu(g) * u) with g, u the bf16 gate and up
 * projections, bitwise the result of uno_gated_gemm_grouped for gate and up
 * under the same plan followed by uno_silu_mul.  (At 32 rows or fewer this
 * launch takes a tile of its own -- 32 rows by half a gate block and half
 * its up block, one K group -- whose fp32 sums run in another order than
 * the grouped launch's two-K-group tiles: there the two agree to rounding.)
 * Domain: N_half a positive multiple of 128, rt a multiple of 8 in [8, 256],
 * otherwise as uno_gated_gemm; act must not alias the inputs. */
size_t uno_gated_gemm_swiglu_workspace_size(int64_t M, int64_t N_half, int64_t K, int32_t rt);
uno_status uno_gated_gemm_swiglu(const void* x, const void* w_packed, const void* t, const void* b_packed,
                                 const void* row_plan, void* act, int64_t M, int64_t N_half, int64_t K, int32_t rt,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Packing for uno_gated_gemm_swiglu: w_gate, w_up [N_half, K] and b_gate,
 * b_up [N_half, r] (bf16) into w_packed [2 N_half, K] and b_packed
 * [2 N_half, 2 r] as described there.  Domain: N_half a positive multiple of
 * 128; K, r multiples of 8, r <= 512; outputs must not alias inputs. */
uno_status uno_swiglu_pack(const void* w_gate, const void* w_up, const void* b_gate, const void* b_up,
                           int64_t N_half, int64_t K, int32_t r, void* w_packed, void* b_packed,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Block verification ("The Psi-Spec Sampler" on the aifromscratch.in page:
 * rejection-sample the drafted block against the AR model and keep the
 * longest valid prefix, with the AR distribution preserved; "What 'lossless'
 * means here" on the cctest.ai page: the AR model rejects or adjusts
 * candidates).  For each of B sequences with L drafted tokens x_i:
 *
 *   p_i = softmax(z_i / T),  q_i = softmax(d_i / T)
 *   accept_i  <=>  u[s, i] < min(1, p_i(x_i) / q_i(x_i))
 *   n_acc     =  index of the first rejected position (L if none)
 *   if n_acc < L : y ~ normalize(max(0, p_j - q_j)), j = n_acc
 *                  (from p_j if that residual has zero mass)
 *   elif has_bonus: y ~ p_L (target row L)
 *   draws use the inverse CDF with u[s, L]: the smallest k with C_k > u R.
 *   out_tokens[s] = x_0 .. x_{n_acc-1}, y, then -1 padding
 *   n_emitted[s]  = n_acc + 1 if a token was drawn, else L
 *
 * target_logits : device, dtype; row (s, i), i < L + has_bonus, starts at
 *                 s * target_seq_stride + i * V elements
 * draft_logits  : device, dtype; row (s, i), i < L, at s * draft_seq_stride + i * V
 *                 (a stride of 0 broadcasts one block to every sequence)
 * draft_tokens  : device int32 [B, L]
 * uniforms      : device float [B, L + 1]; slots 0..L-1 accept, slot L draw
 * n_accepted    : device int32 [B]; -1 if some draft token lies outside [0, V)
 *                 (then n_emitted = 0 and out_tokens are all -1)
 * out_tokens    : device int32 [B, L + 1]
 * n_emitted     : device int32 [B]
 * Arithmetic: row maxima and sums of exp stream in fp32 per element with
 * fp64 accumulation; the acceptance ratio is formed in fp64 in log space;
 * the redraw CDF sums fp32 weights of 16-token segments and carries across
 * segments in fp64.  Vocabularies of at most 1024 tokens are verified by one
 * wavefront per sequence (the workspace is then not touched), larger ones by
 * a statistics pass over every row followed by the decision and the draw.
 *
 * Domain: B >= 0 (B = 0 is a no-op), 1 <= L <= 64 (L <= 63 with has_bonus),
 * V >= 1, T > 0 and finite, logits UNO_BF16 or UNO_F32, each row holding at
 * least one finite logit (NaN and +inf are outside the contract; -inf masks
 * a token).  Stride 0 is allowed for either logit array.
 * workspace: at least uno_block_verify_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
size_t uno_block_verify_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus);
uno_status uno_block_verify(const void* target_logits, const void* draft_logits,
                            int64_t target_seq_stride, int64_t draft_seq_stride,
                            const int32_t* draft_tokens, const float* uniforms,
                            int64_t B, int32_t L, int64_t V, int32_t has_bonus,
                            float temperature, int32_t logits_dtype,
                            int32_t* n_accepted, int32_t* out_tokens, int32_t* n_emitted,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Block verification without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments, arithmetic, domain and outputs are those
 * of uno_block_verify (the same kernels: the outputs are bitwise equal); the
 * scratch space is the library's own device array of
 * uno_block_verify_noalloc_max_bytes() bytes (32 MiB), one per GPU, held
 * until the process ends.  A problem whose uno_block_verify_workspace_size()
 * exceeds it returns UNO_ERR_UNSUPPORTED before anything is enqueued
 * (B = 256, L = 32, V = 128256 needs 16 MiB).  Every call on one GPU shares
 * that GPU's array, so calls that overlap in time on one GPU (two streams,
 * two host threads) race and must be ordered by the caller.  The first call
 * on a device looks the array's device address up (no allocation); nothing
 * in the array needs to start at zero.
 * ------------------------------------------------------------------------ */
size_t uno_block_verify_noalloc_max_bytes(void);
uno_status uno_block_verify_noalloc(const void* target_logits, const void* draft_logits,
                                    int64_t target_seq_stride, int64_t draft_seq_stride,
                                    const int32_t* draft_tokens, const float* uniforms,
                                    int64_t B, int32_t L, int64_t V, int32_t has_bonus,
                                    float temperature, int32_t logits_dtype,
                                    int32_t* n_accepted, int32_t* out_tokens, int32_t* n_emitted,
                                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Block verification with early exit.  Only the prefix up to the first
 * rejection decides the output ("The Psi-Spec Sampler" on the
 * aifromscratch.in page: the longest valid prefix is kept), so positions are
 * taken in chunks of chunk, 2 chunk, 4 chunk, ... positions: the logit rows of
 * a chunk are streamed only for sequences with no rejection in earlier
 * chunks, and a sequence stops at the chunk holding its first rejection (the
 * bonus row, if any, streams with the last chunk).  Rows read per sequence
 * fall from L (+1) to the end of that chunk.
 *
 * Arguments, arithmetic, domain and outputs are those of uno_block_verify,
 * plus chunk in [1, 64]; every output equals uno_block_verify's bit for bit
 * (a row's statistics are formed with the same chunking of V, and every
 * position is decided by the same code).  Launches one statistics kernel per
 * chunk -- each opens with the decision on the positions before its chunk,
 * and a sequence already rejected streams nothing -- then the one-pass
 * verifier's tail, so it pays where rejections come early and rows are long.
 * workspace: at least uno_block_verify_early_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
size_t uno_block_verify_early_workspace_size(int64_t B, int32_t L, int64_t V, int32_t has_bonus);
uno_status uno_block_verify_early(const void* target_logits, const void* draft_logits,
                                  int64_t target_seq_stride, int64_t draft_seq_stride,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  int64_t B, int32_t L, int64_t V, int32_t has_bonus,
                                  float temperature, int32_t logits_dtype, int32_t chunk,
                                  int32_t* n_accepted, int32_t* out_tokens, int32_t* n_emitted,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Draft proposal: one token per drafted position, drawn in parallel from the
 * diffusion pathway's distribution q_i = softmax(d_i / T) by inverse CDF
 * ("The Psi-Spec Sampler" on the aifromscratch.in page: the diffusion
 * pathway proposes a block in parallel; the linear sampler takes one
 * candidate per position).
 *
 *   tokens[s, i] = smallest k with C_k > u[s, i] * R over the weights q_i
 *
 * draft_logits : device, dtype; row (s, i) at s * seq_stride + i * V elements
 * uniforms     : device float [B, L]
 * tokens       : device int32 [B, L]
 * Same arithmetic and domain as uno_block_verify (no upper limit on L).
 * workspace: at least uno_draft_sample_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
size_t uno_draft_sample_workspace_size(int64_t B, int32_t L, int64_t V);
uno_status uno_draft_sample(const void* draft_logits, int64_t seq_stride,
                            const float* uniforms, int64_t B, int32_t L, int64_t V,
                            float temperature, int32_t logits_dtype, int32_t* tokens,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Tree verification ("The Psi-Spec Sampler" on the aifromscratch.in page:
 * the tree sampler takes several candidates per position -- the top K --
 * and verifies them in a prefix tree, keeping the AR model's law).  The
 * pages give no rule; with fixed candidates, rejection over a node's
 * children is in law one draw from the node's AR distribution followed by a
 * look-up among the children, which is what runs:
 *
 *   v = root; depth = 0
 *   loop: y = smallest k with C_k > u[s, depth] R over p_v = softmax(z_v / T)
 *         out_tokens[s, depth] = y
 *         if a child c of v has token y (the lowest-numbered if several):
 *             v = c, depth += 1
 *         else stop
 *   n_accepted[s] = depth (tree tokens kept), n_emitted[s] = depth + 1,
 *   last_node[s] = v; out_tokens padded with -1.
 *
 * node_logits : device, dtype; the AR logits after node n's prefix (node 0:
 *               after the committed context) at s * seq_stride + n * V
 * parents     : device int32 [B, N]; parents[s, 0] = -1 and
 *               0 <= parents[s, n] < n for n >= 1
 * tokens      : device int32 [B, N]; the token of node n (node 0's unused),
 *               in [0, V)
 * uniforms    : device float [B, N]; slot d is the draw at depth d
 * out_tokens  : device int32 [B, N]; n_accepted, n_emitted, last_node [B]
 * A tree breaking the parent or token rule gives n_accepted = -1,
 * n_emitted = 0, last_node = -1 and out_tokens all -1.  Arithmetic: that of
 * uno_draft_sample (fp32 exponentials, fp64 sums, the same inverse CDF).
 * Large problems run one workgroup per tree that reads only the walked
 * rows, each once (a 16-token segment's mass is formed from the segment's
 * own maximum, then scaled to the row's); small ones draw every node's
 * token with its depth's uniform across the GPU and then walk (the two
 * differ only where a uniform falls within rounding of a CDF boundary).
 *
 * Domain: B >= 0 (B = 0 is a no-op), 1 <= N <= 4096, V >= 1, T > 0 and
 * finite, logits UNO_BF16 or UNO_F32 with a finite value in every row.
 * workspace: at least uno_tree_verify_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
size_t uno_tree_verify_workspace_size(int64_t B, int32_t N, int64_t V);
uno_status uno_tree_verify(const void* node_logits, int64_t seq_stride, const int32_t* parents,
                           const int32_t* tokens, const float* uniforms, int64_t B, int32_t N, int64_t V,
                           float temperature, int32_t logits_dtype, int32_t* n_accepted, int32_t* out_tokens,
                           int32_t* n_emitted, int32_t* last_node, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * The LM head fused with the statistics of block verification.  The
 * verifier ("The Psi-Spec Sampler" on the aifromscratch.in page) needs, per
 * position, the softmax normalisers of the target and draft rows and their
 * logits at the drafted token; only the redraw needs whole rows, and only
 * one pair per sequence.  Here the LM-head GEMM (bf16 MFMA, fp32
 * accumulation) forms those statistics in its epilogue, tile by tile, so the
 * logits need never reach memory:
 *
 *   z = bf16(hidden_target W^T),  d = bf16(hidden_draft W^T)
 *   then exactly what uno_block_verify computes on (z, d).
 *
 * hidden       : device bf16 [B (L + has_bonus) + B L, K], row-major: target
 *                row (s, i) at row s (L + has_bonus) + i, then draft row (s, i)
 *                at row B (L + has_bonus) + s L + i
 * w_lm         : device bf16 [V, K] (the head's weight, nn.Linear layout)
 * draft_tokens, uniforms, n_accepted, out_tokens, n_emitted, temperature,
 * has_bonus    : as in uno_block_verify
 * logits       : device bf16 [B (L + has_bonus) + B L, V] receiving z then d
 *                (the same row order as hidden), or NULL.  With NULL no logit
 *                row is written; the target and draft rows of each
 *                sequence's redraw are recomputed after the decision (one
 *                more pass over W for 2 B rows, the same bits).  Storing pays
 *                while 2 rows V bytes of logits cost less than reading W once.
 * Statistics are formed per 256-column tile of the head with the arithmetic
 * of uno_block_verify (fp32 exponentials of max-subtracted logits, fp64
 * sums) and merged per row in fp64 in a fixed order.  The sums run in
 * another order than uno_block_verify's, so the two agree except where a
 * uniform falls within rounding (about 1e-7 relative) of an acceptance
 * probability or a CDF boundary.  Both modes (logits stored or not) give
 * the same bits.
 *
 * Domain: B >= 0 (B = 0 is a no-op), 1 <= L <= 64 (L <= 63 with has_bonus),
 * V >= 1, K % 8 == 0, V K < 2^30, rows K < 2^30, T > 0 and finite; hidden,
 * w_lm, logits 16-byte aligned.  Every logit row must hold a finite value.
 * workspace: at least uno_lm_head_verify_workspace_size() bytes (about
 * 24 (B (L+1)) ceil(V / 256) + 4 B V bytes).
 * ------------------------------------------------------------------------ */
size_t uno_lm_head_verify_workspace_size(int64_t B, int32_t L, int64_t V, int64_t K, int32_t has_bonus);
uno_status uno_lm_head_verify(const void* hidden, const void* w_lm, int64_t B, int32_t L, int64_t V, int64_t K,
                              int32_t has_bonus, float temperature, const int32_t* draft_tokens,
                              const float* uniforms, int32_t* n_accepted, int32_t* out_tokens,
                              int32_t* n_emitted, void* logits, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Glue between projections of a layer with the attention mixing left out
 * (the pages add the LoRA pathway to each transformer layer -- "How It Works:
 * The 'Uno' Architecture" on the aifromscratch.in page -- but describe no
 * other part of the layer).  bf16 in and out, fp32 arithmetic.
 *
 * uno_rmsnorm      : y[m, :] = x[m, :] / sqrt(mean_k x[m, k]^2 + eps), x, y [M, K]
 * uno_silu_mul     : out = silu(gate) * up elementwise, silu(t) = t / (1 + e^-t)
 * uno_residual_add : out = a + b elementwise (out may alias a or b)
 * uno_residual_rmsnorm : s = x + y (rounded to bf16) into s_out, then h = rmsnorm(s);
 *                    x, y, s_out, h [M, K]; s_out may alias x (the residual stream
 *                    updated in place), h must not alias any of them.  Both outputs
 *                    are bitwise those of uno_residual_add followed by uno_rmsnorm.
 * Domain: sizes >= 0; K % 8 == 0 and K <= 65536 for the two norms; eps >= 0; only UNO_BF16;
 * every pointer 16-byte aligned.
 * ------------------------------------------------------------------------ */
uno_status uno_rmsnorm(const void* x, void* y, int64_t M, int64_t K, float eps, int32_t dtype,
                       hipStream_t stream);
uno_status uno_silu_mul(const void* gate, const void* up, void* out, int64_t n, int32_t dtype,
                        hipStream_t stream);
uno_status uno_residual_add(const void* a, const void* b, void* out, int64_t n, int32_t dtype,
                            hipStream_t stream);
uno_status uno_residual_rmsnorm(const void* x, const void* y, void* s_out, void* h, int64_t M, int64_t K,
                                float eps, int32_t dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* UNO_H_ */
