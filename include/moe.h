/*
 * moe.h -- C ABI of the MI355X (gfx950) sigmoid-routed mixture-of-experts layer.
 *
 * The layer is the feed-forward half of a GLM-5 / GLM-4.7-Flash mixture block. Per token x (one row of
 * x[T, H]):
 *
 *   z = x W_r                       router logits, one per routed expert
 *   s = sigmoid(z)                  scores
 *   sel = top_k(s + b)              the bias b is added only to choose the experts
 *   G_i = scale s_i / sum_{j in sel} s_j      gates of the chosen experts (they sum to scale)
 *   E_i(x) = (silu(x W1_i) * (x W3_i)) W2_i  SwiGLU routed expert
 *   out = sum_{i in sel} G_i E_i(x) + (silu(x Ws1) * (x Ws3)) Ws2    routed sum plus the shared expert
 *
 * Sources: open-model-atlas, GLM-5 "MoE transformer block", section "All 43 steps", the mixture-of-experts
 * equations (router, sigmoid, top-8 of s + b, gates scaled by 2.5, the SwiGLU expert, the routed sum over
 * experts, the shared expert, the layer output); nnterp encyclopedia glm_moe_dsa and glm4_moe_lite,
 * "The mixture: sigmoid scores, a selection bias, renormalized weights" (router_logits are taken before
 * the sigmoid and before the bias; the bias only chooses; gates are the chosen sigmoids renormalised to
 * one and multiplied by routed_scaling_factor; mlp_output = routed_output + shared_expert_output).
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns (moe_bf16); every tensor is row-major and dense.
 *  - Weights are stored [out_features, in_features] like nn.Linear: W_r [E, H]; W1 (gate) and W3 (up)
 *    [E, I, H]; W2 (down) [E, H, I]; shared Ws1, Ws3 [Is, H] and Ws2 [H, Is].
 *  - Every tensor pointer is a DEVICE pointer, 16-byte aligned; the workspace is 256-byte aligned.
 *  - `stream` is a hipStream_t (NULL: the default stream). All work is enqueued on it and the call
 *    returns without synchronising; results are ready when the stream's work completes.
 *  - The caller owns every buffer and stream. The library never allocates or frees device memory and
 *    never copies to the host. Its only state, made on first use per device, is one pair of HIP events
 *    (for stream_shared) and the device's compute-unit count (it sizes the persistent GEMM grids).
 *  - Arguments are checked before anything is enqueued: a call that returns an error has no effect.
 *    T == 0 returns MOE_OK once the sizes pass their checks, without looking at any pointer, and
 *    enqueues nothing. Non-finite inputs are outside the contract.
 *  - Supported sizes: 1 <= k <= min(E, 32), E <= 256, H, I and Is multiples of 64, T * k < 2^31.
 *  - Calls on one stream run in order; overlapping calls that share output or workspace buffers race.
 *  - Kernels, the spread of GEMM blocks over the chip and any K split are picked from the sizes alone; the
 *    library reads no environment variable. Tests and benchmarks may override those choices through the
 *    process-wide knobs of moe_tuning.h. Every choice computes the same layer; only a K split or a
 *    different kernel changes the fp32 summation order.
 */
#ifndef SIGMOID_ROUTED_MIXTURE_MOE_H
#define SIGMOID_ROUTED_MIXTURE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null required pointer, T < 0, H/E/I <= 0, k < 1, k > E, Is < 0 */
    MOE_ERR_UNSUPPORTED = 2, /* E > 256, k > 32, H/I/Is not a multiple of 64, T * k >= 2^31 */
    MOE_ERR_MISALIGNED = 3,  /* a tensor not 16-byte aligned, or the workspace not 256-byte aligned */
    MOE_ERR_WORKSPACE = 4,   /* workspace_bytes smaller than this call's sizes need (never more than the
                                matching *_workspace_bytes query returns) */
    MOE_ERR_HIP = 5          /* a HIP launch or event call failed; moe_last_error() has the text */
} moe_status;

/*
 * Bytes of workspace moe_forward needs for up to T tokens at these sizes: an upper bound that does not
 * depend on the routing and covers every token count from 0 to T (the layout is not monotone in T, so the
 * query returns the largest one), so one workspace sized for the largest batch serves every smaller one.
 * Pure host arithmetic: no device access. Returns 0 when the sizes are invalid or unsupported.
 */
size_t moe_workspace_bytes(int T, int H, int E, int k, int I, int Is);

/*
 * Router: logits, sigmoid scores, biased top-k and gates for T tokens.
 *   x          [T, H] bf16      tokens (the normalised stream entering the mixture)
 *   w_router   [E, H] bf16      router weight
 *   bias       [E] fp32         selection bias (chooses only; gates use the unbiased scores)
 *   scale                       routed scaling factor (2.5 on GLM-5, 1.8 on GLM-4.7-Flash)
 *   topk_ids   [T, k] int32     out: chosen experts, slot order = descending s + b, ties to the lower index
 *   topk_gates [T, k] fp32      out: G = scale * s / (sum of the chosen s), same slot order
 *   logits     [T, E] fp32      out, nullable: z = x W_r (fp32-accumulated), before sigmoid and bias
 * Logits accumulate in fp32 (exact bf16 products); s = 1 / (1 + exp(-z)) in fp32; s + b in fp32.
 * Here each logit is one fp32 sum over h; inside moe_forward the same logits are summed over K ranges in
 * another fp32 order, so the two may differ in the last bits of z. A token whose k-th and (k+1)-th values
 * of s + b lie that close may then choose differently here than inside moe_forward (so moe_route followed
 * by moe_forward_routed is not bit-identical to moe_forward for such tokens).
 * Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (z = x W_r, s = sigma(z),
 * top-8 of s + b, G_i); nnterp glm_moe_dsa "The mixture" (router_logits, expert_weights, expert_indices).
 */
moe_status moe_route(const moe_bf16* x, const moe_bf16* w_router, const float* bias, int T, int H, int E, int k,
                     float scale, int32_t* topk_ids, float* topk_gates, float* logits, void* stream);

/*
 * Permutation of the T * k routing slots into expert-contiguous rows (a stable counting sort by expert).
 *   x          [T, H] bf16       tokens (read only when x_perm is non-null; may then be null otherwise)
 *   topk_ids   [T, k] int32      experts chosen per token, each in [0, E) and distinct within a token
 *   counts     [E] int32         out: rows given to each expert, one per token whose ids name it
 *   offsets    [E + 1] int32     out: exclusive prefix sum of counts; offsets[E] = T * k when every id is
 *                                in [0, E) and distinct within its token (as moe_route writes them),
 *                                else the number of rows actually given out
 *   row_token  [T * k] int32     out: token of each expert-contiguous row; the rows of expert e are
 *                                offsets[e] .. offsets[e+1]-1, in ascending token order
 *   slot_row   [T * k] int32     out: row that slot j of token t went to, at index t * k + j
 *   x_perm     [T * k, H] bf16   out, nullable: x_perm[r] = x[row_token[r]]
 *   workspace                    device scratch of at least moe_permute_workspace_bytes(T, E) bytes
 * Ids outside [0, E) are skipped (their slots get no row and slot_row -1); repeated ids within one token
 * share a row (the token counts once for that expert).
 * Neither is produced by moe_route. The pages pass (hidden, indices, weights) to the routed experts
 * (nnterp glm_moe_dsa, expert_indices = "experts's inputs, element 1"); this grouping is how the experts
 * here receive their tokens.
 */
size_t moe_permute_workspace_bytes(int T, int E);
moe_status moe_permute(const moe_bf16* x, const int32_t* topk_ids, int T, int H, int E, int k, int32_t* counts,
                       int32_t* offsets, int32_t* row_token, int32_t* slot_row, moe_bf16* x_perm, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * The whole layer: route, permute, SwiGLU routed experts (grouped GEMMs), the shared expert, and the
 * gate-weighted combine.
 *   x, w_router, bias            as for moe_route
 *   w1, w3  [E, I, H] bf16       routed gate (silu) and up projections
 *   w2      [E, H, I] bf16       routed down projection
 *   ws1, ws3 [Is, H], ws2 [H, Is] bf16   shared expert; all three may be null when Is == 0
 *   out     [T, H] fp32          out: sum_j G[t,j] E_{ids[t,j]}(x_t) + shared(x_t)
 *   topk_ids [T, k] int32, topk_gates [T, k] fp32, expert_counts [E] int32   out, nullable
 *   workspace / workspace_bytes  device scratch of at least moe_workspace_bytes(T, H, E, k, I, Is) bytes
 *   stream                       the stream everything is ordered on
 *   stream_shared                nullable: a second stream for the shared expert, which then overlaps the
 *                                routed experts; it waits for work already on `stream` and `stream` waits
 *                                for it before the combine. NULL runs the shared expert on `stream`.
 * Expert GEMMs take bf16 operands with fp32 accumulation; the SwiGLU activation h is stored as bf16
 * between the two GEMMs (it is the down GEMM's bf16 MFMA operand); per-slot expert outputs are stored as
 * bf16 when k >= 8 (their roundings then partly cancel in the gated sum) unless the shared expert runs as
 * one more group of the routed GEMMs (when 0 < Is == I and T * k <= 16 * E), else as fp32; the combine sums
 * the k gated slots in slot order plus the shared expert in fp32.
 * Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (g = x W1, u = x W3,
 * a = g sigma(g), h = a * u, E_i = h W2, y_routed = sum G_i E_i, the shared expert, delta_ffn =
 * y_routed + y_shared); nnterp glm_moe_dsa "The mixture" (routed + shared == mlp_output).
 */
moe_status moe_forward(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                       const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                       const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale, float* out,
                       int32_t* topk_ids, float* topk_gates, int32_t* expert_counts, void* workspace,
                       size_t workspace_bytes, void* stream, void* stream_shared);

/*
 * moe_forward without a caller workspace, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same arguments, computation and
 * results as moe_forward (bit for bit), minus workspace, workspace_bytes and stream_shared (the shared expert
 * runs on `stream`). The workspace is a file-scope device array of moe_forward_noalloc_max_bytes() bytes
 * (64 MiB) inside the library, one per device, held until the process ends; the call allocates nothing.
 *   Sizes whose workspace (the layout moe_forward uses for exactly these sizes) exceeds that maximum return
 *   MOE_ERR_WORKSPACE with the byte counts in moe_last_error(), and enqueue nothing. GLM-5 shapes fit up to
 *   T = 64 tokens, GLM-4.7-Flash shapes up to T = 512.
 *   Every call on a device uses that device's one array and leaves its contents there; each call writes
 *   everything it reads (its block counters included) before reading it, so nothing carries over. Calls
 *   that overlap on one device (two streams, two host threads) race on the array: order them on one
 *   stream. Calls on different devices do not share it.
 *   The first call on each device looks up that device's array (hipGetSymbolAddress), a query that
 *   allocates nothing; capture a graph only after one call on the device has returned.
 */
size_t moe_forward_noalloc_max_bytes(void);
moe_status moe_forward_noalloc(const moe_bf16* x, const moe_bf16* w_router, const float* bias, const moe_bf16* w1,
                               const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1, const moe_bf16* ws3,
                               const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is, float scale,
                               float* out, int32_t* topk_ids, float* topk_gates, int32_t* expert_counts,
                               void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Text of the last error on the calling thread (argument check or HIP message); "" if none. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SIGMOID_ROUTED_MIXTURE_MOE_H */
