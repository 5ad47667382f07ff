/*
 * moe_block.h -- entry points around the mixture of include/moe.h: the mixture with the routing given by
 * the caller, the mixture half of a whole block (RMSNorm before it, the residual add after it), and the
 * dense SwiGLU MLP of the dense-first blocks. The conventions of moe.h hold here too: device pointers,
 * 16-byte aligned tensors, a 256-byte aligned workspace, bf16 as uint16_t bits, weights [out, in], every
 * argument checked before anything is enqueued, T == 0 a no-op once the sizes pass, work enqueued on
 * `stream` without synchronising, no allocation, no host copies.
 */
#ifndef SIGMOID_ROUTED_MIXTURE_MOE_BLOCK_H
#define SIGMOID_ROUTED_MIXTURE_MOE_BLOCK_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The mixture with the routing given instead of computed: slot j of token t goes to expert
 * topk_ids[t, j] with weight topk_gates[t, j], used exactly as given (no renormalisation), plus the
 * shared expert: out[t] = sum_j topk_gates[t, j] E_{topk_ids[t, j]}(x_t) + shared(x_t).
 * This is the pages' ablation and gate editing: zeroing the weight of every slot that chose an expert
 * removes that expert while the other slots keep their weights, so a token's weights then sum to less
 * than the routed scale (nnterp encyclopedia glm_moe_dsa and glm4_moe_lite, "The mixture", the ablation
 * example on expert_weights and expert_indices).
 *   x                   [T, H] bf16      tokens
 *   topk_ids            [T, k] int32     experts, each in [0, E); a slot whose id is outside [0, E)
 *                                        contributes nothing; a token may name one expert in several slots
 *                                        (each slot then adds its own gate times that expert's output)
 *   topk_gates          [T, k] fp32      slot weights, any finite values
 *   w1, w3, w2, ws1, ws3, ws2            as for moe_forward (shared ones null when Is == 0)
 *   out                 [T, H] fp32      out
 *   expert_counts       [E] int32        out, nullable: tokens routed to each expert (a token counts once
 *                                        per expert however many of its slots name it)
 *   workspace           at least moe_workspace_bytes(T, H, E, k, I, Is) bytes
 *   stream, stream_shared                as for moe_forward
 * Numerics as moe_forward: bf16 operands, fp32 accumulation, bf16 h between the GEMMs, per-slot rows bf16
 * or fp32 by the same rule, and fp32 combine in slot order.
 */
moe_status moe_forward_routed(const moe_bf16* x, const int32_t* topk_ids, const float* topk_gates,
                              const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1,
                              const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is,
                              float* out, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                              void* stream, void* stream_shared);

/*
 * Workspace bytes of moe_block_forward (moe_workspace_bytes plus a [T, H] bf16 region for the normalised
 * stream), for up to T tokens like moe_workspace_bytes. 0 when the sizes are invalid or unsupported.
 */
size_t moe_block_workspace_bytes(int T, int H, int E, int k, int I, int Is);

/*
 * The mixture half of a GLM-5 / GLM-4.7-Flash block on the residual stream x' (the stream after the
 * attention add): x_ffn = RMSNorm(x') = gamma * x' / sqrt(mean_h x'^2 + eps), the mixture of moe_forward
 * on x_ffn, and the residual add out = x' + routed + shared.
 * Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (x'_n = x_n + delta_attn,
 * x_ffn = RMSNorm(x'_n), the mixture on x_ffn, x_{n+1} = x'_n + delta_ffn); nnterp encyclopedia
 * glm_moe_dsa / glm4_moe_lite module trees (post_attention_layernorm, an RMSNorm of the hidden size with
 * eps 1e-5, is the MLP's input norm; the block adds the MLP's output to the residual).
 *   resid        [T, H] bf16    x', the residual stream entering the MLP half
 *   gamma        [H] bf16       RMSNorm weight
 *   eps                         RMSNorm epsilon (>= 0; 1e-5 on both models)
 *   w_router, bias, w1, w3, w2, ws1, ws3, ws2, k, scale          as for moe_forward
 *   out          [T, H] fp32    out: x_{n+1} = x' + routed + shared (the residual added last, in fp32)
 *   x_norm       [T, H] bf16    out, nullable: x_ffn, what the router and the experts read
 *   topk_ids, topk_gates, expert_counts                          out, nullable, as for moe_forward
 *   workspace    at least moe_block_workspace_bytes(T, H, E, k, I, Is) bytes
 * x_ffn is computed in fp64 ((x' * rstd) * gamma, rstd = 1 / sqrt(sum x'^2 / H + eps)) and rounded once
 * to bf16 (nearest, ties to even). Returns MOE_ERR_INVALID_ARG when eps is negative or not finite.
 */
moe_status moe_block_forward(const moe_bf16* resid, const moe_bf16* gamma, double eps, const moe_bf16* w_router,
                             const float* bias, const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2,
                             const moe_bf16* ws1, const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E,
                             int k, int I, int Is, float scale, float* out, moe_bf16* x_norm, int32_t* topk_ids,
                             float* topk_gates, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                             void* stream, void* stream_shared);

/* Workspace bytes of moe_dense_mlp for up to T tokens: h [T, I] bf16 and, at few tokens, the fp32 partials
 * of the split-K GEMMs. 0 when the sizes are invalid or unsupported. */
size_t moe_dense_mlp_workspace_bytes(int T, int H, int I);

/*
 * Dense SwiGLU MLP of the dense-first blocks: out = (silu(x W1) * (x W3)) W2, with the same kernels and
 * numerics as the shared expert (bf16 operands, fp32 accumulation, h stored as bf16, fp32 out).
 * Pages: nnterp encyclopedia glm_moe_dsa module tree (blocks 0 to 2: GlmMoeDsaMLP, gate_proj and up_proj
 * 6144 -> 12288, down_proj 12288 -> 6144, SiLU) and glm4_moe_lite (block 0: Glm4MoeLiteMLP, 2048 -> 10240);
 * mlp_neurons is act(gate) * up, what the down projection receives.
 *   x        [T, H] bf16        tokens (the normalised stream)
 *   w1, w3   [I, H] bf16        gate (silu) and up projections
 *   w2       [H, I] bf16        down projection
 *   out      [T, H] fp32        out
 *   workspace                   at least moe_dense_mlp_workspace_bytes(T, H, I) bytes
 * Supported sizes: H and I multiples of 64, T < 2^27.
 */
moe_status moe_dense_mlp(const moe_bf16* x, const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, int T,
                         int H, int I, float* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SIGMOID_ROUTED_MIXTURE_MOE_BLOCK_H */
