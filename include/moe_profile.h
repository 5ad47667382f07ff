/*
 * moe_profile.h -- instrumented variant of moe_forward for benchmarks.
 *
 * Computes exactly what moe_forward (include/moe.h) computes, with the same arguments and rules, and in
 * addition records seven caller-created HIP events (hipEvent_t, created with timing enabled) on `stream`
 * at the stage boundaries:
 *   events[0] start of the layer              events[4] after the routed gate/up (SwiGLU) grouped GEMM
 *   events[1] after the router                events[5] after the routed down grouped GEMM
 *   events[2] after the permutation           events[6] after the combine (the end of the layer)
 *   events[3] after the shared expert (when it runs on `stream`)
 * hipEventElapsedTime between consecutive events gives each stage's device time. A null entry records
 * nothing at its boundary (each recorded event costs the stream a few microseconds, which a decode-sized
 * pass notices; a benchmark that wants one stage's time passes only the two events around it). The events
 * stay owned by the caller. With stream_shared non-null the shared expert runs on that stream, forked after the
 * permutation: events[2] to events[3] is then empty and its time overlaps the routed GEMMs.
 * Pages: as moe_forward (open-model-atlas GLM-5 "MoE transformer block", "All 43 steps").
 */
#ifndef SIGMOID_ROUTED_MIXTURE_MOE_PROFILE_H
#define SIGMOID_ROUTED_MIXTURE_MOE_PROFILE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

moe_status moe_forward_profiled(const moe_bf16* x, const moe_bf16* w_router, const float* bias,
                                const moe_bf16* w1, const moe_bf16* w3, const moe_bf16* w2, const moe_bf16* ws1,
                                const moe_bf16* ws3, const moe_bf16* ws2, int T, int H, int E, int k, int I, int Is,
                                float scale, float* out, int32_t* topk_ids, float* topk_gates,
                                int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream,
                                void* stream_shared, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* SIGMOID_ROUTED_MIXTURE_MOE_PROFILE_H */
