// Top-k routing of one token by one wave, shared by the router kernels and the decode route-and-permute
// kernel: s = sigmoid(z), c = s + b, the k largest c (ties to the lower expert index), gates
// G = scale * s / sum of the chosen s.
// Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (s = sigma(z),
// E_sel = [i in top_8(s + b)], G_i = 2.5 s_i E_sel_i / sum_j s_j E_sel_j); nnterp encyclopedia glm_moe_dsa,
// "The mixture" (the bias only chooses; the gates are renormalised and scaled).
#pragma once

#include "common.h"

namespace moe {

// Orderable key of a biased score: larger c first, then the lower expert index. 0 = no candidate.
__device__ __forceinline__ uint64_t score_key(float c, int e) {
    uint32_t u = __float_as_uint(c);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One wave routes one token. z4[q] is the logit of expert lane + 64 q (ignored when that is >= E).
__device__ __forceinline__ void topk_token(const float (&z4)[4], int t, int E, int k, float scale,
                                           const float* __restrict__ bias, int32_t* __restrict__ ids,
                                           float* __restrict__ gates, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    float s4[4];
    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (e < E) {
            const float s = 1.0f / (1.0f + expf(-z4[q]));
            s4[q] = s;
            key[q] = score_key(s + bias[e], e);
            if (logits) logits[(size_t)t * E + e] = z4[q];
        } else {
            s4[q] = 0.f;
            key[q] = 0;
        }
    }
    int my_id = 0;
    float my_s = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) best = key[q] > best ? key[q] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFu - (uint32_t)(best & 0xFFFFu));
        const int owner = e & 63;
        const int qw = e >> 6;
        float sq = s4[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) sq = qw == q ? s4[q] : sq;
        const float s_w = __shfl(sq, owner, 64);
        if (lane == owner) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q == qw) key[q] = 0;
        }
        if (lane == j) {
            my_id = e;
            my_s = s_w;
        }
    }
    const float den = wave_sum(lane < k ? my_s : 0.f);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        gates[(size_t)t * k + lane] = den > 0.f ? scale * my_s / den : 0.f;
    }
}

} // namespace moe
