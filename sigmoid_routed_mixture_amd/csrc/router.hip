// Router of the sigmoid-routed MoE layer on gfx950: logits z = x W_r (bf16 MFMA, fp32 accumulation),
// s = sigmoid(z), c = s + b, top-k of c per token (ties to the lower expert index) and the gates
// G = scale * s / sum of the chosen s.
// Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (z = x W_r, s = sigma(z),
// E_sel = [i in top_8(s + b)], G_i = 2.5 s_i E_sel_i / sum_j s_j E_sel_j); nnterp encyclopedia glm_moe_dsa,
// "The mixture" (the bias is added to the sigmoids only to choose; gates renormalised, times the scale).
#include "common.h"
#include "kernels.h"
#include "plan.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kBT = kRouterBT; // tokens per workgroup: two 16-token MFMA column blocks
static_assert(kBT == 32, "router tiling assumes 32 tokens per workgroup");

// Accumulates z for tokens [t0, t0 + 32) and experts [64 w, 64 w + 64) of wave w over the 64-wide
// K chunks [c0, c1). acc[b][j]: expert block b (16 experts), token block j (16 tokens); lane l holds
// experts 16 b + 4 (l / 16) + r and token 16 j + l % 16 in element r.
// Each lane reads 32 contiguous bytes per row per chunk (k-group l / 16 covers k 16 g .. 16 g + 15) and
// feeds the first 8 values to one MFMA and the next 8 to a second; x and W_r use the same k mapping, so
// the pair of MFMAs sums all 64 products of the chunk.
__device__ __forceinline__ void router_accumulate(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                  int T, int H, int E, int t0, int c0, int c1, f32x4 (&acc)[4][2]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rl = lane & 15;
    const int kg = lane >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int e_base = wave * 64;
    if (e_base >= E) return;
    int nb = (E - e_base + 15) / 16;
    nb = nb > 4 ? 4 : nb;
    const uint16_t* wrow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int e = e_base + b * 16 + rl;
        e = e < E ? e : E - 1;
        wrow[b] = wr + (size_t)e * H + kg * 16;
    }
    const uint16_t* xrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int t = t0 + j * 16 + rl;
        t = t < T ? t : T - 1;
        xrow[j] = x + (size_t)t * H + kg * 16;
    }
    for (int c = c0; c < c1; ++c) {
        const int k = c * 64;
        Pack16 xa[2], xb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            xa[j] = load16(xrow[j] + k);
            xb[j] = load16(xrow[j] + k + 8);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b < nb) {
                const Pack16 wa = load16(wrow[b] + k);
                const Pack16 wb = load16(wrow[b] + k + 8);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[b][j] = mfma16x16x32(wa, xa[j], acc[b][j]);
                    acc[b][j] = mfma16x16x32(wb, xb[j], acc[b][j]);
                }
            }
        }
    }
}

// Whole router in one workgroup per 32 tokens: full-K logits into LDS, then 8 tokens per wave.
__global__ __launch_bounds__(256) void router_fused_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T, int H, int E,
                                                           int k, float scale, int32_t* __restrict__ ids,
                                                           float* __restrict__ gates, float* __restrict__ logits) {
    __shared__ float zs[kBT][kMaxE + 4];
    const int t0 = blockIdx.x * kBT;
    f32x4 acc[4][2];
    router_accumulate(x, wr, T, H, E, t0, 0, H / 64, acc);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = wave * 64 + b * 16 + 4 * (lane >> 4) + r;
                const int tl = j * 16 + (lane & 15);
                if (e < E) zs[tl][e] = acc[b][j][r];
            }
    __syncthreads();
    for (int tl = wave; tl < kBT; tl += 4) {
        const int t = t0 + tl;
        if (t >= T) break;
        float z4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + 64 * q;
            z4[q] = e < E ? zs[tl][e] : 0.f;
        }
        topk_token(z4, t, E, k, scale, bias, ids, gates, logits);
    }
}

// Logits for at most 16 tokens: one wave per (16 experts, K range) workgroup, 16x16x32 MFMAs over
// 32-wide K chunks (experts are the A rows, tokens the B columns), every chunk's loads issued before its
// MFMAs; each workgroup writes its fp32 partial z for its experts. Many small workgroups keep the whole
// of W_r streaming at once, which a few large ones cannot at decode sizes.
__global__ __launch_bounds__(64) void router_small_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr, int T, int H, int E, int S,
                                                          float* __restrict__ partial, int32_t* __restrict__ ticket) {
    // the decode route-and-permute kernel that follows counts its finished workgroups on `ticket`
    if (ticket != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *ticket = 0;
    const int groups = (E + 15) / 16;
    const int eg = blockIdx.x % groups;
    const int s = blockIdx.x / groups;
    const int lane = threadIdx.x;
    const int rl = lane & 15, kg = lane >> 4;
    const int C = H / 32;
    const int c0 = (int)((int64_t)s * C / S), c1 = (int)((int64_t)(s + 1) * C / S);
    int e = eg * 16 + rl;
    e = e < E ? e : E - 1;
    int t = rl < T ? rl : T - 1;
    const uint16_t* wrow = wr + (size_t)e * H + kg * 8;
    const uint16_t* xrow = x + (size_t)t * H + kg * 8;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = c0; c < c1; c += 4) {
        Pack16 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (c + i < c1) {
                a[i] = load16(wrow + (c + i) * 32);
                b[i] = load16(xrow + (c + i) * 32);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (c + i < c1) acc = mfma16x16x32(a[i], b[i], acc);
    }
    // element r: expert eg * 16 + 4 kg + r, token rl
    if (rl >= T) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ee = eg * 16 + 4 * kg + r;
        if (ee < E) partial[((size_t)s * T + rl) * E + ee] = acc[r];
    }
}

// Sums the S partial logits of each token in split order, then routes it (one wave per token, four
// tokens per workgroup; many tokens).
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial, int S,
                                                          const float* __restrict__ bias, int T, int E, int k,
                                                          float scale, int32_t* __restrict__ ids,
                                                          float* __restrict__ gates, float* __restrict__ logits) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    float z4[4];
    const size_t stride = (size_t)T * E;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        float z = 0.f;
        if (e < E) {
            const float* p = partial + (size_t)t * E + e;
            int s = 0;
            for (; s + 4 <= S; s += 4) { // four independent loads in flight, added in split order
                const float p0 = p[(size_t)s * stride], p1 = p[(size_t)(s + 1) * stride];
                const float p2 = p[(size_t)(s + 2) * stride], p3 = p[(size_t)(s + 3) * stride];
                z += p0;
                z += p1;
                z += p2;
                z += p3;
            }
            for (; s < S; ++s) z += p[(size_t)s * stride];
        }
        z4[q] = z;
    }
    topk_token(z4, t, E, k, scale, bias, ids, gates, logits);
}

// The same for a few tokens: one workgroup per token, one thread per expert with all S loads in flight
// at once (latency, not throughput, bounds decode), then one wave routes the token.
__global__ __launch_bounds__(256) void router_topk_few_kernel(const float* __restrict__ partial, int S,
                                                          const float* __restrict__ bias, int T, int E, int k,
                                                          float scale, int32_t* __restrict__ ids,
                                                          float* __restrict__ gates, float* __restrict__ logits) {
    __shared__ float zs[kMaxE];
    const int t = blockIdx.x;
    const int e = threadIdx.x;
    if (e < E) {
        const size_t stride = (size_t)T * E;
        const float* p = partial + (size_t)t * E + e;
        float v[kRouterMaxSplits];
#pragma unroll
        for (int i = 0; i < kRouterMaxSplits; ++i)
            if (i < S) v[i] = p[(size_t)i * stride];
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < kRouterMaxSplits; ++i)
            if (i < S) z += v[i];
        zs[e] = z;
    }
    __syncthreads();
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    float z4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) z4[q] = lane + 64 * q < E ? zs[lane + 64 * q] : 0.f;
    topk_token(z4, t, E, k, scale, bias, ids, gates, logits);
}

} // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E, int k,
                         float scale, int32_t* ids, float* gates, float* logits, float* partial, int S,
                         hipStream_t stream) {
    if (partial == nullptr) {
        const int tblocks = (T + kBT - 1) / kBT;
        router_fused_kernel<<<tblocks, 256, 0, stream>>>(x, wr, bias, T, H, E, k, scale, ids, gates, logits);
        return hipGetLastError();
    }
    if (T <= kRouterSmallT) {
        const int groups = (E + 15) / 16;
        router_small_kernel<<<groups * S, 64, 0, stream>>>(x, wr, T, H, E, S, partial, nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        router_topk_few_kernel<<<T, 256, 0, stream>>>(partial, S, bias, T, E, k, scale, ids, gates, logits);
        return hipGetLastError();
    }
    // logits as a dense GEMM (W_r rows x token tiles), K split S ways into fp32 partials, then the top-k
    GemmArgs g{};
    g.act = x;
    g.w_a = wr;
    g.out = partial;
    g.dense_rows = T;
    g.N = E;
    g.K = H;
    g.ksplit = S < 1 ? 1 : S;
    hipError_t e = launch_gemm(GemmKind::Logits, GemmPath::Wide, g, ((int64_t)T + kWideBM - 1) / kWideBM, stream);
    if (e != hipSuccess) return e;
    router_topk_kernel<<<(T + 3) / 4, 256, 0, stream>>>(partial, g.ksplit, bias, T, E, k, scale, ids, gates,
                                                         logits);
    return hipGetLastError();
}

hipError_t launch_router_logits_small(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* partial,
                                     int S, int32_t* ticket, hipStream_t stream) {
    const int groups = (E + 15) / 16;
    router_small_kernel<<<groups * S, 64, 0, stream>>>(x, wr, T, H, E, S, partial, ticket);
    return hipGetLastError();
}

} // namespace moe
