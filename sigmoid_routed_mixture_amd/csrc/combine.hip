// Gate-weighted combine on gfx950: out[t] = sum_j G[t, j] * y[slot_row[t, j]] + y_shared[t] (+ x'[t]), in
// fp32 with the k slots added in slot order, then the shared expert, then (block entry point) the residual
// stream. The per-slot expert outputs y are fp32 or bf16 rows (widened to fp32 exactly), y_shared fp32.
// Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (y_routed = sum_i G_i E_i,
// delta_ffn = y_routed + y_shared, x_{n+1} = x'_n + delta_ffn); nnterp encyclopedia glm_moe_dsa, "The
// mixture" (routed + shared == out).
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

// 8 consecutive values of a per-slot row as fp32.
__device__ __forceinline__ void load_row8(const float* y, size_t i, float4& a, float4& b) {
    a = *reinterpret_cast<const float4*>(y + i);
    b = *reinterpret_cast<const float4*>(y + i + 4);
}
__device__ __forceinline__ void load_row8(const uint16_t* y, size_t i, float4& a, float4& b) {
    const Pack16 q = load16(y + i);
    a = make_float4(bf16_to_f32((uint16_t)(q.w[0] & 0xFFFFu)), bf16_to_f32((uint16_t)(q.w[0] >> 16)),
                    bf16_to_f32((uint16_t)(q.w[1] & 0xFFFFu)), bf16_to_f32((uint16_t)(q.w[1] >> 16)));
    b = make_float4(bf16_to_f32((uint16_t)(q.w[2] & 0xFFFFu)), bf16_to_f32((uint16_t)(q.w[2] >> 16)),
                    bf16_to_f32((uint16_t)(q.w[3] & 0xFFFFu)), bf16_to_f32((uint16_t)(q.w[3] >> 16)));
}

// One workgroup per (token, column range); each thread owns 8-column chunks (16-byte loads and stores).
// The k slot rows of a chunk are loaded eight at a time before any is added, so their latencies overlap;
// they are added in slot order. The shared expert's row and the residual do not depend on the slot rows:
// when every thread has one chunk (few tokens, latency-bound) they are loaded before the workgroup reads its
// slots, so their latency hides under the slots'; with several chunks per thread after each chunk's slots.
template <typename Y>
__global__ __launch_bounds__(256) void combine_kernel(const Y* __restrict__ y, const float* __restrict__ gates,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ y_shared,
                                                      const uint16_t* __restrict__ resid, int T, int H, int k,
                                                      float* __restrict__ out, const float* __restrict__ y2,
                                                      const float* __restrict__ y_shared2,
                                                      const int32_t* __restrict__ ysplit, size_t pstride) {
    __shared__ float g[kMaxK];
    __shared__ int rr[kMaxK];
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    // the down GEMM split K into S ranges: a row of y is its first range plus the same row of each of the
    // S - 1 partial buffers y2 + p * pstride, added in range order
    int S = ysplit != nullptr ? ysplit[0] : 1;
    S = S < 1 ? 1 : S > kMaxDownSplits ? kMaxDownSplits : S;
    if (tid < k) {
        g[tid] = gates[(size_t)t * k + tid];
        rr[tid] = slot_row[(size_t)t * k + tid];
    }
    const int chunks = H / 8, stride = (int)blockDim.x * gridDim.y;
    int c = blockIdx.y * (int)blockDim.x + tid;
    // shared-expert row (each range's with a split) and residual of chunk c
    float4 sa[kMaxDownSplits], sb[kMaxDownSplits];
    Pack16 res{};
    auto extras = [&](int cc) {
        const size_t i = (size_t)t * H + cc * 8;
        if (y_shared) {
            sa[0] = *reinterpret_cast<const float4*>(y_shared + i);
            sb[0] = *reinterpret_cast<const float4*>(y_shared + i + 4);
#pragma unroll
            for (int p = 1; p < kMaxDownSplits; ++p)
                if (p < S) {
                    sa[p] = *reinterpret_cast<const float4*>(y_shared2 + (p - 1) * pstride + i);
                    sb[p] = *reinterpret_cast<const float4*>(y_shared2 + (p - 1) * pstride + i + 4);
                }
        }
        if (resid) res = load16(resid + i);
    };
    const bool one = stride >= chunks; // uniform: at most one chunk per thread
    if (one && c < chunks) extras(c);
    __syncthreads();
    for (; c < chunks; c += stride) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j0 = 0; j0 < k; j0 += 8) {
            float4 v0[8], v1[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int j = j0 + jj;
                const int r = j < k ? rr[j] : -1;
                if (r >= 0) {
                    load_row8(y, (size_t)r * H + c * 8, v0[jj], v1[jj]);
#pragma unroll
                    for (int p = 1; p < kMaxDownSplits; ++p)
                        if (p < S) {
                            const float* q = y2 + (p - 1) * pstride + (size_t)r * H + c * 8;
                            const float4 a = *reinterpret_cast<const float4*>(q);
                            const float4 b = *reinterpret_cast<const float4*>(q + 4);
                            v0[jj] = make_float4(v0[jj].x + a.x, v0[jj].y + a.y, v0[jj].z + a.z, v0[jj].w + a.w);
                            v1[jj] = make_float4(v1[jj].x + b.x, v1[jj].y + b.y, v1[jj].z + b.z, v1[jj].w + b.w);
                        }
                }
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int j = j0 + jj;
                if (j < k && rr[j] >= 0) {
                    const float gj = g[j];
                    acc[0] += gj * v0[jj].x; acc[1] += gj * v0[jj].y; acc[2] += gj * v0[jj].z; acc[3] += gj * v0[jj].w;
                    acc[4] += gj * v1[jj].x; acc[5] += gj * v1[jj].y; acc[6] += gj * v1[jj].z; acc[7] += gj * v1[jj].w;
                }
            }
        }
        float* o = out + (size_t)t * H + c * 8;
        if (!one) extras(c);
        if (y_shared) {
            float4 s0 = sa[0], s1 = sb[0];
#pragma unroll
            for (int p = 1; p < kMaxDownSplits; ++p)
                if (p < S) {
                    s0 = make_float4(s0.x + sa[p].x, s0.y + sa[p].y, s0.z + sa[p].z, s0.w + sa[p].w);
                    s1 = make_float4(s1.x + sb[p].x, s1.y + sb[p].y, s1.z + sb[p].z, s1.w + sb[p].w);
                }
            acc[0] += s0.x; acc[1] += s0.y; acc[2] += s0.z; acc[3] += s0.w;
            acc[4] += s1.x; acc[5] += s1.y; acc[6] += s1.z; acc[7] += s1.w;
        }
        if (resid) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += bf16_to_f32((uint16_t)(res.w[i] & 0xFFFFu));
                acc[2 * i + 1] += bf16_to_f32((uint16_t)(res.w[i] >> 16));
            }
        }
        *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

} // namespace

hipError_t launch_combine(const void* y, bool y_bf16, const float* gates, const int32_t* slot_row,
                          const float* y_shared, const uint16_t* resid, int T, int H, int k, float* out,
                          hipStream_t stream, const float* y2, const float* y_shared2, const int32_t* ysplit,
                          size_t part_stride) {
    if (ysplit != nullptr && (y_bf16 || y2 == nullptr || (y_shared != nullptr && y_shared2 == nullptr)))
        return hipErrorInvalidValue;
    if (T <= 0) return hipSuccess;
    // few tokens: spread each token's row over several workgroups so every thread has one chunk
    // few tokens: one-wave workgroups spread each token's row over many CUs, every thread one chunk (the
    // slot loads of a token then come from as many CUs as the row has 512-column pieces); many tokens: a
    // workgroup of 256 threads per token
    const int threads = T < 1024 ? 64 : 256;
    const int ycols = T < 1024 ? (H / 8 + threads - 1) / threads : 1;
    if (y_bf16)
        combine_kernel<<<dim3(T, ycols), threads, 0, stream>>>(static_cast<const uint16_t*>(y), gates, slot_row, y_shared,
                                                          resid, T, H, k, out, y2, y_shared2, ysplit, part_stride);
    else
        combine_kernel<<<dim3(T, ycols), threads, 0, stream>>>(static_cast<const float*>(y), gates, slot_row, y_shared,
                                                          resid, T, H, k, out, y2, y_shared2, ysplit, part_stride);
    return hipGetLastError();
}

} // namespace moe
