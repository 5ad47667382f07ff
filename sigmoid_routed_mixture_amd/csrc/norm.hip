// RMSNorm of the residual stream before the mixture on gfx950: x_ffn = gamma * x' / sqrt(mean(x'^2) + eps),
// stored as bf16 (the mixture's input dtype).
// Pages: open-model-atlas GLM-5 "MoE transformer block", "All 43 steps" (x_ffn = RMSNorm(x'_n) feeds the
// router, the routed experts and the shared expert); nnterp encyclopedia glm_moe_dsa / glm4_moe_lite module
// trees (post_attention_layernorm, an RMSNorm over the hidden size with eps 1e-5, is the MLP's input norm).
//
// The arithmetic is fp64: the sum of squares, rstd = 1 / sqrt(ss / H + eps), and (x * rstd) * gamma, which
// is then rounded to bf16 in one step (round to nearest, ties to even). In fp32 a result lying close to a
// bf16 rounding boundary could round the other way, and every such flip moves the router logits by about
// |W_r| * ulp; fp64 keeps the rounding decision stable. The pass reads x' twice (the second time from
// cache) and writes x_ffn once: it is HBM-bound and its fp64 work is a few operations per element.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

// double -> bf16 bits, round to nearest, ties to even. Normal results: bits 51..45 of the mantissa are
// kept and the 45 below decide the rounding (the carry may step the exponent, or reach infinity).
// Results below 2^-126 are multiples of 2^-133: |v| 2^133 rounded to an integer.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return 0x7FC0u; // NaN
    const int eb = (int)(a >> 52) - 1023 + 127;   // bf16 biased exponent of the unrounded value
    if (eb >= 1) {
        uint64_t r = ((uint64_t)eb << 52) | (a & 0x000FFFFFFFFFFFFFull);
        r += ((1ull << 44) - 1) + ((r >> 45) & 1ull);
        const uint64_t q = r >> 45;
        return q >= (255ull << 7) ? (uint16_t)(sign | 0x7F80u) : (uint16_t)(sign | q);
    }
    const double s = fabs(v) * 0x1p133; // exact: a power-of-two scaling of a value below 2^-126
    const double f = floor(s);
    const double rem = s - f;
    uint32_t n = (uint32_t)f;
    if (rem > 0.5 || (rem == 0.5 && (n & 1u))) ++n;
    return (uint16_t)(sign | n);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One workgroup per token; each thread owns 8-element chunks (16-byte loads and stores).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ gamma, double eps, int H,
                                                      uint16_t* __restrict__ out) {
    __shared__ double part[4];
    const size_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* row = x + t * (size_t)H;
    double ss = 0.0;
    for (int c = tid; c < H / 8; c += 256) {
        const Pack16 v = load16(row + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double lo = (double)bf16_to_f32((uint16_t)(v.w[i] & 0xFFFFu));
            const double hi = (double)bf16_to_f32((uint16_t)(v.w[i] >> 16));
            ss += lo * lo;
            ss += hi * hi;
        }
    }
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const double total = ((part[0] + part[1]) + part[2]) + part[3];
    const double rstd = 1.0 / sqrt(total / (double)H + eps);
    uint16_t* orow = out + t * (size_t)H;
    for (int c = tid; c < H / 8; c += 256) {
        const Pack16 v = load16(row + c * 8);
        const Pack16 g = load16(gamma + c * 8);
        Pack16 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double x0 = (double)bf16_to_f32((uint16_t)(v.w[i] & 0xFFFFu));
            const double x1 = (double)bf16_to_f32((uint16_t)(v.w[i] >> 16));
            const double g0 = (double)bf16_to_f32((uint16_t)(g.w[i] & 0xFFFFu));
            const double g1 = (double)bf16_to_f32((uint16_t)(g.w[i] >> 16));
            o.w[i] = (uint32_t)f64_to_bf16(x0 * rstd * g0) | ((uint32_t)f64_to_bf16(x1 * rstd * g1) << 16);
        }
        store16(orow + c * 8, o);
    }
}

} // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, double eps, int T, int H, uint16_t* out,
                          hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    rmsnorm_kernel<<<T, 256, 0, stream>>>(x, gamma, eps, H, out);
    return hipGetLastError();
}

} // namespace moe
