// Device-side types and helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16 bytes = 8 bf16 values, the operand of one lane of a 16x16x32 bf16 MFMA.
struct alignas(16) Pack16 {
    uint32_t w[4];
};

__device__ __forceinline__ Pack16 load16(const void* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return Pack16{{v.x, v.y, v.z, v.w}};
}

__device__ __forceinline__ void store16(void* p, const Pack16& v) {
    *reinterpret_cast<uint4*>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const Pack16& v) { return __builtin_bit_cast(bf16x8, v); }

// D = A * B + C for one 16x16x32 bf16 tile with fp32 accumulation (v_mfma_f32_16x16x32_bf16).
// Lane l supplies A row (l % 16) and B column (l % 16), each 8 consecutive k of the 32 (k-group l / 16);
// D row 4 * (l / 16) + r, column l % 16, sits in element r of lane l's result.
__device__ __forceinline__ f32x4 mfma16x16x32(const Pack16& a, const Pack16& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// silu(g) * u with the sigmoid in fp32: g times the hardware reciprocal (v_rcp_f32, 1 ulp) of 1 + exp(-g)
// instead of an IEEE division (a dozen instructions per value in the gate/up epilogue; h is rounded to bf16
// right after). For g far below zero 1 + exp(-g) overflows to infinity and the product is -0, as the
// division gives.
__device__ __forceinline__ float swiglu(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

} // namespace moe
