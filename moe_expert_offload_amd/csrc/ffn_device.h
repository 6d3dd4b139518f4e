// Device helpers shared by the per-token GEMV FFN kernels and the grouped
// MFMA FFN kernels: bf16 and E8M0 conversions and streaming loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// E8M0 -> float: 2^(E-127); E = 0 is 2^-127 (a denormal), E = 255 is NaN
__device__ __forceinline__ float e8m0(uint32_t e) {
    e &= 0xFFu;
    float f = __uint_as_float(e << 23);
    f = e == 0u ? __uint_as_float(0x00400000u) : f;
    return e == 255u ? __uint_as_float(0x7FC00000u) : f;
}

// float -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// streaming 16-byte load (weights are read once per layer step)
__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// SwiGLU gate: silu(g) * u = g / (1 + e^-g) * u (e^-g = inf gives -0 or +0)
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

}  // namespace moe
