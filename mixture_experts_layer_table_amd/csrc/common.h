// Device-side helpers shared by the HIP kernels of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mok {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// low halves (resp. high halves) of two dwords a, b packed as (a, b)
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
    return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xFFFF0000u);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace mok
