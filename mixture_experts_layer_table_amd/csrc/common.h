// Device-side helpers shared by the HIP kernels of the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mok {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// low halves (resp. high halves) of two dwords a, b packed as (a, b)
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
    return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xFFFF0000u);
}

// 1 / (1 + e^-z) with the hardware reciprocal (1 ulp) instead of an IEEE
// division: the SwiGLU epilogues evaluate it for every element of a tile.
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

}  // namespace mok
