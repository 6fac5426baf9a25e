// MXFP8 block codec on the device (OCP MX v1.0 MXFP8: 32 contiguous values
// share an E8M0 scale, elements are E4M3FN; "Mixture-of-Kittens (MoK)" project
// summary, Key-concepts table, names MXFP8 as the low-precision format).
//
// The scale byte comes from the bit pattern of the block's largest magnitude;
// elements are rounded by the hardware conversion on exactly scaled values:
//   scale byte = 127 for an all-zero block, else clamp(floor(log2 amax) - 8,
//                -127, 127) + 127, which is max(0, biased exponent of amax - 8)
//                (subnormal maxima land on the lower clamp)
//   element    = the value times 2^-e rounded to E4M3's quantum for its binade,
//                to nearest even, saturated to 448 (0x7E), sign kept.
#pragma once
#include "common.h"

namespace mok {

// Scale byte from the biased exponent field of amax (0 and amax == 0 handled).
__device__ __forceinline__ uint32_t mx_scale_from_exp(uint32_t biased_exp, bool zero) {
    return zero ? 127u : (uint32_t)max(0, (int)biased_exp - 8);
}
__device__ __forceinline__ uint32_t mx_scale_byte_bf16(uint32_t amax_bits /* |bf16| bits */) {
    return mx_scale_from_exp(amax_bits >> 7, amax_bits == 0);
}
__device__ __forceinline__ uint32_t mx_scale_byte_f32(uint32_t amax_bits /* |fp32| bits */) {
    return mx_scale_from_exp(amax_bits >> 23, amax_bits == 0);
}

// E4M3FN code of a finite value v times 2^-e. 2^-e is a normal float for
// every scale exponent a block can have (e = scale byte - 127, -127 .. 119),
// so v * 2^-e is exact wherever E4M3 can represent anything (below 2^-126 it
// rounds to a signed zero either way); magnitudes past 448 are clamped to it
// (saturation); and the hardware conversion (v_cvt_pk_fp8_f32: OCP E4M3FN,
// round to nearest even, the sign of zero kept) rounds the rest. A GPU test
// holds it to the oracle's rule bit for bit for every finite bf16 pattern at
// every scale exponent; for fp32 inputs it was checked against a bit-level
// integer form of the rule on 2^28 hashed patterns and on every exponent
// field x 4,096 mantissas (E4M3's rounding bits swept) x both signs x every
// scale exponent, with no difference.
__device__ __forceinline__ float mx_pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
__device__ __forceinline__ float mx_clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Two codes (bytes 0 and 1) of a and b, already multiplied by 2^-e.
__device__ __forceinline__ uint32_t e4m3x2_scaled(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(mx_clamp448(a), mx_clamp448(b), 0, false) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t e4m3_encode_f32(uint32_t b, int e) {
    return e4m3x2_scaled(__uint_as_float(b) * mx_pow2_neg(e), 0.0f) & 0xFFu;
}
__device__ __forceinline__ uint32_t e4m3_encode_bf16(uint32_t b, int e) {
    return e4m3_encode_f32(b << 16, e);
}
// Four codes (bytes 0..3) of the bf16 pairs w0 = (lo, hi) and w1 = (lo, hi).
__device__ __forceinline__ uint32_t e4m3x4_bf16(uint32_t w0, uint32_t w1, int e) {
    const float s = mx_pow2_neg(e);
    return e4m3x2_scaled(__uint_as_float(w0 << 16) * s, __uint_as_float(w0 & 0xFFFF0000u) * s) |
           (e4m3x2_scaled(__uint_as_float(w1 << 16) * s, __uint_as_float(w1 & 0xFFFF0000u) * s) << 16);
}

}  // namespace mok
