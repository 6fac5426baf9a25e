// MXFP8 block codec on the device (OCP MX v1.0 MXFP8: 32 contiguous values
// share an E8M0 scale, elements are E4M3FN; "Mixture-of-Kittens (MoK)" project
// summary, Key-concepts table, names MXFP8 as the low-precision format).
//
// Integer-only, on the bit patterns of bf16 or fp32 inputs, so the result does
// not depend on any floating-point rounding mode:
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

// E4M3FN code of sign * V * 2^X times 2^-e (V an integer significand).
__device__ __forceinline__ uint32_t e4m3_from_parts(uint32_t sign, uint32_t V, int X) {
    uint32_t code = 0;
    if (V != 0) {
        const int bl = 32 - __clz(V);                    // bit length of V
        const int B = bl - 1 + X;                        // binade: floor(log2 |value|)
        const int Qe = B < -6 ? -9 : B - 3;              // exponent of E4M3's quantum
        const int shift = Qe - X;
        uint32_t n;
        if (shift <= 0) {
            n = V << (-shift);
        } else if (shift > 25) {
            n = 0;                                       // below half a quantum (V < 2^25)
        } else {
            n = V >> shift;
            const uint32_t rem = V & ((1u << shift) - 1u), half = 1u << (shift - 1);
            if (rem > half || (rem == half && (n & 1u))) ++n;
        }
        if (Qe == -9)
            code = n;                                    // subnormal (n == 8 is the smallest normal)
        else
            code = (uint32_t)((B + 7) << 3) + (n - 8);   // n == 16 carries into the next binade
        code = min(code, 0x7Eu);                         // saturate at 448
    }
    return code | (sign << 7);
}

__device__ __forceinline__ uint32_t e4m3_encode_bf16(uint32_t b, int e) {
    const int ev = (int)((b >> 7) & 0xFFu);
    const uint32_t mv = b & 0x7Fu;
    return e4m3_from_parts((b >> 15) & 1u, ev ? (0x80u | mv) : mv, (ev ? ev : 1) - 134 - e);
}

__device__ __forceinline__ uint32_t e4m3_encode_f32(uint32_t b, int e) {
    const int ev = (int)((b >> 23) & 0xFFu);
    const uint32_t mv = b & 0x7FFFFFu;
    return e4m3_from_parts(b >> 31, ev ? (0x800000u | mv) : mv, (ev ? ev : 1) - 150 - e);
}

}  // namespace mok
