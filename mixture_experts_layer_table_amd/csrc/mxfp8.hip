// MXFP8 weight quantization ("Mixture-of-Kittens (MoK)" project summary,
// Key-concepts table: weights are quantized before the kernel runs), in the
// OCP MX v1.0 MXFP8 block format: 32 contiguous values share an E8M0 scale,
// elements are E4M3FN.
//
// Integer-only implementation on bf16 bit patterns, so the result does not
// depend on any floating-point rounding mode:
//   scale byte = 127 for an all-zero block, else max(0, exp_field(amax) - 8)
//              (= clamp(floor(log2 amax) - 8, -127, 127) + 127; bf16 subnormal
//              maxima land on the lower clamp)
//   element    = the input's 8-bit significand shifted to E4M3's quantum for
//                its binade, rounded to nearest even, saturated to 448 (0x7E),
//                sign kept.
#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace mok {

__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits /* |bf16| bits */) {
    if (amax_bits == 0) return 127u;
    const int ef = (int)(amax_bits >> 7);
    return (uint32_t)max(0, ef - 8);
}

// E4M3FN code of bf16 value `b` times 2^-e.
__device__ __forceinline__ uint32_t e4m3_encode(uint32_t b, int e) {
    const uint32_t sign = (b >> 15) & 1u;
    const int ev = (int)((b >> 7) & 0xFFu);
    const uint32_t mv = b & 0x7Fu;
    const uint32_t V = ev ? (0x80u | mv) : mv;           // significand, value = V * 2^X
    uint32_t code = 0;
    if (V != 0) {
        const int X = (ev ? ev : 1) - 134 - e;
        const int bl = 32 - __clz(V);                    // bit length of V
        const int B = bl - 1 + X;                        // binade: floor(log2 |value|)
        const int Qe = B < -6 ? -9 : B - 3;              // exponent of E4M3's quantum
        const int shift = Qe - X;
        uint32_t n;
        if (shift <= 0) {
            n = V << (-shift);
        } else if (shift > 9) {
            n = 0;
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

// One thread per 32-value block.
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t *__restrict__ src, int64_t batch,
                                                             int64_t rows, int64_t K, int transposed,
                                                             uint8_t *__restrict__ elems,
                                                             uint8_t *__restrict__ scales) {
    const int64_t nkb = K / 32;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= batch * rows * nkb) return;
    int64_t b, r, kb;
    if (transposed) {   // row fastest, so that neighbouring threads read neighbouring columns
        r = idx % rows;
        kb = (idx / rows) % nkb;
        b = idx / (rows * nkb);
    } else {
        kb = idx % nkb;
        r = (idx / nkb) % rows;
        b = idx / (nkb * rows);
    }
    uint32_t v[32];
    if (transposed) {
        const uint16_t *p = src + (b * K + kb * 32) * rows + r;
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = p[(int64_t)i * rows];
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(src + (b * rows + r) * K + kb * 32);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 x = p[c];
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[c * 8 + 2 * j] = w[j] & 0xFFFFu;
                v[c * 8 + 2 * j + 1] = w[j] >> 16;
            }
        }
    }
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, v[i] & 0x7FFFu);   // |bf16| orders like its bits
    const uint32_t sb = mx_scale_byte(amax);
    const int e = (int)sb - 127;
    uint32_t packed[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) x |= e4m3_encode(v[w * 4 + j], e) << (8 * j);
        packed[w] = x;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(elems + (b * rows + r) * K + kb * 32);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    scales[(b * rows + r) * nkb + kb] = (uint8_t)sb;
}

mok_status launch_mxfp8_quantize(const uint16_t *src, int64_t batch, int64_t rows, int64_t K,
                                 bool src_is_k_by_rows, uint8_t *elems, uint8_t *scales, hipStream_t st) {
    const int64_t n = batch * rows * (K / 32);
    if (n == 0) return MOK_OK;
    const int64_t blocks = (n + 255) / 256;
    KernelTimer tm("mxfp8_quantize", st);
    mxfp8_quantize_kernel<<<(unsigned)blocks, 256, 0, st>>>(src, batch, rows, K, src_is_k_by_rows ? 1 : 0, elems,
                                                            scales);
    return check_hip(hipGetLastError(), "mok_mxfp8_quantize");
}

}  // namespace mok
