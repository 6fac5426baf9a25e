// MXFP8 weight quantization ("Mixture-of-Kittens (MoK)" project summary,
// Key-concepts table: weights are quantized before the kernel runs), in the
// OCP MX v1.0 MXFP8 block format: 32 contiguous values share an E8M0 scale,
// elements are E4M3FN.
// The codec itself (integer-only, bit-exact) is in mx_codec.h.
#include "common.h"
#include "mx_codec.h"
#include "kernels.h"
#include "timing.h"

namespace mok {

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
    const uint32_t sb = mx_scale_byte_bf16(amax);
    const int e = (int)sb - 127;
    uint32_t packed[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        packed[w] = e4m3x4_bf16(v[w * 4] | (v[w * 4 + 1] << 16), v[w * 4 + 2] | (v[w * 4 + 3] << 16), e);
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
