// Router front-end: logits to top-k expert ids and renormalised gate weights,
// and the logit gradient. The layer takes the top-k choice as an input of
// schedule building ("Mixture-of-Kittens (MoK)" project summary, Functional
// API) in a sparse layer where each token activates a few experts
// ("Mixture-of-Kittens(MoK)란?" explainer, section 1); the router itself
// follows the plainest reading: softmax over all experts, the k largest
// logits (descending, the lower expert index first among equal logits), and
// weights renormalised over the chosen k:
//   w_j = exp(l_j - m) / sum_i exp(l_i - m)   over the chosen i, m = max logit
// (the full softmax's denominator cancels in the renormalisation).
// Backward (the choice is piecewise constant):
//   dl_e = w_e (dw_e - sum_j w_j dw_j) for chosen e, 0 for the others.
//
// One wave per token. Expert e's logit is held by lane e % 64 in slot e / 64;
// slot j of the result (j < k) by lane j. Every reduction runs in a fixed
// order, so results do not depend on timing.
#include <cmath>

#include "common.h"
#include "kernels.h"
#include "timing.h"

namespace mok {
namespace {

constexpr int kRouteWaves = 4;   // tokens per workgroup

// (value, index) order of the choice: larger value first, lower index first among equal values.
__device__ __forceinline__ bool before(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }

// Sum over the 64 lanes in a fixed order (xor butterfly); every lane returns lane 0's total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return __shfl(x, 0);
}

template <int SLOTS>
__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(const float *__restrict__ logits, int64_t T, int E,
                                                                 int k, int32_t *__restrict__ ids,
                                                                 float *__restrict__ w) {
    const int64_t t = (int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
    if (t >= T) return;   // a whole wave
    const int lane = threadIdx.x & 63;
    const float *row = logits + t * E;
    float v[SLOTS];
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
        const int e = s * 64 + lane;
        v[s] = e < E ? row[e] : -INFINITY;
    }
    uint32_t taken = 0;   // bit s: slot s already chosen
    float my_v = 0.0f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            const int e = s * 64 + lane;
            if (e < E && !((taken >> s) & 1u) && before(v[s], e, bv, be)) {
                bv = v[s];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oe = __shfl_xor(be, off);
            if (before(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        // every lane now holds the j-th choice (a strict order: one winner)
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }
    const float m = __shfl(my_v, 0);
    const float ex = lane < k ? expf(my_v - m) : 0.0f;
    const float sum = wave_sum(ex);
    if (lane < k) {
        ids[t * k + lane] = my_e;
        w[t * k + lane] = ex / sum;
    }
}

template <int SLOTS>
__global__ __launch_bounds__(64 * kRouteWaves) void route_backward_kernel(const int32_t *__restrict__ ids,
                                                                          const float *__restrict__ w,
                                                                          const float *__restrict__ dw, int64_t T,
                                                                          int E, int k, float *__restrict__ dl) {
    const int64_t t = (int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const float wj = lane < k ? w[t * k + lane] : 0.0f;
    const float dwj = lane < k ? dw[t * k + lane] : 0.0f;
    const int ej = lane < k ? ids[t * k + lane] : -1;
    const float s = wave_sum(wj * dwj);
    const float gj = wj * (dwj - s);
    float g[SLOTS];
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) g[q] = 0.0f;
    for (int j = 0; j < k; ++j) {   // each entry is written once, by the lane that owns it
        const int e = __shfl(ej, j);
        const float gg = __shfl(gj, j);
        if (e >= 0 && e < E && (e & 63) == lane) {
#pragma unroll
            for (int q = 0; q < SLOTS; ++q)
                if (q == (e >> 6)) g[q] = gg;
        }
    }
    float *row = dl + t * E;
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
        const int e = q * 64 + lane;
        if (e < E) row[e] = g[q];
    }
}

int slots_for(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

}  // namespace

mok_status launch_route(const float *logits, int64_t T, int E, int k, int32_t *ids, float *w, hipStream_t st) {
    const unsigned blocks = (unsigned)((T + kRouteWaves - 1) / kRouteWaves);
    KernelTimer tm("route", st);
    switch (slots_for(E)) {
        case 1: route_kernel<1><<<blocks, 64 * kRouteWaves, 0, st>>>(logits, T, E, k, ids, w); break;
        case 2: route_kernel<2><<<blocks, 64 * kRouteWaves, 0, st>>>(logits, T, E, k, ids, w); break;
        case 4: route_kernel<4><<<blocks, 64 * kRouteWaves, 0, st>>>(logits, T, E, k, ids, w); break;
        case 8: route_kernel<8><<<blocks, 64 * kRouteWaves, 0, st>>>(logits, T, E, k, ids, w); break;
        default: route_kernel<16><<<blocks, 64 * kRouteWaves, 0, st>>>(logits, T, E, k, ids, w); break;
    }
    return check_hip(hipGetLastError(), "mok_route");
}

mok_status launch_route_backward(const int32_t *ids, const float *w, const float *dw, int64_t T, int E, int k,
                                 float *dl, hipStream_t st) {
    const unsigned blocks = (unsigned)((T + kRouteWaves - 1) / kRouteWaves);
    KernelTimer tm("route_backward", st);
    switch (slots_for(E)) {
        case 1: route_backward_kernel<1><<<blocks, 64 * kRouteWaves, 0, st>>>(ids, w, dw, T, E, k, dl); break;
        case 2: route_backward_kernel<2><<<blocks, 64 * kRouteWaves, 0, st>>>(ids, w, dw, T, E, k, dl); break;
        case 4: route_backward_kernel<4><<<blocks, 64 * kRouteWaves, 0, st>>>(ids, w, dw, T, E, k, dl); break;
        case 8: route_backward_kernel<8><<<blocks, 64 * kRouteWaves, 0, st>>>(ids, w, dw, T, E, k, dl); break;
        default: route_backward_kernel<16><<<blocks, 64 * kRouteWaves, 0, st>>>(ids, w, dw, T, E, k, dl); break;
    }
    return check_hip(hipGetLastError(), "mok_route_backward");
}

}  // namespace mok
