// mok_forward_noalloc: the forward pass with its scratch in a static device
// array instead of a caller-given workspace, for callers that cannot allocate
// (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Same kernels and launches as mok_forward, so the same bits.
//
// The array lives in this library's code object: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. Host code
// never uses the array's name as an address (on the host it is only a stand-in
// symbol): the device copy's address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <cstdio>
#include <mutex>

#include "kernels.h"
#include "plan.h"

using namespace mok;

static __device__ __align__(256) unsigned char scratch[MOK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The current device's copy of `scratch` (looked up on the first call on it).
mok_status scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return check_hip(e, "mok_forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) {
        set_last_error("mok_forward_noalloc: device index beyond the library's table of 64");
        return MOK_ERROR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return check_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "mok_forward_noalloc: hipGetSymbolAddress");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return MOK_OK;
}

}  // namespace

extern "C" mok_status mok_forward_noalloc(const mok_config *cfg, const mok_shape *shape, const void *schedule,
                                          size_t schedule_bytes, const void *x, const float *topk_w,
                                          const mok_weights *w, void *out, void *fwd_ctx, size_t fwd_ctx_bytes,
                                          void *stream) {
    Plan full;
    mok_status s = make_plan(cfg, shape, &full);
    if (s != MOK_OK) return s;
    size_t need = 0;
    const Plan p = forward_only_workspace(full, &need);
    if (need > (size_t)MOK_NOALLOC_SCRATCH_BYTES) {
        char msg[192];
        std::snprintf(msg, sizeof msg,
                      "mok_forward_noalloc: the forward needs %zu bytes of scratch, more than the static %zu "
                      "(use a smaller ring_bytes or mok_forward with a workspace)",
                      need, (size_t)MOK_NOALLOC_SCRATCH_BYTES);
        set_last_error(msg);
        return MOK_ERROR_BUFFER_TOO_SMALL;
    }
    if (!w) return MOK_ERROR_INVALID_VALUE;
    if (!(p.debug & MOK_DEBUG_IDENTITY_EXPERT)) {
        if (p.precision == MOK_BF16 ? (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down))
                                    : (!aligned16(w->gate_elems) || !aligned16(w->gate_scales) ||
                                       !aligned16(w->up_elems) || !aligned16(w->up_scales) ||
                                       !aligned16(w->down_elems) || !aligned16(w->down_scales)))
            return MOK_ERROR_INVALID_VALUE;
    }
    if (!aligned16(schedule) || !aligned16(fwd_ctx)) return MOK_ERROR_INVALID_VALUE;
    if (p.R > 0 && (!aligned16(x) || !aligned16(topk_w) || !aligned16(out))) return MOK_ERROR_INVALID_VALUE;
    if (schedule_bytes < p.s_total || fwd_ctx_bytes < p.c_total) return MOK_ERROR_BUFFER_TOO_SMALL;
    (void)hipGetLastError();
    void *ws = nullptr;
    if ((s = scratch_on_current_device(&ws)) != MOK_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = launch_schedule_check(p, schedule, st)) != MOK_OK) return s;
    return launch_forward(p, schedule, ws, static_cast<const uint16_t *>(x), topk_w, *w, static_cast<uint16_t *>(out),
                          fwd_ctx, st);
}
