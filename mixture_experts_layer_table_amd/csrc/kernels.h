// Host-side launchers of the device code (one per C-ABI entry point).
#pragma once
#include <hip/hip_runtime.h>

#include "plan.h"

namespace mok {

// Records `err` (with the call site) as the calling thread's last error when it
// is not hipSuccess, and maps it to a status.
mok_status check_hip(hipError_t err, const char *where);
// Sets the calling thread's mok_last_error text.
void set_last_error(const char *text);

mok_status launch_build_schedule(const Plan &p, const int32_t *ids, void *schedule, hipStream_t st);

// Enqueues the fingerprint check of a schedule table against the plan of the
// call that is about to read it (sets MOK_SCHEDULE_MISMATCH on a mismatch).
mok_status launch_schedule_check(const Plan &p, const void *schedule, hipStream_t st);

mok_status launch_forward(const Plan &p, const void *schedule, void *workspace, const uint16_t *x,
                          const float *topk_w, const mok_weights &w, uint16_t *out, void *fwd_ctx,
                          hipStream_t st);

mok_status launch_backward(const Plan &p, const void *schedule, void *workspace, const uint16_t *x,
                           const float *topk_w, const mok_weights &w, const void *fwd_ctx,
                           const uint16_t *dy, uint16_t *dx, uint16_t *dw_gate, uint16_t *dw_up,
                           uint16_t *dw_down, float *dtopk_w, hipStream_t st);

mok_status launch_mxfp8_quantize(const uint16_t *src, int64_t batch, int64_t rows, int64_t K,
                                 bool src_is_k_by_rows, uint8_t *elems, uint8_t *scales, hipStream_t st);

mok_status launch_route(const float *logits, int64_t T, int E, int k, int32_t *ids, float *w, hipStream_t st);

mok_status launch_route_backward(const int32_t *ids, const float *w, const float *dw, int64_t T, int E, int k,
                                 float *dl, hipStream_t st);

}  // namespace mok
