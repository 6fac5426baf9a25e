// MXFP8 mode of the layer: the per-round launches that differ from BF16
// (quantizing gathers and the four block-scaled GEMMs). Everything else of a
// pass (combines, router-gradient reduction, weight gradients) is shared.
#pragma once
#include <hip/hip_runtime.h>

#include "plan.h"
#include "views.h"

namespace mok {

struct TraceArgs;
// The per-item trace destination for the next launch of a GEMM kernel
// (kernel: a MOK_TRACE_* value; all null while tracing is off).
TraceArgs item_trace_args(int kernel);

// Forward round g0 .. g1-1: gather + quantize x rows into the ring (and, when
// xc is not null, the bf16 rows at their canonical positions in xc), gate/up
// GEMM (h and g * a -> fwd_ctx, a quantized along I -> the a-ring), down GEMM.
hipError_t mx_forward_round(const Plan &p, const SchedView &v, int g0, int g1, int64_t mt_bound,
                            const uint16_t *x, const mok_weights &w, char *ws, uint16_t *h, uint16_t *ga,
                            uint16_t *xc, const float *topk_w, uint16_t *out, uint16_t *stage, hipStream_t st);

// Backward round g0 .. g1-1, in two parts: the gather + quantize of the dy
// rows into the ring (and the bf16 rows at their canonical positions in dyc,
// when not null); then the dA GEMM with the SwiGLU backward (dh in bf16 and
// quantized along I) and the dX GEMM.
hipError_t mx_gather_dy(const Plan &p, const SchedView &v, int g0, int g1, const uint16_t *dy, char *ws,
                        uint16_t *dyc, hipStream_t st);
hipError_t mx_backward_gemms(const Plan &p, const SchedView &v, int g0, int g1, int64_t mt_bound,
                             const mok_weights &w, char *ws, const uint16_t *h, const float *topk_w, uint16_t *dx,
                             uint16_t *stage, hipStream_t st);

// MXFP8 weight gradients (MOK_MXFP8_WGRAD). begin, before the backward
// rounds: the padded expert offsets and x and dy quantized along the token
// axis, on the side stream forked from st (*side; st itself when none is
// available). finish, after the rounds: joins *side, then dh and g*a (ga,
// from fwd_ctx) quantized the same way (canonical order), then the two
// block-scaled weight-gradient GEMMs on st (compute = false: only the join,
// after an error). The quantized operands live in the workspace.
hipError_t mx_wgrad_begin(const Plan &p, const SchedView &v, char *ws, const uint16_t *x, const uint16_t *dy,
                          hipStream_t st, hipStream_t *side);
hipError_t mx_wgrad_finish(const Plan &p, const SchedView &v, char *ws, const uint16_t *ga, hipStream_t side,
                           bool compute, uint16_t *dw_gate, uint16_t *dw_up, uint16_t *dw_down, hipStream_t st);

}  // namespace mok
