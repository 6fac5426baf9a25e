// C ABI entry points: argument validation on the host, then launches.
#include <algorithm>
#include <cstdint>

#include "kernels.h"
#include "plan.h"

using namespace mok;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dev_ok(const void *p) { return p != nullptr && aligned16(p); }

}  // namespace

extern "C" {

mok_status mok_config_default(mok_config *cfg) {
    if (!cfg) return MOK_ERROR_INVALID_VALUE;
    cfg->minibatch_rows = 512;
    cfg->precision = MOK_BF16;
    cfg->macrobatch_tokens = 0;
    cfg->ring_bytes = int64_t(256) << 20;
    cfg->capacity_multiplier = 1.0f;
    cfg->debug_flags = 0;
    cfg->persistent_workgroups = 0;
    return MOK_OK;
}

mok_status mok_config_autosize(mok_config *cfg, const mok_shape *shape, int32_t n_cu) {
    if (!cfg || !shape) return MOK_ERROR_INVALID_VALUE;
    const int64_t units = n_cu > 0 ? n_cu : 256;
    // Validate the shape and the other knobs with the smallest mini-batch and
    // an unbounded ring; the plan also gives the tile rows and the row bytes.
    mok_config probe = *cfg;
    probe.minibatch_rows = 16;
    probe.ring_bytes = int64_t(1) << 50;
    Plan p;
    mok_status s = make_plan(&probe, shape, &p);
    if (s != MOK_OK) return s;
    const int64_t BM = p.tile.BM;
    const int64_t rows = (2 * units * BM * kTileN + 2 * (int64_t)p.I - 1) / (2 * (int64_t)p.I);
    int64_t mb = (rows + BM - 1) / BM * BM;
    const int64_t macro_rows = ((int64_t)p.k * p.MT + 15) / 16 * 16;
    mb = std::max<int64_t>(16, std::min(mb, macro_rows));
    if (mb > (int64_t(1) << 30)) return MOK_ERROR_INVALID_VALUE;
    mok_config out = *cfg;
    out.minibatch_rows = (int32_t)mb;
    const int64_t two_slots = 2 * mb * (int64_t)p.ring_row_bytes;
    if (out.ring_bytes < two_slots) out.ring_bytes = two_slots;
    s = make_plan(&out, shape, &p);
    if (s != MOK_OK) return s;
    *cfg = out;
    return MOK_OK;
}

mok_status mok_query_sizes(const mok_config *cfg, const mok_shape *shape, size_t *workspace_bytes,
                           size_t *schedule_bytes, size_t *fwd_ctx_bytes) {
    Plan p;
    const mok_status s = make_plan(cfg, shape, &p);
    if (s != MOK_OK) return s;
    if (workspace_bytes) *workspace_bytes = p.w_total;
    if (schedule_bytes) *schedule_bytes = p.s_total;
    if (fwd_ctx_bytes) *fwd_ctx_bytes = p.c_total;
    return MOK_OK;
}

mok_status mok_schedule_layout_query(const mok_config *cfg, const mok_shape *shape, mok_schedule_layout *l) {
    if (!l) return MOK_ERROR_INVALID_VALUE;
    Plan p;
    const mok_status s = make_plan(cfg, shape, &p);
    if (s != MOK_OK) return s;
    l->R = p.R;
    l->NM = p.NM;
    l->G = p.G;
    l->cap = p.cap;
    l->status = p.s_status;
    l->n_seg = p.s_nseg;
    l->counts = p.s_counts;
    l->offsets = p.s_offsets;
    l->mcounts = p.s_mcounts;
    l->moffsets = p.s_moffsets;
    l->perm = p.s_perm;
    l->inv = p.s_inv;
    l->canon = p.s_canon;
    l->mb_start = p.s_mbstart;
    l->segments = p.s_segments;
    l->total_bytes = p.s_total;
    return MOK_OK;
}

mok_status mok_build_schedule(const mok_config *cfg, const mok_shape *shape, const int32_t *topk_ids,
                              void *schedule, size_t schedule_bytes, void *stream) {
    Plan p;
    mok_status s = make_plan(cfg, shape, &p);
    if (s != MOK_OK) return s;
    if (!dev_ok(schedule) || (p.R > 0 && !dev_ok(topk_ids))) return MOK_ERROR_INVALID_VALUE;
    if (schedule_bytes < p.s_total) return MOK_ERROR_BUFFER_TOO_SMALL;
    (void)hipGetLastError();   // drop an earlier, unrelated error of this thread
    return launch_build_schedule(p, topk_ids, schedule, static_cast<hipStream_t>(stream));
}

static mok_status check_weights(const Plan &p, const mok_weights *w) {
    if (!w) return MOK_ERROR_INVALID_VALUE;
    if (p.precision == MOK_BF16) {
        if (!dev_ok(w->w_gate) || !dev_ok(w->w_up) || !dev_ok(w->w_down)) return MOK_ERROR_INVALID_VALUE;
    } else {
        if (!dev_ok(w->gate_elems) || !dev_ok(w->gate_scales) || !dev_ok(w->up_elems) || !dev_ok(w->up_scales) ||
            !dev_ok(w->down_elems) || !dev_ok(w->down_scales))
            return MOK_ERROR_INVALID_VALUE;
    }
    return MOK_OK;
}

mok_status mok_forward(const mok_config *cfg, const mok_shape *shape, const void *schedule, size_t schedule_bytes,
                       void *workspace, size_t workspace_bytes, const void *x, const float *topk_w,
                       const mok_weights *w, void *out, void *fwd_ctx, size_t fwd_ctx_bytes, void *stream) {
    Plan p;
    mok_status s = make_plan(cfg, shape, &p);
    if (s != MOK_OK) return s;
    if ((s = check_weights(p, w)) != MOK_OK && !(p.debug & MOK_DEBUG_IDENTITY_EXPERT)) return s;
    if (!dev_ok(schedule) || !dev_ok(workspace) || !dev_ok(fwd_ctx)) return MOK_ERROR_INVALID_VALUE;
    if (p.R > 0 && (!dev_ok(x) || !dev_ok(topk_w) || !dev_ok(out))) return MOK_ERROR_INVALID_VALUE;
    if (schedule_bytes < p.s_total || workspace_bytes < p.w_total || fwd_ctx_bytes < p.c_total)
        return MOK_ERROR_BUFFER_TOO_SMALL;
    (void)hipGetLastError();
    if ((s = launch_schedule_check(p, schedule, static_cast<hipStream_t>(stream))) != MOK_OK) return s;
    return launch_forward(p, schedule, workspace, static_cast<const uint16_t *>(x), topk_w, *w,
                          static_cast<uint16_t *>(out), fwd_ctx, static_cast<hipStream_t>(stream));
}

mok_status mok_backward(const mok_config *cfg, const mok_shape *shape, const void *schedule, size_t schedule_bytes,
                        void *workspace, size_t workspace_bytes, const void *x, const float *topk_w,
                        const mok_weights *w,
                        const void *fwd_ctx, size_t fwd_ctx_bytes, const void *dy, void *dx, void *dw_gate,
                        void *dw_up, void *dw_down, float *dtopk_w, void *stream) {
    Plan p;
    mok_status s = make_plan(cfg, shape, &p);
    if (s != MOK_OK) return s;
    if (p.debug & MOK_DEBUG_IDENTITY_EXPERT) return MOK_ERROR_UNSUPPORTED;
    if ((s = check_weights(p, w)) != MOK_OK) return s;
    if (!dev_ok(schedule) || !dev_ok(workspace) || !dev_ok(fwd_ctx)) return MOK_ERROR_INVALID_VALUE;
    if (!dev_ok(dw_gate) || !dev_ok(dw_up) || !dev_ok(dw_down)) return MOK_ERROR_INVALID_VALUE;
    if (p.R > 0 && (!dev_ok(x) || !dev_ok(topk_w) || !dev_ok(dy) || !dev_ok(dx) || !dev_ok(dtopk_w)))
        return MOK_ERROR_INVALID_VALUE;
    if (schedule_bytes < p.s_total || workspace_bytes < p.w_total || fwd_ctx_bytes < p.c_total)
        return MOK_ERROR_BUFFER_TOO_SMALL;
    (void)hipGetLastError();
    if ((s = launch_schedule_check(p, schedule, static_cast<hipStream_t>(stream))) != MOK_OK) return s;
    return launch_backward(p, schedule, workspace, static_cast<const uint16_t *>(x), topk_w, *w, fwd_ctx,
                           static_cast<const uint16_t *>(dy), static_cast<uint16_t *>(dx),
                           static_cast<uint16_t *>(dw_gate), static_cast<uint16_t *>(dw_up),
                           static_cast<uint16_t *>(dw_down), dtopk_w, static_cast<hipStream_t>(stream));
}

mok_status mok_mxfp8_quantize(const void *src, int64_t batch, int64_t rows, int64_t K, int32_t src_is_k_by_rows,
                              uint8_t *elems, uint8_t *scales, void *stream) {
    if (batch < 0 || rows < 0 || K < 0 || K % 32) return MOK_ERROR_INVALID_VALUE;
    if (src_is_k_by_rows != 0 && src_is_k_by_rows != 1) return MOK_ERROR_INVALID_VALUE;
    if (batch * rows * K == 0) return MOK_OK;
    if (!dev_ok(src) || !dev_ok(elems) || !scales) return MOK_ERROR_INVALID_VALUE;
    (void)hipGetLastError();
    return launch_mxfp8_quantize(static_cast<const uint16_t *>(src), batch, rows, K, src_is_k_by_rows == 1, elems,
                                 scales, static_cast<hipStream_t>(stream));
}

mok_status mok_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *topk_ids, float *topk_w,
                     void *stream) {
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64) return MOK_ERROR_INVALID_VALUE;
    if (T == 0) return MOK_OK;
    if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w)) return MOK_ERROR_INVALID_VALUE;
    (void)hipGetLastError();
    return launch_route(logits, T, E, k, topk_ids, topk_w, static_cast<hipStream_t>(stream));
}

mok_status mok_route_backward(const int32_t *topk_ids, const float *topk_w, const float *dtopk_w, int64_t T,
                              int32_t E, int32_t k, float *dlogits, void *stream) {
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 64) return MOK_ERROR_INVALID_VALUE;
    if (T == 0) return MOK_OK;
    if (!aligned4(topk_ids) || !aligned4(topk_w) || !aligned4(dtopk_w) || !aligned4(dlogits))
        return MOK_ERROR_INVALID_VALUE;
    (void)hipGetLastError();
    return launch_route_backward(topk_ids, topk_w, dtopk_w, T, E, k, dlogits, static_cast<hipStream_t>(stream));
}

const char *mok_status_string(mok_status status) {
    switch (status) {
        case MOK_OK: return "MOK_OK";
        case MOK_ERROR_INVALID_VALUE: return "MOK_ERROR_INVALID_VALUE";
        case MOK_ERROR_UNSUPPORTED: return "MOK_ERROR_UNSUPPORTED";
        case MOK_ERROR_BUFFER_TOO_SMALL: return "MOK_ERROR_BUFFER_TOO_SMALL";
        case MOK_ERROR_LAUNCH_FAILED: return "MOK_ERROR_LAUNCH_FAILED";
    }
    return "MOK_ERROR_UNKNOWN";
}

}  // extern "C"
