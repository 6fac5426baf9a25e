/*
 * mok.h — C ABI of the MI355X (gfx950) MoE-layer library.
 *
 * One GPU's share of a deterministic mixture-of-experts training layer,
 * forward and backward: top-k ids -> schedule table -> drop-free permute of
 * token rows through a fixed ring buffer in mini-batches -> SwiGLU experts as
 * grouped GEMMs -> weighted combine back to token order; the backward pass
 * mirrors these steps and computes the router-weight gradient inside the
 * SwiGLU backward.
 *
 * Sources: "Mixture-of-Kittens (MoK)" project summary (Functional API; Key
 * concepts table), "Cursor Open-Sources Mixture-of-Kittens (MoK)" digest
 * (English abstract) and "Mixture-of-Kittens(MoK)란?" explainer (sections 1,
 * 4 ①-③). Each call below names the passage that defines it.
 *
 * Conventions for every call:
 *  - Every buffer is allocated and freed by the caller. The library never
 *    allocates, frees, synchronises or copies device memory back to the host.
 *  - Device pointers must be 16-byte aligned. Work is enqueued on `stream`
 *    (a hipStream_t; NULL = the legacy default stream) and the call returns
 *    without waiting for it.
 *  - Host-checkable problems (bad sizes, misaligned or NULL pointers, a buffer
 *    smaller than mok_query_sizes reports, fewer than 2 ring slots) return a
 *    non-zero mok_status and enqueue nothing.
 *  - Data-dependent problems set bits in the device status word (uint32 at
 *    byte 0 of the schedule buffer): MOK_SCHEDULE_OVERFLOW, MOK_BAD_EXPERT_ID.
 *    mok_forward / mok_backward then do no work and their outputs are
 *    undefined. The caller reads the word whenever it synchronises; no
 *    routed row is ever dropped silently.
 *  - Calls are re-entrant; concurrent calls need distinct workspaces.
 *  - bf16 tensors are raw 16-bit patterns; all tensors are dense row-major.
 */
#ifndef MOK_H
#define MOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mok_status {
    MOK_OK = 0,
    MOK_ERROR_INVALID_VALUE = 1,
    MOK_ERROR_UNSUPPORTED = 2,
    MOK_ERROR_BUFFER_TOO_SMALL = 3,
    MOK_ERROR_LAUNCH_FAILED = 4
} mok_status;

/* precision modes ("Mixture-of-Kittens (MoK)" project summary, Overview) */
#define MOK_BF16 0
#define MOK_MXFP8 1
/* MXFP8 with the weight gradients on the block-scaled MFMA as well: their
   operands (x, dh, g*a, dy) are quantized along the token axis, 32 rows of one
   expert per E8M0 scale in canonical order, each expert's rows zero-padded to
   a multiple of 128 ("Mixture-of-Kittens (MoK)" project summary, Key-concepts
   table: MXFP8 mode; the pages leave the weight-gradient precision open). */
#define MOK_MXFP8_WGRAD 2

/* device status word bits */
#define MOK_SCHEDULE_OVERFLOW 1u
#define MOK_BAD_EXPERT_ID 2u
/* a persistent kernel's work queue made no progress within its spin limit
   (never expected; outputs are then undefined and the kernel has exited) */
#define MOK_SCHEDULER_STALLED 4u
/* mok_forward / mok_backward got a schedule table built for another layout:
   a different shape, minibatch_rows, macrobatch_tokens, capacity_multiplier
   or m-tile height (set by the precision). The builder writes a fingerprint of
   these into the table and each reader checks it before reading anything
   else; no work is done after a mismatch. */
#define MOK_SCHEDULE_MISMATCH 8u

/* debug_flags: replace every expert by the identity on its rows (forward only;
   out_t = sum_j g_tj * x_t). Used to test permute followed by unpermute. */
#define MOK_DEBUG_IDENTITY_EXPERT 1u
/* debug_flags: run each grouped GEMM of a ring round as its own launch
   instead of the persistent producer/consumer kernel (same results, bit for
   bit; used to cross-check the scheduler and to time GEMMs one by one).
   BF16 only: MXFP8 rounds always launch their GEMMs one by one. */
#define MOK_DEBUG_SEPARATE_LAUNCHES 2u
/* debug_flags (k == 1 only): run each whole forward / dgrad pass as one
   persistent launch in which gathers and both GEMMs of every ring round
   follow the in-kernel ring protocol (slot full / release counters) instead
   of stream order between rounds. Currently switched off: every call that
   sets it returns MOK_ERROR_UNSUPPORTED and enqueues nothing, because runs
   that included this mode hung twice without a shown cause. */
#define MOK_DEBUG_WHOLE_PASS 4u
/* debug_flags: every wait inside the persistent kernels gives up at once, as
   if its poll budget were spent. The call then ends with
   MOK_SCHEDULER_STALLED in the status word, leaving the outputs that depend
   on the abandoned waits unwritten. Tests the stall exit path; never for
   production use. */
#define MOK_DEBUG_FORCE_STALL 8u

/*
 * Layer knobs ("Mixture-of-Kittens (MoK)" project summary, Key-concepts table:
 * mini-batch granularity, macro-batch size, schedule capacity multiplier; the
 * communication-SM knob has no meaning without peers and is not present).
 * No knob changes any output bit.
 *   minibatch_rows      rows per mini-batch, a multiple of 16 (default 512)
 *   macrobatch_tokens   tokens per macro-batch; 0 = one macro-batch
 *   ring_bytes          size of the ring token buffer; must hold >= 2 mini-batches
 *   capacity_multiplier schedule capacity relative to the worst case, in (0, 4]
 *   precision           MOK_BF16, MOK_MXFP8 or MOK_MXFP8_WGRAD
 *   debug_flags         0 in production
 *   persistent_workgroups  workgroups of each persistent-kernel launch, in
 *                       [0, 65535]; 0 (the default) = one per compute unit.
 *                       Fewer leave units idle, more wait behind the resident
 *                       ones; the work queues give every value the same bits
 *                       (a grid-size sweep is part of the race tests).
 */
typedef struct mok_config {
    int32_t minibatch_rows;
    int32_t precision;
    int64_t macrobatch_tokens;
    int64_t ring_bytes;
    float capacity_multiplier;
    uint32_t debug_flags;
    int32_t persistent_workgroups;
} mok_config;

/*
 * Layer shape: T rows handed to the layer (tokens; for an expert-parallel
 * share, the received routed rows with k = 1), hidden size H, expert
 * intermediate size I, E local experts, k routed rows per token.
 * H and I are multiples of 64; 1 <= k <= E <= 4096; T >= 0;
 * T*k < 2^31. Activations are addressed with 32-bit byte offsets, so also
 * T*H*2 < 2^31 (x, dy, out, dx), T*k*I*4 < 2^31 (h, dh) and (H+256)*I*2 <
 * 2^31 (one expert's weight gradient). A shape outside these bounds makes
 * every call that takes it return MOK_ERROR_INVALID_VALUE.
 */
typedef struct mok_shape {
    int64_t T;
    int32_t H, I, E, k;
} mok_shape;

/*
 * Expert weights.
 * BF16 mode: w_gate, w_up [E,H,I] and w_down [E,I,H], bf16.
 * MXFP8 mode (weights pre-quantized by mok_mxfp8_quantize; "Mixture-of-Kittens
 * (MoK)" project summary, Key-concepts table), elements E4M3 bytes and scales
 * E8M0 bytes, one scale per 32 contiguous elements along the contraction axis:
 *   for mok_forward : gate/up elems [E,I,H] scales [E,I,H/32]   (W^T, along H)
 *                     down    elems [E,H,I] scales [E,H,I/32]   (W_down^T, along I)
 *   for mok_backward: gate/up elems [E,H,I] scales [E,H,I/32]   (along I)
 *                     down    elems [E,I,H] scales [E,I,H/32]   (along H)
 * In MXFP8 mode the bf16 pointers are ignored: the weight gradients use
 * activations only.
 */
typedef struct mok_weights {
    const void *w_gate, *w_up, *w_down;
    const uint8_t *gate_elems, *gate_scales;
    const uint8_t *up_elems, *up_scales;
    const uint8_t *down_elems, *down_scales;
} mok_weights;

/*
 * Byte offsets of the schedule table's fields inside the schedule buffer, and
 * its sizes, for inspection by tests and tools. Fields are int32 arrays:
 *   counts[E]            rows per expert (sum = T*k: nothing is dropped)
 *   offsets[E+1]         exclusive scan of counts
 *   mcounts[NM*E]        rows per (macro-batch, expert)
 *   moffsets[NM*(E+1)]   first processing position of each (macro-batch, expert)
 *   perm[R]              processing position q -> routed row f = t*k + j
 *   inv[R]               routed row f -> processing position q
 *   canon[R]             position in (expert, f) order -> processing position
 *   mb_start[G+1]        first processing position of each mini-batch
 *   segments[cap*4]      (mini-batch g, expert e, first position q0, rows) for
 *                        each non-empty (mini-batch, expert) intersection
 * plus uint32 status (byte 0) and int32 n_seg (byte 4).
 */
typedef struct mok_schedule_layout {
    int64_t R, NM, G, cap;
    size_t status, n_seg, counts, offsets, mcounts, moffsets, perm, inv, canon,
           mb_start, segments;
    size_t total_bytes;
} mok_schedule_layout;

/* Fill *cfg with the defaults: 512-row mini-batches, one macro-batch, a
   256 MiB ring, capacity multiplier 1, BF16, no debug flags, one persistent
   workgroup per compute unit. */
mok_status mok_config_default(mok_config *cfg);

/*
 * Host-only: size the mini-batch by the two-wave rule ("Mixture-of-Kittens(MoK)
 * 란?" explainer, section 4 ②: the overlap unit is the smallest that still
 * gives every expert-grouped GEMM at least two full waves of compute units;
 * its worked example is 2,368 tokens for a Kimi 2.5-shaped layer).
 * The gate/up GEMM of r rows has r*2I/(BM*256) output tiles counted
 * fractionally, BM being the layer's m-tile rows (256, or 128 for BF16 layers
 * of many small groups) and 256 the n-tile width; two waves over n_cu compute
 * units need r >= 2*n_cu*BM*256/(2I). minibatch_rows becomes that minimum
 * rounded up to whole m-tiles (m-tiles are cut at mini-batch boundaries),
 * capped at one macro-batch's routed rows rounded up to 16; ring_bytes is
 * raised to two slots of that size if it holds fewer and otherwise kept (it is
 * the caller's memory budget). Every other field is kept.
 *   cfg    in/out: the caller's knobs; written only on MOK_OK
 *   shape  the layer shape, validated as by mok_query_sizes
 *   n_cu   compute units to fill; <= 0 means 256 (one MI355X)
 * Returns MOK_ERROR_INVALID_VALUE for a null pointer or a shape or knob
 * mok_query_sizes would reject. Results never depend on the knobs it sets.
 */
mok_status mok_config_autosize(mok_config *cfg, const mok_shape *shape, int32_t n_cu);

/*
 * Host-only size query (the pages' get_workspace sizing, "Mixture-of-Kittens
 * (MoK)" project summary, Functional API; the workspace is made once and
 * reused, Key-concepts table). Writes the byte sizes of the workspace
 * (ring + scratch, reusable across calls), the schedule buffer (one per
 * routing) and fwd_ctx (forward saves for backward). Any output pointer may
 * be NULL. Enqueues nothing; needs no GPU.
 */
mok_status mok_query_sizes(const mok_config *cfg, const mok_shape *shape,
                           size_t *workspace_bytes, size_t *schedule_bytes,
                           size_t *fwd_ctx_bytes);

/* Host-only: the schedule buffer's field offsets for cfg and shape. */
mok_status mok_schedule_layout_query(const mok_config *cfg, const mok_shape *shape,
                                     mok_schedule_layout *layout);

/*
 * Build the schedule table on the device from top-k expert ids
 * ("Mixture-of-Kittens (MoK)" project summary, Functional API: build_schedule;
 * "Mixture-of-Kittens(MoK)란?" explainer, section 4 ①: one table drives both
 * passes; section 4 ③: drop-free, no CPU-GPU synchronisation).
 *   topk_ids  device int32 [T,k], each in [0,E) (else MOK_BAD_EXPERT_ID)
 *   schedule  device buffer of schedule_bytes >= mok_query_sizes' value
 * Processing order sorts routed rows by (macro-batch, expert, row); the table
 * is a pure function of (topk_ids, shape, config).
 */
mok_status mok_build_schedule(const mok_config *cfg, const mok_shape *shape,
                              const int32_t *topk_ids, void *schedule,
                              size_t schedule_bytes, void *stream);

/*
 * Forward pass ("Mixture-of-Kittens (MoK)" project summary, Functional API:
 * forward -> (out, fwd_ctx); "Mixture-of-Kittens(MoK)란?" explainer, section
 * 4 ③: ring token buffer consumed in mini-batches).
 *   schedule the table mok_build_schedule wrote (schedule_bytes long) for
 *            the same shape, minibatch_rows, macrobatch_tokens,
 *            capacity_multiplier and precision; checked against a layout
 *            fingerprint before use (MOK_SCHEDULE_MISMATCH)
 *   x        device bf16 [T,H]
 *   topk_w   device fp32 [T,k] gate weights
 *   w        expert weights (see mok_weights)
 *   out      device bf16 [T,H]: out_t = sum_j topk_w[t,j] * SwiGLU_e(x_t),
 *            accumulated in fp32 in order j = 0..k-1
 *   fwd_ctx  device buffer (fwd_ctx_bytes), written; read by mok_backward
 */
mok_status mok_forward(const mok_config *cfg, const mok_shape *shape,
                       const void *schedule, size_t schedule_bytes,
                       void *workspace, size_t workspace_bytes,
                       const void *x, const float *topk_w, const mok_weights *w,
                       void *out, void *fwd_ctx, size_t fwd_ctx_bytes, void *stream);

/*
 * Backward pass for upstream gradient dy of out ("Mixture-of-Kittens (MoK)"
 * project summary, Functional API: backward -> grads; "Mixture-of-Kittens(MoK)
 * 란?" explainer, section 4 ③: the ring is walked in reverse; "Cursor
 * Open-Sources Mixture-of-Kittens (MoK)" digest, English abstract: the
 * router-weight gradient is fused into the SwiGLU backward).
 *   x, topk_w, w, schedule, fwd_ctx   as given to mok_forward (the schedule
 *            is checked as there)
 *   dy       device bf16 [T,H]
 *   dx       device bf16 [T,H]
 *   dw_gate, dw_up [E,H,I] and dw_down [E,I,H], device bf16, overwritten
 *            (experts that received no rows get zeros)
 *   dtopk_w  device fp32 [T,k]: d loss / d topk_w[t,j] = <dy_t, y_{t,j}>
 */
mok_status mok_backward(const mok_config *cfg, const mok_shape *shape,
                        const void *schedule, size_t schedule_bytes,
                        void *workspace, size_t workspace_bytes,
                        const void *x, const float *topk_w, const mok_weights *w,
                        const void *fwd_ctx, size_t fwd_ctx_bytes, const void *dy,
                        void *dx, void *dw_gate, void *dw_up, void *dw_down,
                        float *dtopk_w, void *stream);

/*
 * mok_forward without a workspace argument: the forward pass's scratch (ring,
 * a-ring, combine staging, work-queue counters) lives in a static device array
 * of MOK_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends. For callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device looks up that device's copy
 * of the array. Arguments and results are mok_forward's, bit for bit.
 * A layer whose forward needs more scratch than the array holds (about
 * ring_bytes + ring_bytes * I / H + the k > 1 combine staging) returns
 * MOK_ERROR_BUFFER_TOO_SMALL, with the sizes in mok_last_error(); a smaller
 * ring_bytes knob changes no output bit. Every call on one GPU shares that
 * GPU's array and leaves its contents behind: calls that overlap on one GPU
 * (concurrent streams or threads) race and must be serialised by the caller.
 */
#define MOK_NOALLOC_SCRATCH_BYTES (64u << 20)
mok_status mok_forward_noalloc(const mok_config *cfg, const mok_shape *shape,
                               const void *schedule, size_t schedule_bytes,
                               const void *x, const float *topk_w, const mok_weights *w,
                               void *out, void *fwd_ctx, size_t fwd_ctx_bytes, void *stream);

/*
 * MXFP8 quantization ("Mixture-of-Kittens (MoK)" project summary, Key-concepts
 * table: weights are pre-quantized before the kernel; block format: OCP MX
 * v1.0 MXFP8). For each run of 32 contiguous values along K:
 *   scale byte = clamp(floor(log2 amax) - 8, -127, 127) + 127  (127 if amax = 0)
 *   element    = E4M3FN(v * 2^-(scale-127)), nearest-even, saturating to +-448
 *   src            device bf16; [batch, rows, K] if src_is_k_by_rows == 0,
 *                  [batch, K, rows] if 1 (quantizes the transpose)
 *   elems          device uint8 [batch, rows, K]
 *   scales         device uint8 [batch, rows, K/32]
 * K must be a multiple of 32. NaN/Inf inputs are unsupported.
 */
mok_status mok_mxfp8_quantize(const void *src, int64_t batch, int64_t rows, int64_t K,
                              int32_t src_is_k_by_rows, uint8_t *elems, uint8_t *scales,
                              void *stream);

/*
 * Router front-end: the step before schedule building, which takes the top-k
 * expert choice as input ("Mixture-of-Kittens (MoK)" project summary,
 * Functional API; "Mixture-of-Kittens(MoK)란?" explainer, section 1: each
 * token activates a few experts). The pages leave the router's formula open;
 * this is softmax over all E experts, the k largest logits, and weights
 * renormalised over the chosen k:
 *   topk_ids[t, j]  the j-th largest logit of row t (the lower expert index
 *                   first among equal logits)
 *   topk_w[t, j]    exp(l_j - m) / sum_i exp(l_i - m) over the chosen i,
 *                   m = the row's largest logit (fp32)
 *   logits          device fp32 [T, E], row-major, finite
 *   topk_ids        device int32 [T, k];  topk_w  device fp32 [T, k]
 * 1 <= k <= min(E, 64), E <= 1024; T == 0 is a no-op. Bitwise deterministic.
 */
mok_status mok_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *topk_ids,
                     float *topk_w, void *stream);

/*
 * Logit gradient of mok_route (the choice is piecewise constant):
 *   dlogits[t, e] = w_e * (dtopk_w_e - sum_j w_j * dtopk_w_j)  for chosen e,
 *                   0 for every other expert
 * topk_ids and topk_w as mok_route returned them, dtopk_w device fp32 [T, k]
 * (for instance mok_backward's dtopk_w); dlogits device fp32 [T, E], every
 * entry written. Same limits as mok_route.
 */
mok_status mok_route_backward(const int32_t *topk_ids, const float *topk_w, const float *dtopk_w,
                              int64_t T, int32_t E, int32_t k, float *dlogits, void *stream);

/*
 * Measurement aid, not part of the layer: per-kernel durations for tools such
 * as benchmarks. While enabled, every kernel launch of the library is
 * bracketed by two HIP events recorded on the launch's own stream (the
 * schedule builder's launches count as one "schedule" entry).
 * mok_kernel_timing_enable(1) discards earlier records and starts recording;
 * mok_kernel_timing_enable(0) discards records and stops. mok_kernel_timing_read
 * waits for the recorded events, writes up to `capacity` per-kernel sums in
 * first-launch order, sets *count to the number of distinct kernels, and
 * discards the records. Off by default; not meant for production loops.
 */
typedef struct mok_kernel_stat {
    char name[32];
    int64_t launches;
    double total_ms;
    double max_ms;
} mok_kernel_stat;

mok_status mok_kernel_timing_enable(int32_t enable);
mok_status mok_kernel_timing_read(mok_kernel_stat *stats, int32_t capacity, int32_t *count);

/*
 * Measurement aid, not part of the layer: a per-item trace of the GEMM
 * kernels, to see how the tiles of a pass overlap and where a compute unit's
 * time goes ("Mixture-of-Kittens(MoK)란?" explainer, section 4 ②: the overlap
 * granularity is checked against its estimate). One record per tile of the
 * persistent pair kernels (forward gate/up + down, backward dA + dX) and of
 * the weight-gradient kernels. Times are the GPU's constant 100 MHz clock
 * (s_memrealtime). While tracing is off a kernel pays one scalar branch per
 * tile.
 */
typedef struct mok_item_record {
    uint64_t t_claim;    /* the workgroup began to claim the item (other kernels: the tile started) */
    uint64_t t_start;    /* the item was claimed and its inputs were ready */
    uint64_t t_kloop;    /* its K loop ended (the epilogue begins) */
    uint64_t t_end;      /* its outputs were stored (and, in a pair kernel, published) */
    uint32_t launch;     /* launches since tracing was enabled, in issue order */
    uint8_t kernel;      /* MOK_TRACE_* */
    uint8_t item_class;  /* pair kernels: 1 producer tile, 2 consumer tile; otherwise 0 */
    uint16_t xcd;        /* workgroup index mod 8, its XCD */
    uint32_t item;       /* pair kernels: index in its class's queue; otherwise the workgroup's tile */
    uint32_t workgroup;  /* workgroup index */
} mok_item_record;
#define MOK_TRACE_FWD_GEMMS 0
#define MOK_TRACE_BWD_GEMMS 1
#define MOK_TRACE_WGRAD_GATE_UP 2
#define MOK_TRACE_WGRAD_DOWN 3
#define MOK_TRACE_OTHER 4
#define MOK_ITEM_TRACE_CAPACITY 65536
/* enable(1): discard earlier records and start recording into a device
   buffer of MOK_ITEM_TRACE_CAPACITY records inside the library (later ones are
   dropped); enable(0): stop. read: wait for the device, copy up to `capacity`
   records in completion order, set *count to the number recorded (it may
   exceed MOK_ITEM_TRACE_CAPACITY when records were dropped). Single device,
   not for production loops. */
mok_status mok_item_trace_enable(int32_t enable);
mok_status mok_item_trace_read(mok_item_record *records, int32_t capacity, int32_t *count);

/* Text of the calling thread's last HIP error reported as
   MOK_ERROR_LAUNCH_FAILED ("" if none); valid until the thread's next call. */
const char *mok_last_error(void);

/* Static string naming a status code. */
const char *mok_status_string(mok_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOK_H */
