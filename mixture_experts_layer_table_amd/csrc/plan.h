// Host-side plan: every size and byte offset derived from (config, shape).
// Pure C++ with no HIP calls, so size queries and argument validation run
// without a GPU.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/mok.h"
#include "tiles.h"

namespace mok {

constexpr int kSchedChunk = 1024;   // routed rows per block in the schedule kernels
constexpr size_t kAlign = 256;      // alignment of every sub-buffer
constexpr int kSyncHeads = 16;      // claim counters of a persistent kernel: 2 item classes x 8 XCDs

struct Plan {
    // shape
    int64_t T = 0, R = 0;
    int H = 0, I = 0, E = 0, k = 0;
    // knobs
    int MB = 0;
    int64_t MT = 0;          // effective macro-batch tokens (T if 0 or >= T; 1 if T == 0)
    int precision = MOK_BF16;   // MOK_BF16 or MOK_MXFP8 (MOK_MXFP8_WGRAD sets MOK_MXFP8 and mx_wgrad)
    bool mx_wgrad = false;      // weight gradients on the block-scaled MFMA
    uint32_t debug = 0;
    int grid = 0;            // persistent-kernel workgroups (0: one per compute unit)
    // derived
    int NM = 0;              // macro-batches
    int nb_full = 0;         // mini-batches in a full macro-batch
    int G = 0;               // mini-batches
    int64_t W = 0, cap = 0;  // worst-case segments, segment capacity
    int64_t n_slots = 0;     // ring slots (mini-batches the ring holds)
    size_t ring_row_bytes = 0;
    TileChoice tile{};
    int64_t max_mtiles = 0;  // bound on m-tiles over all segments
    int nchunks = 0;         // schedule chunks of kSchedChunk rows
    int dg_slices = 0;       // router-grad partial sums per routed row
    int64_t stage_rows = 0;  // rows of the per-macro-batch combine staging (k > 1)

    // schedule buffer (byte offsets)
    // layout fingerprint: a hash of every size the schedule's layout depends
    // on, written into the table by its builder and checked by its readers
    uint32_t fingerprint = 0;
    size_t s_status = 0, s_nseg = 0, s_fprint = 0, s_counts = 0, s_offsets = 0, s_mcounts = 0,
           s_moffsets = 0, s_perm = 0, s_inv = 0, s_canon = 0, s_ctok = 0, s_mbstart = 0,
           s_segments = 0, s_chunk = 0, s_bound = 0, s_segfirst = 0, s_mtfirst = 0,
           s_mtiles = 0, s_total = 0;
    // workspace (byte offsets)
    size_t w_ring = 0, w_aring = 0, w_stage = 0, w_dh = 0, w_dgp = 0, w_total = 0;
    // persistent-kernel work queues: kSyncHeads claim counters, then one
    // completion counter per m-tile of a ring round
    size_t w_sync = 0;
    // MXFP8 only: dh quantized along I, elements [R][2I] and scales [R][2I/32]
    size_t w_dhq = 0, w_dhq_scales = 0;
    // MXFP8 weight gradients only: operands quantized along the token axis,
    // transposed: [cols][Kp] elements and [cols][Kp/32] scales for x (H cols),
    // dh (2I), g*a (I) and dy (H), expert e's rows at [po[e], po[e+1]) of Kp,
    // po[e+1] - po[e] = its row count rounded up to 128; po [E+1] int32.
    int64_t Kp = 0;
    size_t w_qx = 0, w_qxs = 0, w_qdh = 0, w_qdhs = 0, w_qga = 0, w_qgas = 0, w_qdy = 0, w_qdys = 0, w_po = 0;
    // BF16 weight gradients with k = 1 only: dy rows in canonical (expert, f)
    // order, [R][H] bf16, written by the backward's dy gather (0 when unused,
    // or when the ring already holds them so: dy_in_ring)
    size_t w_dyc = 0;
    bool dy_in_ring = false;
    // the same condition in the forward (BF16, k = 1, one macro-batch, every
    // mini-batch in its own slot): ring row q is canonical row q, so the
    // forward uses fwd_ctx's x copy as its ring and writes each x row once
    bool x_ring_is_copy = false;
    // fwd_ctx (byte offsets): h [R][2I] bf16 in processing order; g * a
    // [R][I] bf16 in canonical order (the down weight gradient's operand,
    // written by the gate/up epilogue so that the backward can start that
    // gradient as soon as its dy rows are in place); with BF16 weight
    // gradients and k = 1 also the x rows in canonical order, [R][H] bf16,
    // written by the forward's gather (c_xc 0 when unused)
    size_t c_h = 0, c_ga = 0, c_xc = 0, c_total = 0;
    bool keep_canonical = false;   // the two canonical copies above exist
};

mok_status make_plan(const mok_config *cfg, const mok_shape *shape, Plan *p);

// The forward pass reads and writes only the ring, the a-ring, the combine
// staging and the persistent queues' counters of the workspace. Returns a copy
// of p whose workspace holds just those, packed from offset 0, and its size.
Plan forward_only_workspace(const Plan &p, size_t *bytes);

// Rows [q0, q1) of mini-batch g: host-computable (depends on sizes only).
void minibatch_rows(const Plan &p, int g, int64_t *q0, int64_t *q1);
// Macro-batch of mini-batch g and the first mini-batch of macro-batch m.
int macro_of_minibatch(const Plan &p, int g);
int first_minibatch(const Plan &p, int m);

}  // namespace mok
