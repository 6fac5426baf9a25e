// Kernel-argument views of the schedule buffer and the layer buffers,
// built on the host from a Plan and the caller's pointers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace mok {

// One m-tile of a segment GEMM: up to BM routed rows of one expert inside one
// mini-batch, starting at processing position q0 and at position c0 of the
// canonical (expert, routed row) order.
struct MTile {
    int32_t q0, rows, e, g, c0, pad0, pad1, pad2;
};

struct SchedView {
    uint32_t *status;
    int32_t *n_seg;
    uint32_t *fprint;
    int32_t *counts, *offsets, *mcounts, *moffsets, *perm, *inv, *canon, *ctok, *mb_start,
        *segments, *chunk, *bound, *segfirst, *mtfirst;
    MTile *mtiles;
    int32_t R, T, k, E, MB, MT, NM, nb_full, G, cap, BM, nchunks, max_mtiles;
    uint32_t fingerprint;   // the plan's: what sched_init writes and sched_check expects
};

inline SchedView make_sched_view(const Plan &p, void *buf) {
    char *b = static_cast<char *>(buf);
    SchedView v;
    v.status = reinterpret_cast<uint32_t *>(b + p.s_status);
    v.n_seg = reinterpret_cast<int32_t *>(b + p.s_nseg);
    v.fprint = reinterpret_cast<uint32_t *>(b + p.s_fprint);
    auto I32 = [&](size_t off) { return reinterpret_cast<int32_t *>(b + off); };
    v.counts = I32(p.s_counts);
    v.offsets = I32(p.s_offsets);
    v.mcounts = I32(p.s_mcounts);
    v.moffsets = I32(p.s_moffsets);
    v.perm = I32(p.s_perm);
    v.inv = I32(p.s_inv);
    v.canon = I32(p.s_canon);
    v.ctok = I32(p.s_ctok);
    v.mb_start = I32(p.s_mbstart);
    v.segments = I32(p.s_segments);
    v.chunk = I32(p.s_chunk);
    v.bound = I32(p.s_bound);
    v.segfirst = I32(p.s_segfirst);
    v.mtfirst = I32(p.s_mtfirst);
    v.mtiles = reinterpret_cast<MTile *>(b + p.s_mtiles);
    v.R = (int32_t)p.R;
    v.T = (int32_t)p.T;
    v.k = p.k;
    v.E = p.E;
    v.MB = p.MB;
    v.MT = (int32_t)p.MT;
    v.NM = p.NM;
    v.nb_full = p.nb_full;
    v.G = p.G;
    v.cap = (int32_t)p.cap;
    v.BM = p.tile.BM;
    v.nchunks = p.nchunks;
    v.max_mtiles = (int32_t)p.max_mtiles;
    v.fingerprint = p.fingerprint;
    return v;
}

}  // namespace mok
