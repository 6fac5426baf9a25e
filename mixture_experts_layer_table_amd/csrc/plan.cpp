// Host-side plan: validation, sizes and buffer layouts (no HIP calls).
#include "plan.h"

#include <algorithm>
#include <cmath>

#include "tiles.h"

namespace mok {

namespace {

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Carver {
    size_t off = 0;
    size_t take(size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes);
        return o;
    }
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FNV-1a over the sizes that fix the schedule table's layout and meaning
// (a table built under other knobs, another shape or another m-tile height
// would be read at wrong offsets).
uint32_t schedule_fingerprint(const Plan &q) {
    const int64_t v[] = {q.T, q.H, q.I, q.E, q.k, q.MB, q.MT, q.NM, q.G, q.cap, q.tile.BM, q.nchunks,
                         q.max_mtiles, (int64_t)q.s_total};
    uint32_t h = 2166136261u;
    for (int64_t x : v)
        for (int b = 0; b < 8; ++b) {
            h ^= (uint32_t)((uint64_t)x >> (8 * b)) & 0xFFu;
            h *= 16777619u;
        }
    return h == 0 ? 1u : h;   // never 0, the value of a cleared buffer
}

}  // namespace

mok_status make_plan(const mok_config *cfg, const mok_shape *shape, Plan *p) {
    if (!cfg || !shape || !p) return MOK_ERROR_INVALID_VALUE;
    const mok_shape &s = *shape;
    if (s.T < 0 || s.H <= 0 || s.I <= 0 || s.E <= 0 || s.k <= 0) return MOK_ERROR_INVALID_VALUE;
    if (s.H % 64 || s.I % 64) return MOK_ERROR_INVALID_VALUE;
    if (s.k > s.E || s.E > kMaxExperts) return MOK_ERROR_INVALID_VALUE;
    if (s.T * (int64_t)s.k >= (int64_t(1) << 31)) return MOK_ERROR_INVALID_VALUE;
    // Activation tensors are addressed through buffer descriptors with 32-bit
    // byte offsets: x / dy / out / dx [T,H] and h / dh [R,2I] stay below 2 GiB.
    if (s.T * (int64_t)s.H * 2 >= (int64_t(1) << 31)) return MOK_ERROR_INVALID_VALUE;
    if (s.T * (int64_t)s.k * s.I * 4 >= (int64_t(1) << 31)) return MOK_ERROR_INVALID_VALUE;
    // so does one expert's weight gradient [H][I], rows of a partial last tile included
    if ((s.H + 256) * (int64_t)s.I * 2 >= (int64_t(1) << 31)) return MOK_ERROR_INVALID_VALUE;
    if (cfg->minibatch_rows < 16 || cfg->minibatch_rows % 16) return MOK_ERROR_INVALID_VALUE;
    if (cfg->macrobatch_tokens < 0 || cfg->ring_bytes <= 0) return MOK_ERROR_INVALID_VALUE;
    if (!(cfg->capacity_multiplier > 0.0f && cfg->capacity_multiplier <= 4.0f))
        return MOK_ERROR_INVALID_VALUE;
    if (cfg->precision != MOK_BF16 && cfg->precision != MOK_MXFP8 && cfg->precision != MOK_MXFP8_WGRAD)
        return MOK_ERROR_INVALID_VALUE;
    if (cfg->persistent_workgroups < 0 || cfg->persistent_workgroups > 65535) return MOK_ERROR_INVALID_VALUE;
    if (cfg->debug_flags &
        ~(MOK_DEBUG_IDENTITY_EXPERT | MOK_DEBUG_SEPARATE_LAUNCHES | MOK_DEBUG_WHOLE_PASS | MOK_DEBUG_FORCE_STALL))
        return MOK_ERROR_INVALID_VALUE;
    // The whole-pass debug mode is switched off: runs that included it hung
    // twice without a shown cause (the claim/wait protocol itself is modelled
    // and found deadlock-free on the host; the hang was not explained).
    if (cfg->debug_flags & MOK_DEBUG_WHOLE_PASS) return MOK_ERROR_UNSUPPORTED;
    // MXFP8 GEMMs load the scale bytes of four 32-blocks as one aligned dword
    if (cfg->precision != MOK_BF16 && (s.H % 128 || s.I % 128)) return MOK_ERROR_INVALID_VALUE;

    Plan q;
    q.T = s.T;
    q.H = s.H;
    q.I = s.I;
    q.E = s.E;
    q.k = s.k;
    q.R = s.T * s.k;
    q.MB = cfg->minibatch_rows;
    q.precision = cfg->precision == MOK_BF16 ? MOK_BF16 : MOK_MXFP8;
    q.mx_wgrad = cfg->precision == MOK_MXFP8_WGRAD;
    q.debug = cfg->debug_flags;
    q.grid = cfg->persistent_workgroups;
    q.MT = (cfg->macrobatch_tokens == 0 || cfg->macrobatch_tokens >= s.T) ? std::max<int64_t>(s.T, 1)
                                                                            : cfg->macrobatch_tokens;
    q.NM = s.T == 0 ? 0 : (int)ceil_div(s.T, q.MT);
    q.nb_full = (int)ceil_div(q.k * q.MT, q.MB);
    q.G = 0;
    q.W = 0;
    if (q.NM > 0) {
        const int64_t t_last = s.T - (int64_t)(q.NM - 1) * q.MT;
        const int64_t r_full = q.k * q.MT, r_last = q.k * t_last;
        q.G = (q.NM - 1) * q.nb_full + (int)ceil_div(r_last, q.MB);
        q.W = (int64_t)(q.NM - 1) * (q.nb_full + std::min<int64_t>(q.E, r_full) - 1) +
              (ceil_div(r_last, q.MB) + std::min<int64_t>(q.E, r_last) - 1);
    }
    q.cap = (int64_t)std::ceil((double)cfg->capacity_multiplier * (double)q.W);
    q.ring_row_bytes = q.precision == MOK_BF16 ? (size_t)2 * q.H : (size_t)q.H + q.H / 32;
    q.n_slots = cfg->ring_bytes / ((int64_t)q.MB * (int64_t)q.ring_row_bytes);
    if (q.n_slots < 2) return MOK_ERROR_INVALID_VALUE;
    q.tile = choose_tiles(q.H, q.I, q.E, q.k, q.T, q.precision);
    q.max_mtiles = q.R / q.tile.BM + q.cap + 1;
    q.nchunks = (int)ceil_div(q.R, kSchedChunk);
    q.dg_slices = (int)ceil_div(q.I, q.tile.da_wn);
    q.stage_rows = q.k > 1 ? q.k * std::min<int64_t>(q.MT, q.T) : 0;

    Carver c;
    q.s_status = c.take(4);
    q.s_nseg = 4;
    q.s_fprint = 8;
    q.s_counts = c.take(4 * (size_t)q.E);
    q.s_offsets = c.take(4 * (size_t)(q.E + 1));
    q.s_mcounts = c.take(4 * (size_t)q.NM * q.E);
    q.s_moffsets = c.take(4 * (size_t)q.NM * (q.E + 1));
    q.s_perm = c.take(4 * (size_t)q.R);
    q.s_inv = c.take(4 * (size_t)q.R);
    q.s_canon = c.take(4 * (size_t)q.R);
    q.s_ctok = c.take(4 * (size_t)q.R);
    q.s_mbstart = c.take(4 * (size_t)(q.G + 1));
    q.s_segments = c.take(16 * (size_t)q.cap);
    q.s_chunk = c.take(4 * (size_t)q.nchunks * q.E);
    q.s_bound = c.take(4 * (size_t)(q.NM + 1) * q.E);
    q.s_segfirst = c.take(4 * (size_t)(q.G + 1));
    q.s_mtfirst = c.take(4 * (size_t)(q.G + 1));
    q.s_mtiles = c.take(32 * (size_t)q.max_mtiles);
    q.s_total = c.off;

    Carver w;
    q.w_ring = w.take((size_t)q.n_slots * q.MB * q.ring_row_bytes);
    q.w_aring = w.take((size_t)q.n_slots * q.MB * q.I * 2);
    q.w_stage = w.take((size_t)q.stage_rows * q.H * 2);
    q.w_dh = w.take((size_t)q.R * 2 * q.I * 2);
    q.w_dgp = w.take((size_t)q.R * q.dg_slices * 4);
    {   // persistent-kernel counters: the larger of the pair layout and the whole-pass layout
        const int64_t S = std::max<int64_t>(1, std::min<int64_t>(q.n_slots, (int64_t)q.G));
        const int64_t NR = (q.G + S - 1) / S;
        const int64_t pass = 3 * NR * 8 + 2 * (int64_t)q.G + S + q.max_mtiles;
        q.w_sync = w.take(4 * (size_t)std::max<int64_t>(kSyncHeads + q.max_mtiles, pass));
    }
    if (q.precision == MOK_MXFP8) {
        q.w_dhq = w.take((size_t)q.R * 2 * q.I);
        q.w_dhq_scales = w.take((size_t)q.R * 2 * q.I / 32);
    }
    if (q.mx_wgrad) {
        // every non-empty expert adds at most 127 rows of padding
        q.Kp = (q.R + 127 * std::min<int64_t>(q.E, q.R) + 127) / 128 * 128;
        const size_t kp = (size_t)q.Kp;
        q.w_qx = w.take((size_t)q.H * kp);
        q.w_qxs = w.take((size_t)q.H * kp / 32);
        q.w_qdh = w.take((size_t)2 * q.I * kp);
        q.w_qdhs = w.take((size_t)2 * q.I * kp / 32);
        q.w_qga = w.take((size_t)q.I * kp);
        q.w_qgas = w.take((size_t)q.I * kp / 32);
        q.w_qdy = w.take((size_t)q.H * kp);
        q.w_qdys = w.take((size_t)q.H * kp / 32);
        q.w_po = w.take(4 * (size_t)(q.E + 1));
    }
    // With k = 1 every routed row is its own token, and the BF16 weight
    // gradients read the x and dy rows of each expert in canonical order as
    // contiguous rows saved by the gathers, instead of gathering them through
    // the token index (measured 15% faster for both weight-gradient GEMMs at
    // the EP-64 share). With k > 1 the token matrices are k times smaller than
    // the routed rows and the indexed reads hit in cache, so the copies would
    // cost more than they save (measured 0.9 ms slower at the full layer). The
    // MXFP8 weight gradients quantize their own token-axis copies instead.
    // One macro-batch whose mini-batches all fit the ring leaves the dy rows
    // in the ring at their canonical positions (processing order equals
    // canonical order then, and mini-batch g occupies slot g): the dy copy is
    // then the ring itself.
    q.keep_canonical = !q.mx_wgrad && q.k == 1;
    q.dy_in_ring = q.keep_canonical && q.precision == MOK_BF16 && q.NM == 1 && (int64_t)q.G <= q.n_slots;
    q.x_ring_is_copy = q.dy_in_ring;
    if (q.keep_canonical && !q.dy_in_ring) q.w_dyc = w.take((size_t)q.R * q.H * 2);
    q.w_total = w.off;

    Carver x;
    q.c_h = x.take((size_t)q.R * 2 * q.I * 2);
    q.c_ga = x.take((size_t)q.R * q.I * 2);
    if (q.keep_canonical) q.c_xc = x.take((size_t)q.R * q.H * 2);
    q.c_total = x.off;
    q.fingerprint = schedule_fingerprint(q);
    *p = q;
    return MOK_OK;
}

Plan forward_only_workspace(const Plan &p, size_t *bytes) {
    Plan q = p;
    Carver w;
    q.w_ring = w.take((size_t)q.n_slots * q.MB * q.ring_row_bytes);
    q.w_aring = w.take((size_t)q.n_slots * q.MB * q.I * 2);
    q.w_stage = w.take((size_t)q.stage_rows * q.H * 2);
    q.w_sync = w.take(4 * (size_t)(kSyncHeads + q.max_mtiles));
    // backward-only regions: none in this layout (a forward never touches them)
    q.w_dh = q.w_dgp = q.w_dhq = q.w_dhq_scales = q.w_dyc = 0;
    q.w_qx = q.w_qxs = q.w_qdh = q.w_qdhs = q.w_qga = q.w_qgas = q.w_qdy = q.w_qdys = q.w_po = 0;
    q.w_total = w.off;
    *bytes = w.off;
    return q;
}

void minibatch_rows(const Plan &p, int g, int64_t *q0, int64_t *q1) {
    const int m = g / p.nb_full, b = g % p.nb_full;
    const int64_t t0 = (int64_t)m * p.MT;
    const int64_t rm = p.k * (std::min<int64_t>(p.T, t0 + p.MT) - t0);
    const int64_t base = p.k * t0;
    *q0 = base + (int64_t)b * p.MB;
    *q1 = base + std::min<int64_t>(rm, (int64_t)(b + 1) * p.MB);
}

int macro_of_minibatch(const Plan &p, int g) { return g / p.nb_full; }
int first_minibatch(const Plan &p, int m) { return m * p.nb_full; }

}  // namespace mok
