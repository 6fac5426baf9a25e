// Pieces shared by the BF16 and MXFP8 layer kernels: the m-tile decode of
// the segment GEMMs, the combine-side epilogue store, and the host-side ring
// rounds and grid bounds.
#pragma once
#include <algorithm>
#include <vector>

#include "gemm.h"
#include "kernels.h"
#include "timing.h"
#include "views.h"

namespace mok {
namespace {

// ----------------------------------------------------------------------------- tile decode

struct SegTile {
    MTile mt;
    int nt;       // n-tile index
    int slot;     // ring slot of the tile's mini-batch
    int rowoff;   // first row of the tile inside that mini-batch
};

constexpr int kXcds = 8;       // MI355X: 8 accelerator dies, each with its own L2
constexpr int kGroupM = 4;     // m-tiles per group of the tile order

// Tile of a segment GEMM for this workgroup. The 1-D grid (a multiple of 8
// workgroups, at least the number of tiles) is dispatched round-robin over the
// XCDs; with `per` = ceil(tiles / 8), workgroup b is mapped to tile
// t = (b % 8) * per + b / 8 so that each XCD walks a contiguous range of
// tiles, ordered in groups of kGroupM m-tiles x all n-tiles: the tiles an XCD
// runs together share few operand slices in its L2.
__device__ __forceinline__ bool decode_seg_tile(const SchedView &v, int g0, int g1, int64_t n_slots, int n_tiles,
                                                SegTile &t) {
    if (*v.status) return false;
    const int lo = v.mtfirst[g0], mtc = v.mtfirst[g1] - lo;
    const int total = mtc * n_tiles;                      // tiles that exist (device-side count)
    const int per = (total + kXcds - 1) / kXcds, b = (int)blockIdx.x;
    if (b / kXcds >= per) return false;                   // the grid is a host-side upper bound
    const int id = (b % kXcds) * per + b / kXcds;
    if (id >= total) return false;
    const int gsize = kGroupM * n_tiles, grp = id / gsize, first = grp * kGroupM;
    const int gm = min(kGroupM, mtc - first), r = id % gsize;
    t.mt = v.mtiles[lo + first + r % gm];
    t.nt = r / gm;
    t.slot = (int)(t.mt.g % n_slots);
    t.rowoff = t.mt.q0 - v.mb_start[t.mt.g];
    return true;
}

__device__ __forceinline__ void store4_bf16(uint16_t *p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

__device__ __forceinline__ float bf16r(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// Rows of y (forward down GEMM) or of dx (backward dX GEMM) leave the GEMM
// towards token order. k == 1: straight to the token's row, the forward one
// scaled by its gate weight after rounding y to bf16 (the weighted combine);
// k > 1: into the macro-batch's staging rows, combined later in j order.
template <class C>
__device__ __forceinline__ void store_token_rows(const f32x16_t (&acc)[C::FM][C::FN], const SegTile &t, int n0,
                                                 int wm, int wn, const SchedView &v, int H, int k, int MT,
                                                 int nb_full, const float *topk_w, bool weighted, uint16_t *dst_k1,
                                                 uint16_t *stage) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        const int m = wm * C::WM + fm * 32 + (lane & 31);
        if (m >= t.mt.rows) continue;
        const int q = t.mt.q0 + m;
        uint16_t *dst;
        float gw = 1.0f;
        if (k == 1) {
            const int tok = v.perm[q];
            if (weighted) gw = topk_w[tok];
            dst = dst_k1 + (int64_t)tok * H;
        } else {
            const int64_t base = (int64_t)k * ((t.mt.g / nb_full) * (int64_t)MT);
            dst = stage + (q - base) * H;
        }
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int n = n0 + wn * C::WN + fn * 32 + g4 * 8 + (lane >> 5) * 4;
                if (n >= H) continue;
                float y[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    y[j] = acc[fm][fn][g4 * 4 + j];
                    if (weighted && k == 1) y[j] = gw * bf16r(y[j]);   // y rows are bf16
                }
                store4_bf16(dst + n, y[0], y[1], y[2], y[3]);
            }
    }
}

constexpr int kRowsPerBlock = 4;   // one 64-lane wave per row

// Dispatch copy of one row (bf16 ring): one wave moves the row of processing
// position q = mb_start[g] + r from token order into ring slot g % n_slots.
struct GatherBf16 {
    SchedView v;
    int64_t n_slots;
    int MB, H, k;
    const uint16_t *src;
    uint16_t *ring;

    // 8 loads in flight per lane before the stores: a wave moving rows one
    // after the other is otherwise bound by one memory round trip per 1 KiB.
    __device__ __forceinline__ void row(int g, int r) const {
        const int tok = v.perm[v.mb_start[g] + r] / k;
        const uint4 *s = reinterpret_cast<const uint4 *>(src + (int64_t)tok * H);
        uint4 *d = reinterpret_cast<uint4 *>(ring + ((g % n_slots) * MB + r) * (int64_t)H);
        const int n = H / 8, lane = threadIdx.x & 63;
        for (int c0 = 0; c0 < n; c0 += 64 * 8) {
            uint4 t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = c0 + i * 64 + lane;
                t[i] = c < n ? s[c] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = c0 + i * 64 + lane;
                if (c < n) d[c] = t[i];
            }
        }
    }

    // Rows [r0, r0 + nrows) of mini-batch g by the whole workgroup (nt threads):
    // one flat pass over (row, 16-byte chunk) with 16 loads in flight per
    // thread. tok: the rows' token indices, already in LDS.
    template <int NT>
    __device__ __forceinline__ void rows(int g, int r0, int nrows, const int *tok) const {
        const int n = H / 8, total = nrows * n;
        uint4 *dslot = reinterpret_cast<uint4 *>(ring + ((g % n_slots) * MB + r0) * (int64_t)H);
        for (int e0 = 0; e0 < total; e0 += NT * 16) {
            uint4 t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = e0 + i * NT + (int)threadIdx.x;
                t[i] = e < total ? reinterpret_cast<const uint4 *>(src + (int64_t)tok[e / n] * H)[e % n]
                                 : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = e0 + i * NT + (int)threadIdx.x;
                if (e < total) dslot[e] = t[i];   // slot rows are contiguous: element e at row e / n, chunk e % n
            }
        }
    }
};

struct Round {
    int g0, g1;
};

// Ring rounds: consecutive mini-batches, at most n_slots per round (distinct
// slots), not crossing a macro-batch boundary when the combine is staged (k > 1).
std::vector<Round> make_rounds(const Plan &p, bool reverse) {
    std::vector<Round> out;
    const int S = (int)std::min<int64_t>(p.n_slots, (int64_t)p.G);
    auto add_span = [&](int a, int b) {
        if (!reverse)
            for (int g = a; g < b; g += S) out.push_back({g, std::min(b, g + S)});
        else
            for (int g = b; g > a; g -= S) out.push_back({std::max(a, g - S), g});
    };
    if (p.k == 1) {
        add_span(0, p.G);
    } else if (!reverse) {
        for (int m = 0; m < p.NM; ++m) add_span(first_minibatch(p, m), std::min(p.G, first_minibatch(p, m + 1)));
    } else {
        for (int m = p.NM - 1; m >= 0; --m) add_span(first_minibatch(p, m), std::min(p.G, first_minibatch(p, m + 1)));
    }
    return out;
}

int64_t mtile_bound(const Plan &p, Round r) {
    int64_t q0, q1, a, b;
    minibatch_rows(p, r.g0, &q0, &a);
    minibatch_rows(p, r.g1 - 1, &b, &q1);
    const int64_t nmacro = macro_of_minibatch(p, r.g1 - 1) - macro_of_minibatch(p, r.g0) + 1;
    const int64_t nseg = std::min<int64_t>(p.cap, (int64_t)(r.g1 - r.g0) + (int64_t)(p.E - 1) * nmacro);
    return (q1 - q0) / p.tile.BM + nseg + 1;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 1-D grid for a segment GEMM: n_tiles x m-tile bound, rounded up to whole XCD rounds.
dim3 seg_grid(int n_tiles, int64_t mt_bound) {
    return dim3((unsigned)(ceil_div((int64_t)n_tiles * mt_bound, kXcds) * kXcds));
}

struct Macro {
    int m;
    int t0, t1;
    int64_t base;
};

Macro macro_info(const Plan &p, int m) {
    const int64_t t0 = (int64_t)m * p.MT, t1 = std::min<int64_t>(p.T, t0 + p.MT);
    return Macro{m, (int)t0, (int)t1, (int64_t)p.k * t0};
}


}  // namespace
}  // namespace mok
