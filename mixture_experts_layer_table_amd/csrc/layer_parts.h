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

// Tile of a weight-gradient GEMM for workgroup b of the 1-D grid (gx n-tiles
// x gy m-tiles per expert, experts in the order below): b is read as an index into the
// group order of the segment GEMMs, groups of kGroupM m-tiles x all n-tiles.
// Workgroups are dispatched round-robin over the 8 XCDs, so each XCD takes
// every 8th tile of every group: with kGroupM = 4 one m-tile of each group
// and half of its n-tiles, i.e. the 32 tiles an XCD runs together read
// 4 m-slices and 8 n-slices of operands (instead of 2 n-slices and 16
// m-slices in n-fastest order), and every XCD gets the same share of each
// expert's tiles, whose K is the expert's row count.
//
// Experts go in descending order of their row count (ties: lower index
// first) when there are at most kLptExperts of them, so that the longest
// tiles start first and the short ones fill the end (longest-processing-time
// order; the loads of the streaming share are Dirichlet-skewed, and the
// heaviest expert's tiles starting last left half the compute units idle for
// a third of the kernel). With more experts each group is small and the
// order stays by index. Each tile's arithmetic is the same in either order.
constexpr int kLptExperts = 32;
__device__ __forceinline__ int expert_by_rank(const SchedView &v, int r) {
    if (v.E > kLptExperts) return r;
    for (int e = 0; e < v.E; ++e) {
        const int ce = v.counts[e];
        int rank = 0;
        for (int f = 0; f < v.E; ++f) {
            const int cf = v.counts[f];
            rank += (cf > ce || (cf == ce && f < e)) ? 1 : 0;
        }
        if (rank == r) return e;
    }
    return r;   // not reached: the ranks are a permutation of 0 .. E-1
}

__device__ __forceinline__ void wgrad_tile(const SchedView &v, int b, int gx, int gy, int &e, int &m, int &n) {
    const int per_e = gx * gy;
    const int rank = b / per_e;
    e = expert_by_rank(v, rank);
    const int o = b - rank * per_e, gsize = kGroupM * gx, g = o / gsize, first = g * kGroupM;
    const int gm = min(kGroupM, gy - first), r = o - g * gsize;
    m = first + r % gm;
    n = r / gm;
}

// Tile of a segment GEMM for this workgroup. The 1-D grid (a multiple of 8
// workgroups, at least the number of tiles) is dispatched round-robin over the
// XCDs; with `per` = ceil(tiles / 8), workgroup b is mapped to tile
// t = (b % 8) * per + b / 8 so that each XCD walks a contiguous range of
// tiles, ordered in groups of kGroupM m-tiles x all n-tiles: the tiles an XCD
// runs together share few operand slices in its L2.
__device__ __forceinline__ bool decode_seg_tile(const SchedView &v, int g0, int g1, int64_t n_slots, int n_tiles,
                                                int b, SegTile &t) {
    if (*v.status) return false;
    const int lo = v.mtfirst[g0], mtc = v.mtfirst[g1] - lo;
    const int total = mtc * n_tiles;                      // tiles that exist (device-side count)
    const int per = (total + kXcds - 1) / kXcds;
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

// Epilogue rows through buffer descriptors: a descriptor covers the tile's
// valid rows only, so loads of rows past them return zeros and stores to them
// are dropped by the range check, with no branch. A branch around a store
// leaves the number of stores in flight unknown to the compiler, and every
// later wait for a load then waits for all stores (s_waitcnt vmcnt(0)): the
// stores of one fragment would hold up the next fragment's loads. Offsets
// are in bytes.
typedef __amdgpu_buffer_rsrc_t brsrc_t;
__device__ __forceinline__ brsrc_t rows_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), 0,
                                             __builtin_amdgcn_readfirstlane((int)bytes), kBufWord3);
}
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 bload8(brsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x2v_t w = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return make_uint2(w.x, w.y);
}
// non-temporal (cache policy bit 1 on gfx950): see store8_nt
__device__ __forceinline__ void bstore8_nt(brsrc_t r, uint32_t voff, uint32_t soff, uint2 v) {
    u32x2v_t w;
    w.x = v.x;
    w.y = v.y;
    __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)voff, (int)soff, 2);
}
__device__ __forceinline__ void bstore4(brsrc_t r, uint32_t voff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, 0, 0);
}

// The saved pre-activations one lane needs for one 32-row fragment of the
// MXFP8 dA epilogue: for each (fn, g4) block, 4 consecutive columns i of the
// gate half and of the up half of its row (columns >= I read as zeros). The
// epilogue loads one fragment's batch at a time (loading the next one ahead
// of the current one's stores measured slower there).
template <class C>
struct HBatch {
    uint2 g[C::FN][4], u[C::FN][4];
    __device__ __forceinline__ void load(const uint16_t *hrow, int I, int ib, int lane) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int i = ib + fn * 32 + g4 * 8 + (lane >> 5) * 4;
                if (i < I) {
                    g[fn][g4] = *reinterpret_cast<const uint2 *>(hrow + i);
                    u[fn][g4] = *reinterpret_cast<const uint2 *>(hrow + I + i);
                } else {
                    g[fn][g4] = make_uint2(0, 0);
                    u[fn][g4] = make_uint2(0, 0);
                }
            }
    }
};

// ----------------------------------------------------------------------------- LDS-staged epilogue rows

// Epilogue output and input pass through LDS one 32-row fragment at a time,
// so that global memory sees whole 128-byte row runs: a fragment's
// accumulators hold 32 rows x 4 columns per lane, and storing them directly
// writes 8-byte pieces of 32 rows per instruction. Each wave has its own
// 4 KiB area per array ([32 rows][64 columns] bf16); the areas of all waves
// sit at the end of the tile's LDS (LDS_END), inside the last pipeline
// stage(s), which no load targets once every wave has passed the last
// barrier of the K loop. A wave's LDS accesses complete in order, so no
// barrier is needed inside the epilogue. The 8-byte unit u of row r is kept
// at unit u ^ (r % 16): the 32 lanes that hold one column group of 32 rows
// then fall on distinct bank pairs (two rows per pair).
// Lane index as a value the compiler cannot see through: epilogue offsets
// derived from it are computed where they are used instead of being hoisted
// out of a persistent kernel's tile loop and kept live across the K loop.
__device__ __forceinline__ int epi_lane() {
    int l = (int)(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

template <class C, size_t LDS_END>
struct FragStage {
    static_assert(C::WN == 64, "one staged row is 128 bytes");
    static constexpr int ROW = 128;                   // bytes per staged row
    static constexpr int BYTES = 32 * ROW;            // one array of one wave
    static constexpr int LPR = 16;                    // lanes per row in a row pass (8 bytes each)
    static constexpr int RPP = 64 / LPR;              // rows per row pass
    static constexpr int PASSES = 32 / RPP;

    // dynamic LDS starts at offset 0 in every kernel that runs these tiles
    static __device__ __forceinline__ uint32_t area(int wave, int narrays) {
        static_assert(LDS_END >= (size_t)C::NT / 64 * BYTES, "staging must fit the tile's LDS");
        extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
        return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_raw + (uint32_t)LDS_END -
               (uint32_t)((C::NT / 64 - wave) * narrays * BYTES);
    }
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ void put(uint32_t a, uint2 v) {
        u32x2_t w;
        w.x = v.x;
        w.y = v.y;
        *reinterpret_cast<__attribute__((address_space(3))) u32x2_t *>((uintptr_t)a) = w;
    }
    static __device__ __forceinline__ uint2 get(uint32_t a) {
        const u32x2_t w = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t *>((uintptr_t)a);
        return make_uint2(w.x, w.y);
    }
    static __device__ __forceinline__ uint32_t at(int r, int u) { return (uint32_t)(r * ROW + ((u ^ (r & 15)) << 3)); }
    // fragment layout: 4 columns (fn, g4) of row lane % 32
    static __device__ __forceinline__ uint32_t frag_off(int fn, int g4, int lane) {
        return at(lane & 31, fn * 8 + g4 * 2 + (lane >> 5));
    }
    // row-pass layout: pass p covers rows p*RPP .. p*RPP+RPP-1, 4 columns per lane
    static __device__ __forceinline__ int pass_row(int p, int lane) { return p * RPP + lane / LPR; }
    static __device__ __forceinline__ int pass_col(int lane) { return (lane % LPR) * 4; }
    static __device__ __forceinline__ uint32_t pass_off(int p, int lane) { return at(pass_row(p, lane), lane % LPR); }
};

// Gate weight of each fragment row the lane holds (row lane % 32 of each fm),
// loaded when a tile is set up so that the loads hide behind its K loop.
template <class C>
struct RowGates {
    float gw[C::FM];
    __device__ __forceinline__ void load(const SegTile &t, int wm, const SchedView &v, const float *topk_w) {
        const int lane = epi_lane();
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int m = wm * C::WM + fm * 32 + (lane & 31);
            gw[fm] = topk_w[v.perm[t.mt.q0 + (m < t.mt.rows ? m : 0)]];
        }
    }
    // see TokenRows::settle
    __device__ __forceinline__ void settle() {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) asm volatile("" : "+v"(gw[fm]));
    }
};

// 8-byte row-run store of epilogue output with the non-temporal hint: output
// rows are not read again by this kernel, and keeping them out of the L2's
// retained lines leaves room for the operand slices that tiles share.
__device__ __forceinline__ void store8_nt(uint16_t *p, uint2 v) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    v2u w;
    w.x = v.x;
    w.y = v.y;
    __builtin_nontemporal_store(w, reinterpret_cast<v2u *>(p));
}

// One wave's share of a tile leaves as rows, through its FragStage area:
// for each 32-row fragment fm, value(fm, fn, g4, j) is the element of
// fragment row lane % 32 at wave column fn*32 + g4*8 + 4*(lane/32) + j, and
// row_off(fm, r) the byte offset in dst of wave column 0 of fragment row r,
// as this lane stores it (an offset past dst's range, e.g. kOutOfRange: row
// not stored). Every column of the wave is stored (callers return early for
// waves whose columns lie past the output's width).
template <class C, size_t LDS_END, class Val, class Off>
__device__ __forceinline__ void staged_rows(Val value, brsrc_t dst, Off row_off) {
    using FS = FragStage<C, LDS_END>;
    const int lane = epi_lane();
    const uint32_t area = FS::area(wave_id(), 1);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float y[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = value(fm, fn, g4, j);
                FS::put(area + FS::frag_off(fn, g4, lane), make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])));
            }
#pragma unroll
        for (int p = 0; p < FS::PASSES; ++p)
            bstore8_nt(dst, row_off(fm, FS::pass_row(p, lane)) + 2u * (uint32_t)FS::pass_col(lane), 0,
                       FS::get(area + FS::pass_off(p, lane)));
    }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return bf16_to_f32(w & 0xFFFFu); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bf16_to_f32(w >> 16); }
__device__ __forceinline__ float bf16_at(const uint2 &v, int j) {
    return j == 0 ? bf16_lo(v.x) : j == 1 ? bf16_hi(v.x) : j == 2 ? bf16_lo(v.y) : bf16_hi(v.y);
}

// Rows of y (forward down GEMM) or of dx (backward dX GEMM) leave the GEMM
// towards token order. k == 1: straight to the token's row, the forward one
// scaled by its gate weight after rounding y to bf16 (the weighted combine);
// k > 1: into the macro-batch's staging rows, combined later in j order.
//
// k == 1: token (and gate weight) of the lane's fragment rows, row lane % 32
// of each fm. TokenRows::load issues these index loads; a tile calls it before
// its K loop, so that their two dependent round trips (perm, then topk_w) are
// hidden behind the K loop instead of opening the epilogue. (Loaded per pass,
// each fragment's index loads would also wait behind the previous fragment's
// stores.)
template <class C>
struct TokenRows {
    int tok[C::FM];
    float gw[C::FM];
    __device__ __forceinline__ void load(const SegTile &t, int wm, const SchedView &v, int k, const float *topk_w,
                                         bool weighted) {
        const int lane = epi_lane();
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int m = wm * C::WM + fm * 32 + (lane & 31);
            tok[fm] = k == 1 ? v.perm[t.mt.q0 + (m < t.mt.rows ? m : 0)] : 0;
        }
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) gw[fm] = (weighted && k == 1) ? topk_w[tok[fm]] : 1.0f;
    }
    // The loads are long done when the epilogue starts. Waiting for them
    // there, before any store, lets later uses go without a wait; a first use
    // after the epilogue's first stores would wait for those stores as well.
    __device__ __forceinline__ void settle() {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) asm volatile("" : "+v"(tok[fm]), "+v"(gw[fm]));
    }
};

template <class C, size_t LDS_END>
__device__ __forceinline__ void store_token_rows(const f32x16_t (&acc)[C::FM][C::FN], const SegTile &t, int n0,
                                                 int wm, int wn, const TokenRows<C> &tr, int T, int H, int k,
                                                 int MT, int nb_full, bool weighted, uint16_t *dst_k1,
                                                 uint16_t *stage) {
    // H % 64 == 0: the wave's columns are all valid or all past H. A wave past
    // H runs the same stores into an empty range (no early return: every wave
    // then issues the same number of stores, which keeps the compiler's count
    // of stores in flight exact for the waits that follow the tile).
    const int nb = n0 + wn * C::WN;
    const bool live = nb < H;
    TokenRows<C> trs = tr;
    trs.settle();
    const uint32_t row_bytes = 2u * (uint32_t)H;
    // k == 1: the whole output [T][H], rows by token; k > 1: the macro-batch's
    // staging rows, from the tile's first row (byte sizes stay below 2^31)
    const int64_t sbase = (int64_t)k * ((t.mt.g / nb_full) * (int64_t)MT);
    const int cb = live ? nb : 0;
    const brsrc_t dst = k == 1 ? rows_rsrc(dst_k1 + cb, live ? (uint32_t)T * row_bytes : 0u)
                               : rows_rsrc(stage + (t.mt.q0 - sbase) * H + cb,
                                           live ? (uint32_t)t.mt.rows * row_bytes : 0u);
    staged_rows<C, LDS_END>(
        [&](int fm, int fn, int g4, int j) {
            const float y = acc[fm][fn][g4 * 4 + j];
            return (weighted && k == 1) ? trs.gw[fm] * bf16r(y) : y;   // y rows are bf16
        },
        dst, [&](int fm, int r) -> uint32_t {
            const int m = wm * C::WM + fm * 32 + r;
            if (k != 1) return (uint32_t)m * row_bytes;   // rows past the tile lie past dst
            // every lane takes part in the shuffle: lane r holds row r's token
            const int tok_r = __shfl(trs.tok[fm], r);
            return m < t.mt.rows ? (uint32_t)tok_r * row_bytes : kOutOfRange;
        });
}

// The same, loading the token rows at the epilogue (tiles that do not prefetch them).
template <class C, size_t LDS_END>
__device__ __forceinline__ void store_token_rows(const f32x16_t (&acc)[C::FM][C::FN], const SegTile &t, int n0,
                                                 int wm, int wn, const SchedView &v, int H, int k, int MT,
                                                 int nb_full, const float *topk_w, bool weighted, uint16_t *dst_k1,
                                                 uint16_t *stage) {
    TokenRows<C> tr;
    tr.load(t, wm, v, k, topk_w, weighted);
    store_token_rows<C, LDS_END>(acc, t, n0, wm, wn, tr, v.T, H, k, MT, nb_full, weighted, dst_k1, stage);
}

constexpr int kRowsPerBlock = 4;   // one 64-lane wave per row

// Dispatch copy of one row (bf16 ring): one wave moves the row of processing
// position q = mb_start[g] + r from token order into ring slot g % n_slots.
// Canonical (expert, f) position of processing position q of mini-batch g:
// the m-tiles of g are runs of consecutive positions in both orders, listed
// with ascending q0, so a binary search over them finds q's run.
__device__ __forceinline__ int canon_pos(const SchedView &v, int g, int q) {
    int lo = v.mtfirst[g], hi = v.mtfirst[g + 1] - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (v.mtiles[mid].q0 <= q)
            lo = mid;
        else
            hi = mid - 1;
    }
    const MTile t = v.mtiles[lo];
    return t.c0 + (q - t.q0);
}

// 16-byte store with the non-temporal hint (see store8_nt).
__device__ __forceinline__ void store16_nt(uint4 *p, uint4 v) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    v4u w;
    w.x = v.x;
    w.y = v.y;
    w.z = v.z;
    w.w = v.w;
    __builtin_nontemporal_store(w, reinterpret_cast<v4u *>(p));
}

struct GatherBf16 {
    SchedView v;
    int64_t n_slots;
    int MB, H, k;
    const uint16_t *src;
    uint16_t *ring;
    // optional second destination: the same rows at their canonical
    // positions, [R][H] (the weight gradients read them from there)
    uint16_t *canon = nullptr;

    // 8 loads in flight per lane before the stores: a wave moving rows one
    // after the other is otherwise bound by one memory round trip per 1 KiB.
    __device__ __forceinline__ void row(int g, int r) const {
        const int q = v.mb_start[g] + r;
        const int tok = v.perm[q] / k;
        const uint4 *s = reinterpret_cast<const uint4 *>(src + (int64_t)tok * H);
        uint4 *d = reinterpret_cast<uint4 *>(ring + ((g % n_slots) * MB + r) * (int64_t)H);
        uint4 *dc = canon ? reinterpret_cast<uint4 *>(canon + (int64_t)canon_pos(v, g, q) * H) : nullptr;
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
            if (dc) {   // read only by the weight gradients, much later: kept out of the caches
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int c = c0 + i * 64 + lane;
                    if (c < n) store16_nt(dc + c, t[i]);
                }
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
