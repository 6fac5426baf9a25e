// Forward and backward of the MoE layer on gfx950.
//
// Forward, per ring round of mini-batches ("Mixture-of-Kittens(MoK)란?"
// explainer, section 4 ③: a fixed ring buffer consumed in mini-batches):
//   gather   ring[slot(g)] <- x rows in processing order          (dispatch)
//   gate/up  h = x W_gate | x W_up per segment, SwiGLU epilogue   (a -> ring-side buffer;
//            h and g * a, the down weight gradient's operand, -> fwd_ctx)
//   down     y = a W_down, then the weighted combine back to token order
//            (fused into the epilogue when k = 1; staged per macro-batch and
//            summed over j = 0..k-1 in fp32 otherwise)
// Backward walks the rounds in reverse:
//   gather   ring <- dy rows
//   dA       G = dy W_down^T with the SwiGLU backward and the router-weight
//            gradient <G, a> fused into the epilogue ("Cursor Open-Sources
//            Mixture-of-Kittens (MoK)" digest, English abstract)
//   dX       dx rows = dh_g W_gate^T + dh_u W_up^T, combined back to tokens
//   then     router-weight partials summed in ascending order, and the weight
//            gradients per expert over its rows in (expert, f) order (dW_down
//            on a side stream from the last dy gather on, beside the last
//            dgrad GEMMs and dW_gate | dW_up).
// Every output element is produced by one owner with a fixed reduction order
// and no floating-point atomics, so results are bitwise reproducible and
// independent of mini-batch, macro-batch, ring and capacity settings.
#include <mutex>
#include <type_traits>

#include "layer_mx.h"
#include "layer_parts.h"
#include "persist.h"
#include "streams.h"

namespace mok {
namespace {

using CfgA = TileCfg<256, 256, 2, 4, 4>;   // 4 stages of 32 KiB: 3 in flight while one is multiplied
using CfgS = TileCfg<128, 256, 2, 4, 6>;   // small groups: 6 stages of 24 KiB, 80 KiB of weights in flight
// Weight gradients of small groups: K (the expert's rows) is a few k-steps, so
// a tile is mostly its loads and its output stores; two workgroups per compute
// unit (72 KiB of LDS each, at most 128 registers) overlap one's stores with
// the other's loads.
using CfgW = TileCfg<128, 256, 2, 4, 3, 4>;
static_assert(CfgA::BN == kTileN && CfgS::BN == kTileN, "host sizing assumes kTileN-column tiles");

// ----------------------------------------------------------------------------- forward gate/up

struct GateUpArgs {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int MB, H, I;
    const uint16_t *ring, *wg, *wu;
    uint16_t *h, *aring;
    const float *topk_w;
    uint16_t *ga;   // fwd_ctx: g * a rows in canonical order, the down weight gradient's operand
};

template <class Cfg>
struct GateUp {
    using C = Cfg;
    using Args = GateUpArgs;
    static constexpr bool FP8 = false;
    static constexpr bool X_TRANS = false, W_TRANS = true;
    RowLoader<C, C::BM> xl;
    TransLoader<C, C::BN> wl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + TransLoader<C, C::BN>::IPW;
    SegTile t;
    __device__ int mvalid() const { return t.mt.rows; }
    int i0, nk, H, I, MB;
    uint16_t *h, *aring, *ga;
    RowGates<C> rg;

    __device__ bool setup(const Args &a, Blk b) {
        SegTile tt;
        if (!decode_seg_tile(a.v, a.g0, a.g1, a.n_slots, a.n_tiles, b.x, tt)) return false;
        init(a, tt);
        return true;
    }
    // the tile's operands, from an m-tile and n-tile chosen by the caller
    __device__ __forceinline__ void init(const Args &a, const SegTile &tile) {
        t = tile;
        H = a.H;
        I = a.I;
        MB = a.MB;
        i0 = t.nt * (C::BN / 2);
        const int64_t row0 = (int64_t)t.slot * MB + t.rowoff;
        xl.init(a.ring + row0 * H, H, t.mt.rows);
        const int64_t eoff = (int64_t)t.mt.e * H * I;
        wl.init(a.wg + eoff + i0, I, H, I - i0, a.wu + eoff + i0);
        h = a.h;
        aring = a.aring;
        ga = a.ga;
        nk = H / C::BK;
        rg.load(t, wave_id() / C::WAVES_N, a.v, a.topk_w);   // hidden behind the K loop
    }
    __device__ void issue(int kt, uint32_t tile) {
        xl.issue(kt * C::BK, tile);
        wl.issue(kt * C::BK, tile + C::X_BYTES);
    }
    // gate block fn pairs with up block fn + FN/2 inside the same wave
    __device__ int wrow(int wn, int fn) const {
        return fn < C::FN / 2 ? wn * (C::WN / 2) + fn * 32 : C::BN / 2 + wn * (C::WN / 2) + (fn - C::FN / 2) * 32;
    }
    // a = silu(h_gate) * h_up rows for the down GEMM, then publish(), then
    // h = [x W_gate | x W_up] rows and g * a rows (the gate weight times the
    // bf16 a the down GEMM reads), which only the backward reads: all staged
    // through LDS (FragStage). The wave's columns are 32 gate then 32 up
    // columns of the same 32 values of i; every wave calls publish().
    static constexpr bool SPLIT_EPILOGUE = true;
    template <class G>
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn, G &&publish) {
        using FS = FragStage<C, C::LDS_BYTES>;
        // I % 64 == 0: the wave's i are all valid or all past I. The publish
        // below waits for every store anyway, so a wave past I may skip them.
        const bool live = i0 + wn * (C::WN / 2) < I;
        const int ib = live ? i0 + wn * (C::WN / 2) : 0;
        const uint32_t rows = live ? (uint32_t)t.mt.rows : 0u;
        const int lane = epi_lane();
        const uint32_t area = FS::area(wave_id(), 1);
        rg.settle();
        // a (then g * a) for fragment fm in the first half of each staged row
        auto stage_a = [&](int fm, bool weighted) {
#pragma unroll
            for (int fn = 0; fn < C::FN / 2; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float hg = acc[fm][fn][g4 * 4 + j], hu = acc[fm][fn + C::FN / 2][g4 * 4 + j];
                        v[j] = hg * sigmoidf_(hg) * hu;
                        if (weighted) v[j] = rg.gw[fm] * bf16r(v[j]);
                    }
                    FS::put(area + FS::frag_off(fn, g4, lane),
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
                }
        };
        // the first half of each staged row (32 values of i); off(m, cc): byte
        // offset of column cc of tile row m, kOutOfRange for rows not stored;
        // lanes holding the unused second half store nothing
        auto store_a = [&](int fm, brsrc_t dst, auto off) {
#pragma unroll
            for (int p = 0; p < FS::PASSES; ++p) {
                const int m = wm * C::WM + fm * 32 + FS::pass_row(p, lane);
                const int cc = FS::pass_col(lane);
                bstore8_nt(dst, cc < C::WN / 2 ? off(m, cc) : kOutOfRange, 0, FS::get(area + FS::pass_off(p, lane)));
            }
        };
        const uint32_t a_bytes = rows * 2u * (uint32_t)I;
        if (live) {
            // a-ring slot, K-tiled for the down GEMM's loads: [I/32][MB][32]
            // bf16, so that a K-step of 256 rows is one contiguous 16 KiB run
            const brsrc_t adst = rows_rsrc(aring + (int64_t)t.slot * MB * I, (uint32_t)MB * 2u * (uint32_t)I);
            const uint32_t a0 = (uint32_t)(ib / 32) * (uint32_t)MB * 64u + (uint32_t)t.rowoff * 64u;
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
                stage_a(fm, false);
                store_a(fm, adst, [&](int m, int cc) {
                    return m < t.mt.rows ? a0 + (uint32_t)m * 64u + 2u * (uint32_t)cc : kOutOfRange;
                });
            }
        }
        publish();
        if (!live) return;
        // gate columns go to h[.., i], up columns to h[.., I + i]
        const uint32_t h_row = 4u * (uint32_t)I;
        const uint32_t h_col = 2u * (uint32_t)(ib + (FS::pass_col(lane) >= C::WN / 2 ? I - C::WN / 2 : 0));
        staged_rows<C, C::LDS_BYTES>([&](int fm, int fn, int g4, int j) { return acc[fm][fn][g4 * 4 + j]; },
                                     rows_rsrc(h + (int64_t)t.mt.q0 * 2 * I, rows * h_row),
                                     [&](int fm, int r) -> uint32_t {
                                         return (uint32_t)(wm * C::WM + fm * 32 + r) * h_row + h_col;
                                     });
        const brsrc_t gdst = rows_rsrc(ga + (int64_t)t.mt.c0 * I, a_bytes);   // canonical order
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            stage_a(fm, true);
            store_a(fm, gdst, [&](int m, int cc) { return 2u * (uint32_t)(m * I + ib + cc); });
        }
    }
};

// ----------------------------------------------------------------------------- forward down (+ combine)

struct DownArgs {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int MB, H, I, k, MT, nb_full;
    const uint16_t *aring, *wd;
    const float *topk_w;
    uint16_t *out, *stage;
};

template <class Cfg>
struct Down {
    using C = Cfg;
    using Args = DownArgs;
    static constexpr bool FP8 = false;
    static constexpr bool X_TRANS = false, W_TRANS = true;
    RowLoader<C, C::BM> xl;
    TransLoader<C, C::BN> wl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + TransLoader<C, C::BN>::IPW;
    SegTile t;
    __device__ int mvalid() const { return t.mt.rows; }
    int n0, nk, H;
    Args a;
    TokenRows<C> tr;

    __device__ bool setup(const Args &args, Blk b) {
        SegTile tt;
        if (!decode_seg_tile(args.v, args.g0, args.g1, args.n_slots, args.n_tiles, b.x, tt)) return false;
        init(args, tt);
        return true;
    }
    // the tile's operands, from an m-tile and n-tile chosen by the caller
    __device__ __forceinline__ void init(const Args &args, const SegTile &tile) {
        t = tile;
        a = args;
        H = args.H;
        n0 = t.nt * C::BN;
        // a-ring slot: K-tiled, [I/32][MB][32] bf16 (see GateUp's epilogue)
        const uint32_t slot_bytes = (uint32_t)args.MB * (uint32_t)args.I * 2u;
        xl.init_tiled(args.aring + (int64_t)t.slot * args.MB * args.I + (int64_t)t.rowoff * 32,
                      (uint32_t)args.MB * 64u, slot_bytes - (uint32_t)t.rowoff * 64u);
        wl.init(args.wd + (int64_t)t.mt.e * args.I * H + n0, H, args.I, H - n0);
        nk = args.I / C::BK;
        tr.load(t, wave_id() / C::WAVES_N, args.v, args.k, args.topk_w, true);   // hidden behind the K loop
    }
    __device__ void issue(int kt, uint32_t tile) {
        xl.issue(kt * C::BK, tile);
        wl.issue(kt * C::BK, tile + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        store_token_rows<C, C::LDS_BYTES>(acc, t, n0, wm, wn, tr, a.v.T, H, a.k, a.MT, a.nb_full, true, a.out, a.stage);
    }
};

// ----------------------------------------------------------------------------- backward dA (+ SwiGLU bwd, router grad)

struct DAArgs {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int MB, H, I, S;
    const uint16_t *ring, *wd, *h;
    const float *topk_w;
    uint16_t *dh;
    float *dgp;
};

template <class Cfg>
struct DA {
    using C = Cfg;
    using Args = DAArgs;
    static constexpr bool FP8 = false;
    static constexpr bool X_TRANS = false, W_TRANS = false;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    SegTile t;
    __device__ int mvalid() const { return t.mt.rows; }
    int i0, nk;
    Args a;

    __device__ bool setup(const Args &args, Blk b) {
        SegTile tt;
        if (!decode_seg_tile(args.v, args.g0, args.g1, args.n_slots, args.n_tiles, b.x, tt)) return false;
        init(args, tt);
        return true;
    }
    // the tile's operands, from an m-tile and n-tile chosen by the caller
    __device__ __forceinline__ void init(const Args &args, const SegTile &tile) {
        t = tile;
        a = args;
        i0 = t.nt * C::BN;
        const int H = args.H, I = args.I;
        const int64_t row0 = (int64_t)t.slot * args.MB + t.rowoff;
        xl.init(args.ring + row0 * H, H, t.mt.rows);
        wl.init(args.wd + (int64_t)t.mt.e * I * H + (int64_t)i0 * H, H, min(C::BN, I - i0));
        nk = H / C::BK;
    }
    __device__ void issue(int kt, uint32_t tile) {
        xl.issue(kt * C::BK, tile);
        wl.issue(kt * C::BK, tile + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    // SwiGLU backward of the tile, staged through LDS per 32-row fragment
    // (FragStage): h rows come in and dh rows leave as whole row runs, through
    // buffer descriptors over the tile's valid rows (no branches: the next
    // fragment's h loads, issued before this fragment's stores, are then
    // waited for with an exact count instead of behind every store).
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        using FS = FragStage<C, C::LDS_BYTES>;
        const int lane = epi_lane();
        const int I = a.I;
        const int slice = t.nt * C::WAVES_N + wn;
        // I % 64 == 0: this wave's columns are all valid or all past I. A wave
        // past I runs the same loads and stores on empty ranges (see
        // store_token_rows: no early return).
        const bool live = i0 + wn * C::WN < I;
        const int ib = live ? i0 + wn * C::WN : 0;
        const uint32_t rows = live ? (uint32_t)t.mt.rows : 0u;
        const uint32_t sg = FS::area(wave_id(), 2), su = sg + FS::BYTES;
        const uint32_t row_bytes = 4u * (uint32_t)I;   // one h or dh row: 2I bf16
        // h rows in processing order, dh rows in canonical order, from the tile's first row
        const brsrc_t hres = rows_rsrc(a.h + (int64_t)t.mt.q0 * 2 * I, rows * row_bytes);
        const brsrc_t dres = rows_rsrc(a.dh + (int64_t)t.mt.c0 * 2 * I, rows * row_bytes);
        const brsrc_t gres = rows_rsrc(a.dgp + (int64_t)t.mt.q0 * a.S, rows * (uint32_t)a.S * 4u);
        const uint32_t up = 2u * (uint32_t)I;   // the up half of a row, in bytes
        // byte offset of the lane's pass-0 element of fragment 0
        const uint32_t voff0 = (uint32_t)(wm * C::WM + FS::pass_row(0, lane)) * row_bytes +
                               2u * (uint32_t)(ib + FS::pass_col(lane));
        auto voff = [&](int fm, int p) { return voff0 + (uint32_t)(fm * 32 + p * FS::RPP) * row_bytes; };
        uint2 hg[FS::PASSES], hu[FS::PASSES];
        auto load_h = [&](int fm) {
#pragma unroll
            for (int p = 0; p < FS::PASSES; ++p) {
                hg[p] = bload8(hres, voff(fm, p), 0);
                hu[p] = bload8(hres, voff(fm, p), up);
            }
        };
        // gate weights of the lane's fragment rows (row lane % 32 of each fm), in
        // flight together with the first fragment's h rows
        float gws[C::FM];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int mrow = wm * C::WM + fm * 32 + (lane & 31);
            gws[fm] = a.topk_w[a.v.perm[t.mt.q0 + (mrow < t.mt.rows ? mrow : 0)]];
        }
        load_h(0);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
            for (int p = 0; p < FS::PASSES; ++p) {
                FS::put(sg + FS::pass_off(p, lane), hg[p]);
                FS::put(su + FS::pass_off(p, lane), hu[p]);
            }
            __builtin_amdgcn_sched_barrier(0);   // phases stay in order: keeps live ranges short
            const float gw = gws[fm];
            float dg = 0.0f;
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const uint32_t o = FS::frag_off(fn, g4, lane);
                    const uint2 hg2 = FS::get(sg + o), hu2 = FS::get(su + o);
                    float dhg[4], dhu[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float G = acc[fm][fn][g4 * 4 + j];
                        const float hgv = bf16_at(hg2, j), huv = bf16_at(hu2, j);
                        const float s = sigmoidf_(hgv);
                        const float sl = hgv * s;
                        const float av = sl * huv;
                        dg += G * av;
                        const float da = gw * G;
                        dhu[j] = da * sl;
                        dhg[j] = da * huv * s * (1.0f + hgv * (1.0f - s));
                    }
                    FS::put(sg + o, make_uint2(pack_bf16x2(dhg[0], dhg[1]), pack_bf16x2(dhg[2], dhg[3])));
                    FS::put(su + o, make_uint2(pack_bf16x2(dhu[0], dhu[1]), pack_bf16x2(dhu[2], dhu[3])));
                }
            __builtin_amdgcn_sched_barrier(0);
            // next fragment's h in flight while this one's rows are stored (its accumulators are dead now)
            if (fm + 1 < C::FM) load_h(fm + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < FS::PASSES; ++p) {
                const uint32_t o = FS::pass_off(p, lane);
                bstore8_nt(dres, voff(fm, p), 0, FS::get(sg + o));
                bstore8_nt(dres, voff(fm, p), up, FS::get(su + o));
            }
            // lanes l and l ^ 32 hold the same row: lower half + upper half, fixed order
            const float other = __shfl_xor(dg, 32);
            const float tot = (lane < 32) ? dg + other : other + dg;
            const int mrow = wm * C::WM + fm * 32 + (lane & 31);
            bstore4(gres, lane < 32 ? (uint32_t)(mrow * a.S + slice) * 4u : kOutOfRange, tot);
        }
    }
};

// ----------------------------------------------------------------------------- backward dX (+ combine)

struct DXArgs {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int H, I, k, MT, nb_full;
    const uint16_t *dh, *wg, *wu;
    uint16_t *dx, *stage;
};

template <class Cfg>
struct DX {
    using C = Cfg;
    using Args = DXArgs;
    static constexpr bool FP8 = false;
    static constexpr bool X_TRANS = false, W_TRANS = false;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    SegTile t;
    __device__ int mvalid() const { return t.mt.rows; }
    int n0, nk, I;
    Args a;
    TokenRows<C> tr;

    __device__ bool setup(const Args &args, Blk b) {
        SegTile tt;
        if (!decode_seg_tile(args.v, args.g0, args.g1, args.n_slots, args.n_tiles, b.x, tt)) return false;
        init(args, tt);
        return true;
    }
    // the tile's operands, from an m-tile and n-tile chosen by the caller
    __device__ __forceinline__ void init(const Args &args, const SegTile &tile) {
        t = tile;
        a = args;
        n0 = t.nt * C::BN;
        I = args.I;
        const int H = args.H;
        xl.init(args.dh + (int64_t)t.mt.c0 * 2 * I, 2 * I, t.mt.rows);
        const int64_t wo = (int64_t)t.mt.e * H * I + (int64_t)n0 * I;
        wl.init(args.wg + wo, I, min(C::BN, H - n0), args.wu + wo, I);
        nk = 2 * I / C::BK;
        tr.load(t, wave_id() / C::WAVES_N, args.v, args.k, nullptr, false);   // hidden behind the K loop
    }
    __device__ void issue(int kt, uint32_t tile) {
        xl.issue(kt * C::BK, tile);
        wl.issue(kt * C::BK, tile + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        store_token_rows<C, C::LDS_BYTES>(acc, t, n0, wm, wn, tr, a.v.T, a.H, a.k, a.MT, a.nb_full, false, a.dx, a.stage);
    }
};

// ----------------------------------------------------------------------------- weight gradients

// dW_gate[e] | dW_up[e] = X_e^T [dh_g | dh_u]: M = H, N = 2I, K = rows of e in
// (expert, f) order, in BK chunks anchored at the expert's first row.
struct WGUArgs {
    SchedView v;
    int H, I;
    const uint16_t *x;    // x [T][H], token order (read through the token index)
    const uint16_t *xc;   // x rows in canonical order [R][H] (CANON), else unused
    const uint16_t *dh;   // dh rows in canonical order
    uint16_t *dwg, *dwu;
};

// CANON: the x rows come from their canonical-order copy as contiguous rows;
// otherwise they are gathered from x through the token index (ctok).
template <class Cfg, bool CANON>
struct WGU {
    using C = Cfg;
    using Args = WGUArgs;
    static constexpr bool X_TRANS = true, W_TRANS = true;
    using XL = std::conditional_t<CANON, TransLoader<C, C::BM>, TransIdxLoader<C, C::BM>>;
    XL xl;                      // x rows of the expert's tokens, k = canonical row
    TransLoader<C, C::BN> wl;   // dh rows of the expert
    static constexpr int LOADS_PER_STAGE = XL::IPW + TransLoader<C, C::BN>::IPW;
    int e, h0, n0, ne, off, nk;
    Args a;
    __device__ int mvalid() const { return a.H - h0; }

    __device__ bool setup(const Args &args, Blk b) {
        // the status word is read together with the expert's count and offset
        // (one round trip); both are in bounds whatever the status
        const int bad = *args.v.status;
        a = args;
        wgrad_tile(args.v, b.x, (2 * args.I + C::BN - 1) / C::BN, (args.H + C::BM - 1) / C::BM, e, h0, n0);
        h0 *= C::BM;
        n0 *= C::BN;
        ne = args.v.counts[e];
        off = args.v.offsets[e];
        if (bad) return false;
        nk = (ne + C::BK - 1) / C::BK;
        if constexpr (CANON)
            xl.init(args.xc + (int64_t)off * args.H + h0, args.H, ne, args.H - h0);
        else
            xl.init(args.v.ctok + off, ne, args.x, args.H, args.v.T, h0);
        const int I2 = 2 * args.I;
        wl.init(args.dh + (int64_t)off * I2 + n0, I2, ne, I2 - n0);
        return true;
    }
    __device__ void fetch(int kt) {
        if constexpr (!CANON) xl.fetch(kt * C::BK);
    }
    __device__ void issue(int kt, uint32_t tile) {
        xl.issue(kt * C::BK, tile);
        wl.issue(kt * C::BK, tile + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        const int H = a.H, I = a.I;
        const int nb = n0 + wn * C::WN;
        if (nb >= 2 * I) return;   // I % 64 == 0: the wave's columns are all gate, all up or all past 2I
        uint16_t *base = (nb < I ? a.dwg + nb : a.dwu + (nb - I)) + (int64_t)e * H * I;   // expert e's rows
        staged_rows<C, C::LDS_BYTES>([&](int fm, int fn, int g4, int j) { return acc[fm][fn][g4 * 4 + j]; },
                                     rows_rsrc(base, 2u * (uint32_t)H * (uint32_t)I), [&](int fm, int r) -> uint32_t {
                                         return 2u * (uint32_t)(h0 + wm * C::WM + fm * 32 + r) * (uint32_t)I;
                                     });
    }
};

// dW_down[e] = (g a)_e^T dY_e: M = I, N = H, K as above.
struct WDArgs {
    SchedView v;
    int H, I;
    const uint16_t *ga;    // g*a rows in canonical order
    const uint16_t *dy;    // dy [T][H], token order (read through the token index)
    const uint16_t *dyc;   // dy rows in canonical order [R][H] (CANON), else unused
    uint16_t *dwd;
};

template <class Cfg, bool CANON>
struct WD {
    using C = Cfg;
    using Args = WDArgs;
    static constexpr bool X_TRANS = true, W_TRANS = true;
    using WL = std::conditional_t<CANON, TransLoader<C, C::BN>, TransIdxLoader<C, C::BN>>;
    TransLoader<C, C::BM> xl;   // g*a rows of the expert
    WL wl;                      // dy rows of the expert's tokens
    static constexpr int LOADS_PER_STAGE = TransLoader<C, C::BM>::IPW + WL::IPW;
    int e, i0, n0, ne, off, nk;
    Args a;
    __device__ int mvalid() const { return a.I - i0; }

    __device__ bool setup(const Args &args, Blk b) {
        const int bad = *args.v.status;   // read with the count and offset, as in WGU
        a = args;
        wgrad_tile(args.v, b.x, (args.H + C::BN - 1) / C::BN, (args.I + C::BM - 1) / C::BM, e, i0, n0);
        i0 *= C::BM;
        n0 *= C::BN;
        ne = args.v.counts[e];
        off = args.v.offsets[e];
        if (bad) return false;
        nk = (ne + C::BK - 1) / C::BK;
        if constexpr (CANON)
            wl.init(args.dyc + (int64_t)off * args.H + n0, args.H, ne, args.H - n0);
        else
            wl.init(args.v.ctok + off, ne, args.dy, args.H, args.v.T, n0);
        xl.init(args.ga + (int64_t)off * args.I + i0, args.I, ne, args.I - i0);
        return true;
    }
    __device__ void fetch(int kt) {
        if constexpr (!CANON) wl.fetch(kt * C::BK);
    }
    __device__ void issue(int kt, uint32_t tile) {
        xl.issue(kt * C::BK, tile);
        wl.issue(kt * C::BK, tile + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        const int H = a.H, I = a.I;
        const int nb = n0 + wn * C::WN;
        if (nb >= H) return;   // H % 64 == 0
        staged_rows<C, C::LDS_BYTES>([&](int fm, int fn, int g4, int j) { return acc[fm][fn][g4 * 4 + j]; },
                                     rows_rsrc(a.dwd + (int64_t)e * I * H + nb, 2u * (uint32_t)I * (uint32_t)H),
                                     [&](int fm, int r) -> uint32_t {
                                         return 2u * (uint32_t)(i0 + wm * C::WM + fm * 32 + r) * (uint32_t)H;
                                     });
    }
};

// ----------------------------------------------------------------------------- streaming kernels


// ring[slot(g)][r] = src[token of processing position q] for q in mini-batch g
__global__ __launch_bounds__(256) void gather_rows(GatherBf16 ga, int g0) {
    if (*ga.v.status) return;
    const int g = g0 + blockIdx.y;
    const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (ga.v.mb_start[g] + r >= ga.v.mb_start[g + 1]) return;
    ga.row(g, r);
}

// Identity experts (debug): y rows = ring rows, then the same combine as the layer.
__global__ __launch_bounds__(256) void identity_rows(SchedView v, int g0, int64_t n_slots, int MB, int H, int k,
                                                     int MT, int nb_full, const float *__restrict__ topk_w,
                                                     const uint16_t *__restrict__ ring, uint16_t *__restrict__ out,
                                                     uint16_t *__restrict__ stage) {
    if (*v.status) return;
    const int g = g0 + blockIdx.y;
    const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    const int q = v.mb_start[g] + r;
    if (q >= v.mb_start[g + 1]) return;
    const uint4 *s = reinterpret_cast<const uint4 *>(ring + ((g % n_slots) * MB + r) * (int64_t)H);
    if (k == 1) {
        const int tok = v.perm[q];
        const float gw = topk_w[tok];
        uint4 *d = reinterpret_cast<uint4 *>(out + (int64_t)tok * H);
        for (int c = threadIdx.x & 63; c < H / 8; c += 64) {
            const uint4 x = s[c];
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = pack_bf16x2(gw * bf16_to_f32(w[j] & 0xFFFFu), gw * bf16_to_f32(w[j] >> 16));
            d[c] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else {
        const int64_t base = (int64_t)k * ((g / nb_full) * (int64_t)MT);
        uint4 *d = reinterpret_cast<uint4 *>(stage + (q - base) * H);
        for (int c = threadIdx.x & 63; c < H / 8; c += 64) d[c] = s[c];
    }
}

// out[t] = sum_{j=0..k-1} g[t,j] * y[t,j] (fp32, j ascending), tokens of one macro-batch;
// with weighted == false the plain sum (input-gradient combine). One workgroup
// per token, kCombineChunks 16-byte chunks of the row per thread: each thread
// issues the loads of a whole batch of kCombineBatch staged rows for all its
// chunks before it adds them, in j order. The row indices and gate weights of
// a batch are read by every lane (one broadcast line): no LDS and no barrier,
// so a workgroup starts streaming at once. (One 256-thread workgroup per token
// staging the indices through LDS moved 67% of the HBM peak on a probe of the
// full layer's k = 8 combine; this form 76%.)
constexpr int kCombineBatch = 8;
constexpr int kCombineChunks = 2;
__global__ __launch_bounds__(512) void combine_rows(SchedView v, int t0, int H, int k, int64_t base,
                                                    const float *__restrict__ topk_w, bool weighted,
                                                    const uint16_t *__restrict__ stage, uint16_t *__restrict__ out) {
    if (*v.status) return;
    const int t = t0 + blockIdx.x;
    const int n = H / 8, nt = (int)blockDim.x;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(stage);   // each staged row is read once
    for (int cb = 0; cb < n; cb += kCombineChunks * nt) {
        float acc[kCombineChunks][8];
#pragma unroll
        for (int c = 0; c < kCombineChunks; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
        for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
            int64_t row[kCombineBatch];
            float gw[kCombineBatch];
#pragma unroll
            for (int b = 0; b < kCombineBatch; ++b) {
                const int f = t * k + min(j0 + b, k - 1);
                row[b] = (int64_t)(v.inv[f] - base) * n;
                gw[b] = weighted ? topk_w[f] : 1.0f;
            }
            u32x4_t x[kCombineChunks][kCombineBatch];
#pragma unroll
            for (int c = 0; c < kCombineChunks; ++c) {
                const int ch = cb + c * nt + (int)threadIdx.x;
#pragma unroll
                for (int b = 0; b < kCombineBatch; ++b)
                    x[c][b] = (j0 + b < k && ch < n) ? __builtin_nontemporal_load(src + row[b] + ch) : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
            for (int b = 0; b < kCombineBatch; ++b) {
                if (j0 + b >= k) break;
                const float g = gw[b];
#pragma unroll
                for (int c = 0; c < kCombineChunks; ++c) {
                    const uint32_t w4[4] = {x[c][b].x, x[c][b].y, x[c][b].z, x[c][b].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float lo = bf16_to_f32(w4[i] & 0xFFFFu), hi = bf16_to_f32(w4[i] >> 16);
                        acc[c][2 * i] = weighted ? __builtin_fmaf(g, lo, acc[c][2 * i]) : acc[c][2 * i] + lo;
                        acc[c][2 * i + 1] = weighted ? __builtin_fmaf(g, hi, acc[c][2 * i + 1]) : acc[c][2 * i + 1] + hi;
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kCombineChunks; ++c) {
            const int ch = cb + c * nt + (int)threadIdx.x;
            if (ch < n)
                reinterpret_cast<uint4 *>(out + (int64_t)t * H)[ch] =
                    make_uint4(pack_bf16x2(acc[c][0], acc[c][1]), pack_bf16x2(acc[c][2], acc[c][3]),
                               pack_bf16x2(acc[c][4], acc[c][5]), pack_bf16x2(acc[c][6], acc[c][7]));
        }
    }
}

// Threads of a combine workgroup: enough for kCombineChunks chunks each of an
// H-wide row, in whole waves, at most 512.
inline unsigned combine_threads(int H) {
    const int n = H / 8;
    return (unsigned)std::min(512, std::max(64, (n + kCombineChunks * 64 - 1) / (kCombineChunks * 64) * 64));
}

// dtopk_w[f] = sum over I-slices s ascending of the partials <G, a> of row inv[f]
__global__ __launch_bounds__(256) void reduce_router_grad(SchedView v, int S, const float *__restrict__ dgp,
                                                          float *__restrict__ dtopk_w) {
    if (*v.status) return;
    const int f = blockIdx.x * 256 + threadIdx.x;
    if (f >= v.R) return;
    const float *p = dgp + (int64_t)v.inv[f] * S;
    float s = 0.0f;
    for (int i = 0; i < S; ++i) s += p[i];
    dtopk_w[f] = s;
}

// ----------------------------------------------------------------------------- item trace (measurement aid)

static __device__ __align__(256) mok_item_record item_trace_records[MOK_ITEM_TRACE_CAPACITY];
static __device__ int item_trace_count;

struct TraceState {
    std::mutex mu;
    bool on = false;
    uint32_t launch = 0;
    int device = -1;
    mok_item_record *rec = nullptr;   // the current device's copies (hipGetSymbolAddress)
    int *count = nullptr;
};
TraceState g_trace;

// The trace destination for the next launch of `kernel` (all null while tracing is off).
TraceArgs trace_args(int kernel) {
    std::lock_guard<std::mutex> lk(g_trace.mu);
    if (!g_trace.on) return TraceArgs{nullptr, nullptr, 0, 0, kernel};
    return TraceArgs{g_trace.rec, g_trace.count, MOK_ITEM_TRACE_CAPACITY, g_trace.launch++, kernel};
}

// ----------------------------------------------------------------------------- host side

template <class P>
hipError_t launch_gemm(const char *name, dim3 grid, const typename P::Args &args, hipStream_t st,
                       int trace_kernel = MOK_TRACE_OTHER) {
    using C = typename P::C;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_kernel<P>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)C::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
    KernelTimer tm(name, st);
    gemm_kernel<P><<<grid, C::NT, C::LDS_BYTES, st>>>(args, trace_args(trace_kernel));
    return hipGetLastError();
}

// BF16 with 256-row tiles only: MXFP8 runs its rounds as separate launches
// whatever the flag, and small-group layers (128-row tiles) run ring rounds.
bool whole_pass(const Plan &p) {
    return p.k == 1 && p.precision == MOK_BF16 && p.tile.BM == CfgA::BM && (p.debug & MOK_DEBUG_WHOLE_PASS) &&
           !(p.debug & MOK_DEBUG_SEPARATE_LAUNCHES);
}

// The two grouped GEMMs of one forward ring round (gate/up, then down), in
// the tile family C.
template <class C>
hipError_t fwd_round_gemms(const Plan &p, const GateUpArgs &ga, const DownArgs &da, int64_t mt, int *sync,
                           hipStream_t st) {
    if (p.debug & MOK_DEBUG_SEPARATE_LAUNCHES) {
        const hipError_t e = launch_gemm<GateUp<C>>("gateup", seg_grid(ga.n_tiles, mt), ga, st);
        return e != hipSuccess ? e : launch_gemm<Down<C>>("down", seg_grid(da.n_tiles, mt), da, st);
    }
    return launch_pair<GateUp<C>, Down<C>, C::LDS_BYTES>("fwd_gemms", ga, da, sync, p.max_mtiles, spin_limit(p),
                                                         persistent_grid(p), st, trace_args(MOK_TRACE_FWD_GEMMS));
}

// The two grouped GEMMs of one backward ring round (dA, then dX).
template <class C>
hipError_t bwd_round_gemms(const Plan &p, const DAArgs &aa, const DXArgs &xa, int64_t mt, int *sync,
                           hipStream_t st) {
    if (p.debug & MOK_DEBUG_SEPARATE_LAUNCHES) {
        const hipError_t e = launch_gemm<DA<C>>("dA", seg_grid(aa.n_tiles, mt), aa, st);
        return e != hipSuccess ? e : launch_gemm<DX<C>>("dX", seg_grid(xa.n_tiles, mt), xa, st);
    }
    return launch_pair<DA<C>, DX<C>, C::LDS_BYTES>("bwd_gemms", aa, xa, sync, p.max_mtiles, spin_limit(p),
                                                   persistent_grid(p), st, trace_args(MOK_TRACE_BWD_GEMMS));
}

// The weight-gradient GEMMs, dW_gate | dW_up and dW_down, in the tile family
// chosen by the plan; CANON: x and dy rows read from their canonical copies.
hipError_t wgrad_gate_up(const Plan &p, const WGUArgs &gu, hipStream_t st) {
    auto run = [&](auto c, auto canon) {
        using C = decltype(c);
        return launch_gemm<WGU<C, decltype(canon)::value>>(
            "wgrad_gate_up", dim3((unsigned)(ceil_div(2 * p.I, C::BN) * ceil_div(p.H, C::BM) * p.E)), gu, st,
            MOK_TRACE_WGRAD_GATE_UP);
    };
    if (p.keep_canonical && !gu.xc) return hipErrorInvalidValue;   // not reachable: derives from validated buffers
    if (p.tile.BM == CfgS::BM)
        return p.keep_canonical ? run(CfgW{}, std::true_type{}) : run(CfgW{}, std::false_type{});
    return p.keep_canonical ? run(CfgA{}, std::true_type{}) : run(CfgA{}, std::false_type{});
}
hipError_t wgrad_down(const Plan &p, const WDArgs &wda, hipStream_t st) {
    auto run = [&](auto c, auto canon) {
        using C = decltype(c);
        return launch_gemm<WD<C, decltype(canon)::value>>(
            "wgrad_down", dim3((unsigned)(ceil_div(p.H, C::BN) * ceil_div(p.I, C::BM) * p.E)), wda, st,
            MOK_TRACE_WGRAD_DOWN);
    };
    if (p.keep_canonical && !wda.dyc) return hipErrorInvalidValue;   // not reachable: derives from validated buffers
    if (p.tile.BM == CfgS::BM)
        return p.keep_canonical ? run(CfgW{}, std::true_type{}) : run(CfgW{}, std::false_type{});
    return p.keep_canonical ? run(CfgA{}, std::true_type{}) : run(CfgA{}, std::false_type{});
}

}  // namespace

TraceArgs item_trace_args(int kernel) { return trace_args(kernel); }

mok_status launch_forward(const Plan &p, const void *schedule, void *workspace, const uint16_t *x,
                          const float *topk_w, const mok_weights &w, uint16_t *out, void *fwd_ctx,
                          hipStream_t st) {
    if (p.R == 0) return MOK_OK;
    const bool mx = p.precision == MOK_MXFP8;
    const bool identity = p.debug & MOK_DEBUG_IDENTITY_EXPERT;
    if (mx && identity) return MOK_ERROR_UNSUPPORTED;
    const SchedView v = make_sched_view(p, const_cast<void *>(schedule));
    char *ws = static_cast<char *>(workspace);
    uint16_t *ring = reinterpret_cast<uint16_t *>(ws + p.w_ring);
    uint16_t *aring = reinterpret_cast<uint16_t *>(ws + p.w_aring);
    uint16_t *stage = reinterpret_cast<uint16_t *>(ws + p.w_stage);
    uint16_t *h = reinterpret_cast<uint16_t *>(static_cast<char *>(fwd_ctx) + p.c_h);
    uint16_t *ga_rows = reinterpret_cast<uint16_t *>(static_cast<char *>(fwd_ctx) + p.c_ga);
    // x rows saved in canonical order for the weight gradients (null when the plan keeps none)
    uint16_t *xc = p.keep_canonical ? reinterpret_cast<uint16_t *>(static_cast<char *>(fwd_ctx) + p.c_xc) : nullptr;
    if (p.x_ring_is_copy && !identity) {   // the copy doubles as the ring: one write per x row
        ring = xc;
        xc = nullptr;
    }
    int *sync = reinterpret_cast<int *>(ws + p.w_sync);
    hipError_t err = hipSuccess;
    if (whole_pass(p) && !identity) {   // one launch for the pass, ring protocol in the kernel
        const int ntg = (int)ceil_div(p.I, CfgA::BN / 2), ntd = (int)ceil_div(p.H, CfgA::BN);
        GateUpArgs ga{v, 0, p.G, ntg, p.n_slots, p.MB, p.H, p.I, ring, static_cast<const uint16_t *>(w.w_gate),
                      static_cast<const uint16_t *>(w.w_up), h, aring, topk_w, ga_rows};
        DownArgs da{v, 0, p.G, ntd, p.n_slots, p.MB, p.H, p.I, p.k, (int)p.MT, p.nb_full, aring,
                    static_cast<const uint16_t *>(w.w_down), topk_w, out, stage};
        err = launch_pass<GatherBf16, GateUp<CfgA>, Down<CfgA>, 3, CfgA::LDS_BYTES>(
            "fwd_pass", p, GatherBf16{v, p.n_slots, p.MB, p.H, p.k, x, ring}, ga, da, false, sync, st);
        if (err == hipSuccess) err = hipGetLastError();
        return check_hip(err, "mok_forward");
    }
    for (const Round r : make_rounds(p, false)) {
        const dim3 sgrid((unsigned)ceil_div(p.MB, kRowsPerBlock), (unsigned)(r.g1 - r.g0));
        if (mx) {
            if ((err = mx_forward_round(p, v, r.g0, r.g1, mtile_bound(p, r), x, w, ws, h, ga_rows, xc, topk_w, out,
                                        stage, st)) != hipSuccess)
                break;
        } else {
            {
            KernelTimer tm("gather", st);
            gather_rows<<<sgrid, 256, 0, st>>>(GatherBf16{v, p.n_slots, p.MB, p.H, p.k, x, ring, xc}, r.g0);
        }
        if (identity) {
            KernelTimer tm("identity", st);
            identity_rows<<<sgrid, 256, 0, st>>>(v, r.g0, p.n_slots, p.MB, p.H, p.k, (int)p.MT, p.nb_full, topk_w,
                                                 ring, out, stage);
        } else {
            const int64_t mt = mtile_bound(p, r);
            const int ntg = (int)ceil_div(p.I, CfgA::BN / 2), ntd = (int)ceil_div(p.H, CfgA::BN);
            GateUpArgs ga{v, r.g0, r.g1, ntg, p.n_slots, p.MB, p.H, p.I, ring, static_cast<const uint16_t *>(w.w_gate),
                          static_cast<const uint16_t *>(w.w_up), h, aring, topk_w, ga_rows};
            DownArgs da{v, r.g0, r.g1, ntd, p.n_slots, p.MB, p.H, p.I, p.k, (int)p.MT, p.nb_full, aring,
                        static_cast<const uint16_t *>(w.w_down), topk_w, out, stage};
            err = p.tile.BM == CfgS::BM ? fwd_round_gemms<CfgS>(p, ga, da, mt, sync, st)
                                        : fwd_round_gemms<CfgA>(p, ga, da, mt, sync, st);
            if (err != hipSuccess) break;
        }
        }
        if (p.k > 1 && (r.g1 == p.G || r.g1 == first_minibatch(p, macro_of_minibatch(p, r.g0) + 1))) {
            const Macro mc = macro_info(p, macro_of_minibatch(p, r.g0));
            KernelTimer tm("combine", st);
            if (mc.t1 > mc.t0)
                combine_rows<<<(unsigned)(mc.t1 - mc.t0), combine_threads(p.H), 0, st>>>(v, mc.t0, p.H, p.k, mc.base,
                                                                                         topk_w, true, stage, out);
        }
    }
    if (err == hipSuccess) err = hipGetLastError();
    return check_hip(err, "mok_forward");
}

mok_status launch_backward(const Plan &p, const void *schedule, void *workspace, const uint16_t *x,
                           const float *topk_w, const mok_weights &w, const void *fwd_ctx, const uint16_t *dy,
                           uint16_t *dx, uint16_t *dw_gate, uint16_t *dw_up, uint16_t *dw_down, float *dtopk_w,
                           hipStream_t st) {
    const bool mx = p.precision == MOK_MXFP8;
    const SchedView v = make_sched_view(p, const_cast<void *>(schedule));
    char *ws = static_cast<char *>(workspace);
    uint16_t *ring = reinterpret_cast<uint16_t *>(ws + p.w_ring);
    uint16_t *stage = reinterpret_cast<uint16_t *>(ws + p.w_stage);
    uint16_t *dh = reinterpret_cast<uint16_t *>(ws + p.w_dh);
    float *dgp = reinterpret_cast<float *>(ws + p.w_dgp);
    const uint16_t *h = reinterpret_cast<const uint16_t *>(static_cast<const char *>(fwd_ctx) + p.c_h);
    const uint16_t *ga = reinterpret_cast<const uint16_t *>(static_cast<const char *>(fwd_ctx) + p.c_ga);
    const uint16_t *xc =
        p.keep_canonical ? reinterpret_cast<const uint16_t *>(static_cast<const char *>(fwd_ctx) + p.c_xc) : nullptr;
    // dy rows in canonical order for the weight gradients: the ring itself
    // when it holds them so, else a copy the dy gather writes
    uint16_t *dyc = !p.keep_canonical ? nullptr : p.dy_in_ring ? ring : reinterpret_cast<uint16_t *>(ws + p.w_dyc);
    uint16_t *dyc_copy = p.keep_canonical && !p.dy_in_ring ? dyc : nullptr;
    const uint16_t *wg = static_cast<const uint16_t *>(w.w_gate);
    const uint16_t *wu = static_cast<const uint16_t *>(w.w_up);
    const uint16_t *wd = static_cast<const uint16_t *>(w.w_down);
    int *sync = reinterpret_cast<int *>(ws + p.w_sync);
    hipError_t err = hipSuccess;
    hipStream_t wq_side = st;   // MXFP8 weight gradients: x and dy quantizers forked to a side stream
    if (p.mx_wgrad) err = mx_wgrad_begin(p, v, ws, x, dy, st, &wq_side);
    // BF16 dW_down needs only g * a (saved by the forward) and the dy rows: it
    // starts on a side stream once the last round's dy gather is enqueued and
    // runs beside the last dgrad GEMMs and dW_gate | dW_up, filling their tails.
    const WDArgs wda{v, p.H, p.I, ga, dy, dyc, dw_down};
    hipStream_t wd_side = st;
    bool wd_launched = false;
    auto launch_wd_beside = [&]() -> hipError_t {
        wd_side = side_fork(st);
        wd_launched = true;
        return wgrad_down(p, wda, wd_side);
    };
    if (err != hipSuccess) {
    } else if (p.R > 0 && whole_pass(p)) {   // one launch for the dgrad pass
        const int nta = (int)ceil_div(p.I, CfgA::BN), ntx = (int)ceil_div(p.H, CfgA::BN);
        DAArgs aa{v, 0, p.G, nta, p.n_slots, p.MB, p.H, p.I, p.dg_slices, ring, wd, h, topk_w, dh, dgp};
        DXArgs xa{v, 0, p.G, ntx, p.n_slots, p.H, p.I, p.k, (int)p.MT, p.nb_full, dh, wg, wu, dx, stage};
        err = launch_pass<GatherBf16, DA<CfgA>, DX<CfgA>, 2, CfgA::LDS_BYTES>(
            "bwd_pass", p, GatherBf16{v, p.n_slots, p.MB, p.H, p.k, dy, ring}, aa, xa, true, sync, st);
        if (err == hipSuccess) {
            KernelTimer tm("router_grad", st);
            reduce_router_grad<<<(unsigned)ceil_div(p.R, 256), 256, 0, st>>>(v, p.dg_slices, dgp, dtopk_w);
        }
    } else if (p.R > 0) {
        const std::vector<Round> rounds = make_rounds(p, true);
        for (size_t ri = 0; ri < rounds.size(); ++ri) {
            const Round r = rounds[ri];
            const bool last = ri + 1 == rounds.size();
            const dim3 sgrid((unsigned)ceil_div(p.MB, kRowsPerBlock), (unsigned)(r.g1 - r.g0));
            if (mx) {
                err = mx_gather_dy(p, v, r.g0, r.g1, dy, ws, dyc_copy, st);
            } else {
                KernelTimer tm("gather_dy", st);
                gather_rows<<<sgrid, 256, 0, st>>>(GatherBf16{v, p.n_slots, p.MB, p.H, p.k, dy, ring, dyc_copy}, r.g0);
                err = hipGetLastError();
            }
            if (err == hipSuccess && last && !p.mx_wgrad) err = launch_wd_beside();
            if (err != hipSuccess) break;
            const int64_t mt = mtile_bound(p, r);
            if (mx) {
                err = mx_backward_gemms(p, v, r.g0, r.g1, mt, w, ws, h, topk_w, dx, stage, st);
            } else {
                const int nta = (int)ceil_div(p.I, CfgA::BN), ntx = (int)ceil_div(p.H, CfgA::BN);
                DAArgs aa{v, r.g0, r.g1, nta, p.n_slots, p.MB, p.H, p.I, p.dg_slices, ring, wd, h, topk_w, dh, dgp};
                DXArgs xa{v, r.g0, r.g1, ntx, p.n_slots, p.H, p.I, p.k, (int)p.MT, p.nb_full, dh, wg, wu, dx, stage};
                err = p.tile.BM == CfgS::BM ? bwd_round_gemms<CfgS>(p, aa, xa, mt, sync, st)
                                            : bwd_round_gemms<CfgA>(p, aa, xa, mt, sync, st);
            }
            if (err != hipSuccess) break;
            if (p.k > 1 && r.g0 == first_minibatch(p, macro_of_minibatch(p, r.g0))) {
                const Macro mc = macro_info(p, macro_of_minibatch(p, r.g0));
                KernelTimer tm("combine_dx", st);
                if (mc.t1 > mc.t0)
                    combine_rows<<<(unsigned)(mc.t1 - mc.t0), combine_threads(p.H), 0, st>>>(
                        v, mc.t0, p.H, p.k, mc.base, topk_w, false, stage, dx);
            }
        }
        if (err == hipSuccess) {
            KernelTimer tm("router_grad", st);
            reduce_router_grad<<<(unsigned)ceil_div(p.R, 256), 256, 0, st>>>(v, p.dg_slices, dgp, dtopk_w);
        }
    }
    if (p.mx_wgrad) {
        // after an error only the join: no fork is left open
        const hipError_t e2 = mx_wgrad_finish(p, v, ws, ga, wq_side, err == hipSuccess, dw_gate, dw_up, dw_down, st);
        if (err == hipSuccess) err = e2;
    } else {
        if (err == hipSuccess) err = wgrad_gate_up(p, WGUArgs{v, p.H, p.I, x, xc, dh, dw_gate, dw_up}, st);
        if (err == hipSuccess && !wd_launched) err = wgrad_down(p, wda, st);
        // the join also after an error: no fork is left open
        const hipError_t e2 = side_join(st, wd_side);
        if (err == hipSuccess) err = e2;
    }
    if (err == hipSuccess) err = hipGetLastError();
    return check_hip(err, "mok_backward");
}

}  // namespace mok

using mok::g_trace;

extern "C" mok_status mok_item_trace_enable(int32_t enable) {
    std::lock_guard<std::mutex> lk(g_trace.mu);
    if (!enable) {
        g_trace.on = false;
        return MOK_OK;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev != g_trace.device || !g_trace.rec)) {
        void *r = nullptr, *c = nullptr;
        e = hipGetSymbolAddress(&r, HIP_SYMBOL(mok::item_trace_records));
        if (e == hipSuccess) e = hipGetSymbolAddress(&c, HIP_SYMBOL(mok::item_trace_count));
        if (e == hipSuccess) {
            g_trace.rec = static_cast<mok_item_record *>(r);
            g_trace.count = static_cast<int *>(c);
            g_trace.device = dev;
        }
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemset(g_trace.count, 0, sizeof(int));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return mok::check_hip(e, "mok_item_trace_enable");
    g_trace.launch = 0;
    g_trace.on = true;
    return MOK_OK;
}

extern "C" mok_status mok_item_trace_read(mok_item_record *records, int32_t capacity, int32_t *count) {
    if (!count || capacity < 0 || (capacity > 0 && !records)) return MOK_ERROR_INVALID_VALUE;
    std::lock_guard<std::mutex> lk(g_trace.mu);
    if (!g_trace.count) {
        *count = 0;
        return MOK_OK;
    }
    int n = 0;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(&n, g_trace.count, sizeof(int), hipMemcpyDeviceToHost);
    const int copy = std::min(std::min(n, (int)MOK_ITEM_TRACE_CAPACITY), capacity);
    if (e == hipSuccess && copy > 0)
        e = hipMemcpy(records, g_trace.rec, sizeof(mok_item_record) * (size_t)copy, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return mok::check_hip(e, "mok_item_trace_read");
    *count = n;
    return MOK_OK;
}
