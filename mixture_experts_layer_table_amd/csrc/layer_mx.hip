// MXFP8 mode of the MoE layer ("Mixture-of-Kittens (MoK)" project summary,
// Overview: BF16 and MXFP8 precision modes; Key-concepts table: MXFP8 weights
// are pre-quantized). The four input-side GEMMs run on the block-scaled FP8
// MFMA; every operand is quantized along its contraction axis, 32 values per
// E8M0 scale:
//   forward gate/up   x rows (quantized by the ring gather) x W_gate^T | W_up^T
//   forward down      a (quantized in the gate/up epilogue from its fp32 value) x W_down^T
//   backward dA       dy rows (quantized by the ring gather) x W_down
//   backward dX       dh (quantized in the dA epilogue from its fp32 value) x W_gate | W_up
// h, y, dh (for the weight gradients), dx rows and all outputs stay bf16. The
// weight gradients run in BF16 (they have no weight operand), or, with
// MOK_MXFP8_WGRAD, on operands quantized along the token axis (below).
//
// Ring slot (MXFP8): elements [MB][H] then scales [MB][H/32]. a-ring slot
// (same slot stride as BF16, MB*I*2 bytes): elements [MB][I], scales [MB][I/32].
// Quantized dh: elements [R][2I], scales [R][2I/32], canonical row order.
#include "gemm8.h"
#include "layer_mx.h"
#include "layer_parts.h"
#include "mx_codec.h"
#include "persist.h"
#include "streams.h"

namespace mok {
namespace {

using CfgA = TileCfg<256, 256, 2, 4, 4>;
static_assert(CfgA::BN == kTileN, "host sizing assumes kTileN-column tiles");
using S8 = Fp8Stage<CfgA>;

__device__ __forceinline__ const uint16_t *as_pairs(const uint8_t *p) { return reinterpret_cast<const uint16_t *>(p); }

// ----------------------------------------------------------------------------- quantizing gather

// Dispatch copy of one row into the MXFP8 ring: one wave quantizes the row of
// processing position q = mb_start[g] + r along H into ring slot g % n_slots;
// lane c handles 8 values, 4 lanes form one 32-block.
struct GatherMx {
    SchedView v;
    int64_t n_slots;
    int MB, H, k;
    const uint16_t *src;
    uint8_t *ring;
    uint16_t *canon;   // optional: the bf16 rows at their canonical positions, [R][H]

    __device__ __forceinline__ void row(int g, int r) const {
        const int q = v.mb_start[g] + r;
        const int tok = v.perm[q] / k;
        uint4 *dc = canon ? reinterpret_cast<uint4 *>(canon + (int64_t)canon_pos(v, g, q) * H) : nullptr;
        const uint4 *s = reinterpret_cast<const uint4 *>(src + (int64_t)tok * H);
        uint8_t *slot = ring + (g % n_slots) * (int64_t)MB * (H + H / 32);
        uint8_t *el = slot + (int64_t)r * H;
        uint8_t *sc = slot + (int64_t)MB * H + (int64_t)r * (H / 32);
        // H % 128 == 0: whole 4-lane groups; 4 loads in flight per lane before encoding
        const int n = H / 8, lane = threadIdx.x & 63;
        for (int c0 = 0; c0 < n; c0 += 64 * 4) {
            uint4 t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + i * 64 + lane;
                t[i] = c < n ? s[c] : make_uint4(0, 0, 0, 0);
            }
            if (dc) {   // read only by the weight gradients, much later: kept out of the caches
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = c0 + i * 64 + lane;
                    if (c < n) store16_nt(dc + c, t[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + i * 64 + lane;
                if (c0 + i * 64 >= n) break;   // wave-uniform
                const uint32_t w[4] = {t[i].x, t[i].y, t[i].z, t[i].w};
                uint32_t amax = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) amax = max(amax, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
                amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));   // the 4 lanes of a 32-block
                amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
                const uint32_t sb = mx_scale_byte_bf16(amax);
                const int e = (int)sb - 127;
                uint32_t o[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) o[d] = e4m3x4_bf16(w[2 * d], w[2 * d + 1], e);
                if (c < n) {
                    *reinterpret_cast<uint2 *>(el + (int64_t)c * 8) = make_uint2(o[0], o[1]);
                    if ((c & 3) == 0) sc[c >> 2] = (uint8_t)sb;
                }
            }
        }
    }
};

__global__ __launch_bounds__(256) void gather_rows_mx(GatherMx ga, int g0) {
    if (*ga.v.status) return;
    const int g = g0 + blockIdx.y;
    const int r = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (ga.v.mb_start[g] + r >= ga.v.mb_start[g + 1]) return;
    ga.row(g, r);
}

// ----------------------------------------------------------------------------- epilogue quantization

// Quantize 16 fp32 values a lane holds of one 32-block (its partner lane
// l ^ 32 holds the other 16, columns g4*8 + 4*(l/32) + j of the block).
// Returns the scale byte and, in enc[g4], the 4 codes of columns
// g4*8 + 4h .. +3. Every lane of the wave must call this (cross-lane
// exchange). Kept out of line: epilogues call it up to 16 times, and inlining
// every copy would stop the accumulator loops from unrolling.
struct Block16 {
    float v[16];
};
struct Enc16 {
    uint32_t enc[4];
    uint32_t scale;
};
__device__ __attribute__((noinline)) Enc16 quantize_block16(Block16 b) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, __float_as_uint(b.v[i]) & 0x7FFFFFFFu);
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
    Enc16 r;
    r.scale = mx_scale_byte_f32(amax);
    const float sc = mx_pow2_neg((int)r.scale - 127);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
        r.enc[g4] = e4m3x2_scaled(b.v[g4 * 4] * sc, b.v[g4 * 4 + 1] * sc) |
                    (e4m3x2_scaled(b.v[g4 * 4 + 2] * sc, b.v[g4 * 4 + 3] * sc) << 16);
    return r;
}

// ----------------------------------------------------------------------------- forward gate/up

struct GateUp8Args {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int MB, H, I;
    const uint8_t *ring;                       // MXFP8 ring (x rows)
    const uint8_t *wg, *wgs, *wu, *wus;        // W_gate^T, W_up^T [E][I][H] and scales [E][I][H/32]
    uint16_t *h;                               // fwd_ctx h [R][2I] bf16, processing order
    uint8_t *aring;                            // a quantized along I
    const float *topk_w;
    uint16_t *ga;                              // fwd_ctx g * a [R][I] bf16, canonical order
};

template <class Cfg>
struct GateUp8 {
    using C = Cfg;
    using Args = GateUp8Args;
    static constexpr bool FP8 = true;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    ScaleLoader<C> sl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    SegTile t;
    int i0, nk;
    Args a;
    RowGates<C> rg;

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
        const int H = args.H, I = args.I;
        i0 = t.nt * (C::BN / 2);
        rg.load(t, wave_id() / C::WAVES_N, args.v, args.topk_w);   // hidden behind the K loop
        const uint8_t *slot = args.ring + t.slot * (int64_t)args.MB * (H + H / 32);
        xl.init(as_pairs(slot + (int64_t)t.rowoff * H), H / 2, t.mt.rows);
        const int64_t eo = (int64_t)t.mt.e * I * H + (int64_t)i0 * H;
        const int nw = min(C::BN / 2, I - i0);
        wl.init_split_rows(as_pairs(args.wg + eo), as_pairs(args.wu + eo), H / 2, nw);
        const int64_t so = (int64_t)t.mt.e * I * (H / 32) + (int64_t)i0 * (H / 32);
        sl.init(slot + (int64_t)args.MB * H + (int64_t)t.rowoff * (H / 32), t.mt.rows, H / 32, args.wgs + so, nw,
                H / 32, args.wus + so);
        nk = H / S8::BK8;
    }
    __device__ void issue(int kt, uint32_t stage) {
        sl.issue(kt, stage - (uint32_t)((kt % C::NSTAGE) * Fp8Stage<C>::BYTES));   // chunk first: see ScaleLoader
        xl.issue(kt * C::BK, stage);
        wl.issue(kt * C::BK, stage + C::X_BYTES);
    }
    // gate rows of the W tile pair with the up rows BN/2 further inside one wave
    __device__ int wrow(int wn, int fn) const {
        return fn < C::FN / 2 ? wn * (C::WN / 2) + fn * 32 : C::BN / 2 + wn * (C::WN / 2) + (fn - C::FN / 2) * 32;
    }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        constexpr size_t END = Fp8Stage<C>::LDS_BYTES;
        const int I = a.I;
        const int ib0 = i0 + wn * (C::WN / 2);
        if (ib0 >= I) return;   // I % 128 == 0: the wave's i are all valid or all past I
        rg.settle();
        // h rows (gate columns to h[.., i], up columns to h[.., I + i]) through LDS
        const uint32_t h_row = 4u * (uint32_t)I;
        const uint32_t h_col =
            2u * (uint32_t)(ib0 + (FragStage<C, END>::pass_col(epi_lane()) >= C::WN / 2 ? I - C::WN / 2 : 0));
        staged_rows<C, END>([&](int fm, int fn, int g4, int j) { return acc[fm][fn][g4 * 4 + j]; },
                            rows_rsrc(a.h + (int64_t)t.mt.q0 * 2 * I, (uint32_t)t.mt.rows * h_row),
                            [&](int fm, int r) -> uint32_t { return (uint32_t)(wm * C::WM + fm * 32 + r) * h_row + h_col; });
        // a, quantized along i (fp8 codes and one scale per 32-block, stored
        // directly), and g * a for the down weight gradient (the gate weight
        // times a rounded to bf16, as the BF16 forward feeds a to its down
        // GEMM), through the first half of each staged row
        using FS = FragStage<C, END>;
        const int lane = epi_lane();
        const uint32_t area = FS::area(wave_id(), 1);
        uint8_t *aslot = a.aring + t.slot * (int64_t)a.MB * I * 2;
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int m = wm * C::WM + fm * 32 + (lane & 31);
            const bool ok = m < t.mt.rows;   // same for lanes l and l ^ 32
            uint8_t *ael = aslot + (int64_t)(t.rowoff + m) * I;
            uint8_t *asc = aslot + (int64_t)a.MB * I + (int64_t)(t.rowoff + m) * (I / 32);
#pragma unroll
            for (int fn = 0; fn < C::FN / 2; ++fn) {
                const int ib = ib0 + fn * 32;   // one 32-block of i
                Block16 av;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    float gav[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float hg = acc[fm][fn][g4 * 4 + j], hu = acc[fm][fn + C::FN / 2][g4 * 4 + j];
                        av.v[g4 * 4 + j] = hg * sigmoidf_(hg) * hu;
                        gav[j] = rg.gw[fm] * bf16r(av.v[g4 * 4 + j]);
                    }
                    FS::put(area + FS::frag_off(fn, g4, lane),
                            make_uint2(pack_bf16x2(gav[0], gav[1]), pack_bf16x2(gav[2], gav[3])));
                }
                const Enc16 q8 = quantize_block16(av);
                if (ok) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        *reinterpret_cast<uint32_t *>(ael + ib + g4 * 8 + (lane >> 5) * 4) = q8.enc[g4];
                    if (lane < 32) asc[ib / 32] = (uint8_t)q8.scale;
                }
            }
#pragma unroll
            for (int p = 0; p < FS::PASSES; ++p) {
                const int mr = wm * C::WM + fm * 32 + FS::pass_row(p, lane);
                const int cc = FS::pass_col(lane);
                if (mr < t.mt.rows && cc < C::WN / 2)
                    store8_nt(a.ga + (int64_t)(t.mt.c0 + mr) * I + ib0 + cc, FS::get(area + FS::pass_off(p, lane)));
            }
        }
    }
};

// ----------------------------------------------------------------------------- forward down

struct Down8Args {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int MB, H, I, k, MT, nb_full;
    const uint8_t *aring;
    const uint8_t *wd, *wds;                   // W_down^T [E][H][I] and scales [E][H][I/32]
    const float *topk_w;
    uint16_t *out, *stage;
};

template <class Cfg>
struct Down8 {
    using C = Cfg;
    using Args = Down8Args;
    static constexpr bool FP8 = true;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    ScaleLoader<C> sl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    SegTile t;
    int n0, nk;
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
        const int H = args.H, I = args.I;
        n0 = t.nt * C::BN;
        const uint8_t *aslot = args.aring + t.slot * (int64_t)args.MB * I * 2;
        xl.init(as_pairs(aslot + (int64_t)t.rowoff * I), I / 2, t.mt.rows);
        const int nw = min(C::BN, H - n0);
        wl.init(as_pairs(args.wd + (int64_t)t.mt.e * H * I + (int64_t)n0 * I), I / 2, nw);
        sl.init(aslot + (int64_t)args.MB * I + (int64_t)t.rowoff * (I / 32), t.mt.rows, I / 32,
                args.wds + (int64_t)t.mt.e * H * (I / 32) + (int64_t)n0 * (I / 32), nw, I / 32);
        nk = I / S8::BK8;
    }
    __device__ void issue(int kt, uint32_t stage) {
        sl.issue(kt, stage - (uint32_t)((kt % C::NSTAGE) * Fp8Stage<C>::BYTES));   // chunk first: see ScaleLoader
        xl.issue(kt * C::BK, stage);
        wl.issue(kt * C::BK, stage + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        store_token_rows<C, Fp8Stage<C>::LDS_BYTES>(acc, t, n0, wm, wn, a.v, a.H, a.k, a.MT, a.nb_full, a.topk_w, true, a.out, a.stage);
    }
};

// ----------------------------------------------------------------------------- backward dA

struct DA8Args {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int MB, H, I, S;
    const uint8_t *ring;                       // MXFP8 ring (dy rows)
    const uint8_t *wd, *wds;                   // W_down [E][I][H] and scales [E][I][H/32]
    const uint16_t *h;
    const float *topk_w;
    uint16_t *dh;
    float *dgp;
    uint8_t *dhq, *dhqs;
};

template <class Cfg>
struct DA8 {
    using C = Cfg;
    using Args = DA8Args;
    static constexpr bool FP8 = true;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    ScaleLoader<C> sl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    SegTile t;
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
        const int H = args.H, I = args.I;
        i0 = t.nt * C::BN;
        const uint8_t *slot = args.ring + t.slot * (int64_t)args.MB * (H + H / 32);
        xl.init(as_pairs(slot + (int64_t)t.rowoff * H), H / 2, t.mt.rows);
        const int nw = min(C::BN, I - i0);
        wl.init(as_pairs(args.wd + (int64_t)t.mt.e * I * H + (int64_t)i0 * H), H / 2, nw);
        sl.init(slot + (int64_t)args.MB * H + (int64_t)t.rowoff * (H / 32), t.mt.rows, H / 32,
                args.wds + (int64_t)t.mt.e * I * (H / 32) + (int64_t)i0 * (H / 32), nw, H / 32);
        nk = H / S8::BK8;
    }
    __device__ void issue(int kt, uint32_t stage) {
        sl.issue(kt, stage - (uint32_t)((kt % C::NSTAGE) * Fp8Stage<C>::BYTES));   // chunk first: see ScaleLoader
        xl.issue(kt * C::BK, stage);
        wl.issue(kt * C::BK, stage + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        const int lane = threadIdx.x & 63;
        const int I = a.I;
        const int slice = t.nt * C::WAVES_N + wn;
        const int ib0 = i0 + wn * C::WN;
        if (ib0 >= I) return;   // I % 128 == 0: a wave's 64 columns are all valid or none
        int q[C::FM];
        bool ok[C::FM];
        float gw[C::FM];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int m = wm * C::WM + fm * 32 + (lane & 31);
            ok[fm] = m < t.mt.rows;
            q[fm] = t.mt.q0 + (ok[fm] ? m : 0);
        }
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) gw[fm] = a.topk_w[a.v.perm[q[fm]]];
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            // one batch per fragment: loading the next one ahead of this fragment's stores measured slower
            HBatch<C> h;
            h.load(a.h + (int64_t)q[fm] * 2 * I, I, ib0, lane);
            const int m = wm * C::WM + fm * 32 + (lane & 31);
            const int64_t c = t.mt.c0 + (ok[fm] ? m : 0);   // dh rows are kept in canonical order
            uint16_t *dhrow = a.dh + c * 2 * I;
            uint8_t *qrow = a.dhq + c * 2 * I;
            uint8_t *srow = a.dhqs + c * (2 * I / 32);
            float dg = 0.0f;
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) {
                const int ib = ib0 + fn * 32;   // one 32-block of i
                Block16 dhg, dhu;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int i = ib + g4 * 8 + (lane >> 5) * 4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float G = acc[fm][fn][g4 * 4 + j];
                        const float hg = bf16_at(h.g[fn][g4], j), hu = bf16_at(h.u[fn][g4], j);
                        const float s = sigmoidf_(hg);
                        const float sl_ = hg * s;
                        const float av = sl_ * hu;
                        dg += G * av;
                        const float da = gw[fm] * G;
                        dhu.v[g4 * 4 + j] = da * sl_;
                        dhg.v[g4 * 4 + j] = da * hu * s * (1.0f + hg * (1.0f - s));
                    }
                    if (ok[fm]) {
                        store4_bf16(dhrow + i, dhg.v[g4 * 4], dhg.v[g4 * 4 + 1], dhg.v[g4 * 4 + 2], dhg.v[g4 * 4 + 3]);
                        store4_bf16(dhrow + I + i, dhu.v[g4 * 4], dhu.v[g4 * 4 + 1], dhu.v[g4 * 4 + 2],
                                    dhu.v[g4 * 4 + 3]);
                    }
                }
                const Enc16 qg = quantize_block16(dhg);
                const Enc16 qu = quantize_block16(dhu);
                if (ok[fm]) {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int i = ib + g4 * 8 + (lane >> 5) * 4;
                        *reinterpret_cast<uint32_t *>(qrow + i) = qg.enc[g4];
                        *reinterpret_cast<uint32_t *>(qrow + I + i) = qu.enc[g4];
                    }
                    if (lane < 32) {
                        srow[ib / 32] = (uint8_t)qg.scale;
                        srow[(I + ib) / 32] = (uint8_t)qu.scale;
                    }
                }
            }
            // lanes l and l ^ 32 hold the same row: lower half + upper half, fixed order
            const float other = __shfl_xor(dg, 32);
            const float tot = (lane < 32) ? dg + other : other + dg;
            if (ok[fm] && lane < 32) a.dgp[(int64_t)q[fm] * a.S + slice] = tot;
        }
    }
};

// ----------------------------------------------------------------------------- backward dX

struct DX8Args {
    SchedView v;
    int g0, g1, n_tiles;
    int64_t n_slots;
    int H, I, k, MT, nb_full;
    const uint8_t *dhq, *dhqs;
    const uint8_t *wg, *wgs, *wu, *wus;        // W_gate, W_up [E][H][I] and scales [E][H][I/32]
    uint16_t *dx, *stage;
};

template <class Cfg>
struct DX8 {
    using C = Cfg;
    using Args = DX8Args;
    static constexpr bool FP8 = true;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    ScaleLoader<C> sl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    SegTile t;
    int n0, nk;
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
        const int H = args.H, I = args.I;
        n0 = t.nt * C::BN;
        xl.init(as_pairs(args.dhq + (int64_t)t.mt.c0 * 2 * I), I, t.mt.rows);   // 2I bytes = I byte pairs
        const int nw = min(C::BN, H - n0);
        const int64_t wo = (int64_t)t.mt.e * H * I + (int64_t)n0 * I;
        wl.init(as_pairs(args.wg + wo), I / 2, nw, as_pairs(args.wu + wo), I / 2);
        const int64_t so = (int64_t)t.mt.e * H * (I / 32) + (int64_t)n0 * (I / 32);
        sl.init(args.dhqs + (int64_t)t.mt.c0 * (2 * I / 32), t.mt.rows, 2 * I / 32, args.wgs + so, nw, I / 32, nullptr,
                args.wus + so, I);
        nk = 2 * I / S8::BK8;
    }
    __device__ void issue(int kt, uint32_t stage) {
        sl.issue(kt, stage - (uint32_t)((kt % C::NSTAGE) * Fp8Stage<C>::BYTES));   // chunk first: see ScaleLoader
        xl.issue(kt * C::BK, stage);
        wl.issue(kt * C::BK, stage + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        store_token_rows<C, Fp8Stage<C>::LDS_BYTES>(acc, t, n0, wm, wn, a.v, a.H, a.k, a.MT, a.nb_full, nullptr, false, a.dx, a.stage);
    }
};

// ----------------------------------------------------------------------------- MXFP8 weight gradients
//
// dW_gate | dW_up [e] = X_e^T [dh_g | dh_u] and dW_down[e] = (g a)_e^T dY_e contract
// over the expert's rows, so both operands are quantized along that axis:
// 32 consecutive rows of one expert (canonical order) per column share one
// E8M0 scale. The quantizer writes them transposed, [column][Kp] (K = rows
// contiguous, as the block-scaled tile reads both operands), expert e's rows
// at [po[e], po[e] + count) and zeros up to po[e+1] = po[e] + count rounded
// up to 128 (the tile's K step for whole scale dwords).

// po[e] = sum over f < e of counts[f] rounded up to 128; one workgroup.
__global__ __launch_bounds__(256) void wq_offsets(SchedView v, int32_t *po) {
    if (*v.status) return;
    __shared__ int32_t part[256];
    const int E = v.E, per = (E + 255) / 256, t = threadIdx.x;
    const int e0 = min(E, t * per), e1 = min(E, e0 + per);
    int32_t sum = 0;
    for (int e = e0; e < e1; ++e) sum += (v.counts[e] + 127) / 128 * 128;
    part[t] = sum;
    __syncthreads();
    if (t == 0) {   // 256 partial sums, serially: fixed order
        int32_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int32_t x = part[i];
            part[i] = run;
            run += x;
        }
    }
    __syncthreads();
    int32_t run = part[t];
    for (int e = e0; e < e1; ++e) {
        po[e] = run;
        run += (v.counts[e] + 127) / 128 * 128;
    }
    if (e1 == E && e0 < e1) po[E] = run;   // the thread holding the last expert
}

struct QuantCols {
    SchedView v;
    const int32_t *po;
    const uint16_t *src;   // bf16 rows: token rows (by_token) or canonical rows
    int64_t ld;            // elements per source row
    int ncols;
    bool by_token;
    int64_t Kp;
    uint8_t *el, *sc;      // [ncols][Kp] codes, [ncols][Kp/32] scale bytes
};

// Workgroup (j, column chunk): padded positions [128j, 128j + 128) (one
// expert's, as po is a multiple of 128) of 64 columns. The 128 x 64 source
// tile is read in 16-byte chunks (4 loads in flight per thread) into LDS;
// thread (c, b) then quantizes column c's 32-row block b and leaves its 32
// code bytes in an LDS row of 33 dwords per column (conflict-free); last,
// every 8 consecutive threads write one column's 128 code bytes as 16-byte
// stores.
constexpr int kQRows = 128, kQCols = 64;
__global__ __launch_bounds__(256) void quantize_cols(QuantCols q) {
    if (*q.v.status) return;
    __shared__ int32_t rows[kQRows];
    __shared__ __attribute__((aligned(16))) uint16_t tile[kQRows][kQCols];
    __shared__ uint32_t codes[kQCols][33];
    const int64_t p0 = (int64_t)blockIdx.x * kQRows;
    const int E = q.v.E;
    if (p0 >= q.po[E]) return;   // past every expert's padded rows: never read
    int lo = 0, hi = E;          // the expert e with po[e] <= p0 < po[e+1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (q.po[mid] <= p0) lo = mid;
        else hi = mid;
    }
    const int e = lo;
    const int r0 = (int)(p0 - q.po[e]), n = q.v.counts[e] - r0;   // valid rows here: min(128, n)
    const int t = threadIdx.x;
    if (t < kQRows) {
        int row = -1;
        if (t < n) {
            const int c = q.v.offsets[e] + r0 + t;
            row = q.by_token ? q.v.ctok[c] : c;
        }
        rows[t] = row;
    }
    __syncthreads();
    const int col0 = blockIdx.y * kQCols;
    constexpr int CPR = kQCols / 8;           // 16-byte chunks per tile row
    constexpr int RPP = 256 / CPR;            // rows per pass
    uint4 v[kQRows / RPP];
#pragma unroll
    for (int pass = 0; pass < kQRows / RPP; ++pass) {
        const int r = pass * RPP + t / CPR, ch = (t % CPR) * 8;
        const int row = rows[r];
        v[pass] = make_uint4(0, 0, 0, 0);
        if (row >= 0 && col0 + ch < q.ncols)   // ncols % 128 == 0: whole chunks
            v[pass] = *reinterpret_cast<const uint4 *>(q.src + (int64_t)row * q.ld + col0 + ch);
    }
#pragma unroll
    for (int pass = 0; pass < kQRows / RPP; ++pass)
        *reinterpret_cast<uint4 *>(&tile[pass * RPP + t / CPR][(t % CPR) * 8]) = v[pass];
    __syncthreads();
#pragma unroll
    for (int cb = t; cb < kQCols * 4; cb += 256) {
        const int c = cb % kQCols, b = cb / kQCols;
        uint32_t x[32];
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            x[i] = tile[b * 32 + i][c];
            amax = max(amax, x[i] & 0x7FFFu);
        }
        const uint32_t sb = mx_scale_byte_bf16(amax);
        const int ex = (int)sb - 127;
#pragma unroll
        for (int d = 0; d < 8; ++d)
            codes[c][b * 8 + d] = e4m3x4_bf16(x[4 * d] | (x[4 * d + 1] << 16), x[4 * d + 2] | (x[4 * d + 3] << 16), ex);
        if (col0 + c < q.ncols) q.sc[(int64_t)(col0 + c) * (q.Kp / 32) + p0 / 32 + b] = (uint8_t)sb;
    }
    __syncthreads();
#pragma unroll
    for (int i = t; i < kQCols * 8; i += 256) {
        const int c = i >> 3, ch = i & 7;
        if (col0 + c < q.ncols) {
            const uint4 w = make_uint4(codes[c][ch * 4], codes[c][ch * 4 + 1], codes[c][ch * 4 + 2],
                                       codes[c][ch * 4 + 3]);
            *reinterpret_cast<uint4 *>(q.el + (int64_t)(col0 + c) * q.Kp + p0 + ch * 16) = w;
        }
    }
}

// dW_gate | dW_up [e]: M = H (x columns), N = 2I (dh columns), K = the expert's padded rows.
struct WGU8Args {
    SchedView v;
    int H, I;
    int64_t Kp;
    const int32_t *po;
    const uint8_t *qx, *qxs, *qdh, *qdhs;
    uint16_t *dwg, *dwu;
};

template <class Cfg>
struct WGU8 {
    using C = Cfg;
    using Args = WGU8Args;
    static constexpr bool FP8 = true;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    ScaleLoader<C> sl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    int e, h0, n0, nk;
    Args a;

    __device__ bool setup(const Args &args, Blk b) {
        if (*args.v.status) return false;
        a = args;
        wgrad_tile(args.v, b.x, (2 * args.I + C::BN - 1) / C::BN, (args.H + C::BM - 1) / C::BM, e, h0, n0);
        h0 *= C::BM;
        n0 *= C::BN;
        const int pe = args.po[e], kpe = args.po[e + 1] - pe;   // a multiple of 128
        nk = kpe / Fp8Stage<C>::BK8;
        const int64_t Kp = args.Kp, kb = Kp / 32;
        const int mx = min(C::BM, args.H - h0), mw = min(C::BN, 2 * args.I - n0);
        xl.init(as_pairs(args.qx + (int64_t)h0 * Kp + pe), Kp / 2, mx);
        wl.init(as_pairs(args.qdh + (int64_t)n0 * Kp + pe), Kp / 2, mw);
        sl.init(args.qxs + (int64_t)h0 * kb + pe / 32, mx, (int)kb, args.qdhs + (int64_t)n0 * kb + pe / 32, mw,
                (int)kb);
        return true;
    }
    __device__ void issue(int kt, uint32_t stage) {
        sl.issue(kt, stage - (uint32_t)((kt % C::NSTAGE) * Fp8Stage<C>::BYTES));   // chunk first: see ScaleLoader
        xl.issue(kt * C::BK, stage);
        wl.issue(kt * C::BK, stage + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        const int H = a.H, I = a.I;
        const int nb = n0 + wn * C::WN;
        if (nb >= 2 * I) return;   // I % 128 == 0: the wave's columns are all gate, all up or all past 2I
        uint16_t *base = (nb < I ? a.dwg + nb : a.dwu + (nb - I)) + (int64_t)e * H * I;   // expert e's rows
        staged_rows<C, Fp8Stage<C>::LDS_BYTES>([&](int fm, int fn, int g4, int j) { return acc[fm][fn][g4 * 4 + j]; },
                                               rows_rsrc(base, 2u * (uint32_t)H * (uint32_t)I),
                                               [&](int fm, int r) -> uint32_t {
                                                   return 2u * (uint32_t)(h0 + wm * C::WM + fm * 32 + r) * (uint32_t)I;
                                               });
    }
};

// dW_down[e]: M = I (g*a columns), N = H (dy columns), K as above.
struct WD8Args {
    SchedView v;
    int H, I;
    int64_t Kp;
    const int32_t *po;
    const uint8_t *qga, *qgas, *qdy, *qdys;
    uint16_t *dwd;
};

template <class Cfg>
struct WD8 {
    using C = Cfg;
    using Args = WD8Args;
    static constexpr bool FP8 = true;
    RowLoader<C, C::BM> xl;
    RowLoader<C, C::BN> wl;
    ScaleLoader<C> sl;
    static constexpr int LOADS_PER_STAGE = RowLoader<C, C::BM>::IPW + RowLoader<C, C::BN>::IPW;
    int e, i0, n0, nk;
    Args a;

    __device__ bool setup(const Args &args, Blk b) {
        if (*args.v.status) return false;
        a = args;
        wgrad_tile(args.v, b.x, (args.H + C::BN - 1) / C::BN, (args.I + C::BM - 1) / C::BM, e, i0, n0);
        i0 *= C::BM;
        n0 *= C::BN;
        const int pe = args.po[e], kpe = args.po[e + 1] - pe;
        nk = kpe / Fp8Stage<C>::BK8;
        const int64_t Kp = args.Kp, kb = Kp / 32;
        const int mx = min(C::BM, args.I - i0), mw = min(C::BN, args.H - n0);
        xl.init(as_pairs(args.qga + (int64_t)i0 * Kp + pe), Kp / 2, mx);
        wl.init(as_pairs(args.qdy + (int64_t)n0 * Kp + pe), Kp / 2, mw);
        sl.init(args.qgas + (int64_t)i0 * kb + pe / 32, mx, (int)kb, args.qdys + (int64_t)n0 * kb + pe / 32, mw,
                (int)kb);
        return true;
    }
    __device__ void issue(int kt, uint32_t stage) {
        sl.issue(kt, stage - (uint32_t)((kt % C::NSTAGE) * Fp8Stage<C>::BYTES));   // chunk first: see ScaleLoader
        xl.issue(kt * C::BK, stage);
        wl.issue(kt * C::BK, stage + C::X_BYTES);
    }
    __device__ int wrow(int wn, int fn) const { return wn * C::WN + fn * 32; }
    __device__ void epilogue(f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
        const int H = a.H, I = a.I;
        const int nb = n0 + wn * C::WN;
        if (nb >= H) return;   // H % 128 == 0
        staged_rows<C, Fp8Stage<C>::LDS_BYTES>([&](int fm, int fn, int g4, int j) { return acc[fm][fn][g4 * 4 + j]; },
                                               rows_rsrc(a.dwd + (int64_t)e * I * H + nb, 2u * (uint32_t)I * (uint32_t)H),
                                               [&](int fm, int r) -> uint32_t {
                                                   return 2u * (uint32_t)(i0 + wm * C::WM + fm * 32 + r) * (uint32_t)H;
                                               });
    }
};

// ----------------------------------------------------------------------------- host side

template <class P>
hipError_t launch_gemm8(const char *name, dim3 grid, const typename P::Args &args, hipStream_t st) {
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm8_kernel<P>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)S8::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
    KernelTimer tm(name, st);
    gemm8_kernel<P><<<grid, CfgA::NT, S8::LDS_BYTES, st>>>(args);
    return hipGetLastError();
}

}  // namespace

hipError_t mx_forward_round(const Plan &p, const SchedView &v, int g0, int g1, int64_t mt_bound,
                            const uint16_t *x, const mok_weights &w, char *ws, uint16_t *h, uint16_t *ga_rows,
                            uint16_t *xc, const float *topk_w, uint16_t *out, uint16_t *stage, hipStream_t st) {
    uint8_t *ring = reinterpret_cast<uint8_t *>(ws + p.w_ring);
    uint8_t *aring = reinterpret_cast<uint8_t *>(ws + p.w_aring);
    {
        const dim3 sgrid((unsigned)ceil_div(p.MB, kRowsPerBlock), (unsigned)(g1 - g0));
        KernelTimer tm("gather", st);
        gather_rows_mx<<<sgrid, 256, 0, st>>>(GatherMx{v, p.n_slots, p.MB, p.H, p.k, x, ring, xc}, g0);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int ntg = (int)ceil_div(p.I, CfgA::BN / 2), ntd = (int)ceil_div(p.H, CfgA::BN);
    GateUp8Args ga{v, g0, g1, ntg, p.n_slots, p.MB, p.H, p.I, ring, w.gate_elems, w.gate_scales,
                   w.up_elems, w.up_scales, h, aring, topk_w, ga_rows};
    Down8Args da{v, g0, g1, ntd, p.n_slots, p.MB, p.H, p.I, p.k, (int)p.MT, p.nb_full, aring,
                 w.down_elems, w.down_scales, topk_w, out, stage};
    if (p.debug & MOK_DEBUG_SEPARATE_LAUNCHES) {
        if ((err = launch_gemm8<GateUp8<CfgA>>("gateup", seg_grid(ntg, mt_bound), ga, st)) != hipSuccess) return err;
        return launch_gemm8<Down8<CfgA>>("down", seg_grid(ntd, mt_bound), da, st);
    }
    // The persistent pair kernel of the BF16 rounds, with block-scaled tiles
    // (241 registers, no spills): down tiles fill the gate/up launch's last
    // partial wave, which the ragged m-tiles of skewed loads leave large
    // (EP-64 share, Zipf: 0.99 -> 0.87 ms for both GEMMs).
    return launch_pair<GateUp8<CfgA>, Down8<CfgA>, S8::LDS_BYTES>(
        "fwd_gemms", ga, da, reinterpret_cast<int *>(ws + p.w_sync), p.max_mtiles, spin_limit(p),
        persistent_grid(p), st, item_trace_args(MOK_TRACE_FWD_GEMMS));
}

hipError_t mx_gather_dy(const Plan &p, const SchedView &v, int g0, int g1, const uint16_t *dy, char *ws,
                        uint16_t *dyc, hipStream_t st) {
    uint8_t *ring = reinterpret_cast<uint8_t *>(ws + p.w_ring);
    const dim3 sgrid((unsigned)ceil_div(p.MB, kRowsPerBlock), (unsigned)(g1 - g0));
    KernelTimer tm("gather_dy", st);
    gather_rows_mx<<<sgrid, 256, 0, st>>>(GatherMx{v, p.n_slots, p.MB, p.H, p.k, dy, ring, dyc}, g0);
    return hipGetLastError();
}

hipError_t mx_backward_gemms(const Plan &p, const SchedView &v, int g0, int g1, int64_t mt_bound,
                             const mok_weights &w, char *ws, const uint16_t *h, const float *topk_w, uint16_t *dx,
                             uint16_t *stage, hipStream_t st) {
    uint8_t *ring = reinterpret_cast<uint8_t *>(ws + p.w_ring);
    uint16_t *dh = reinterpret_cast<uint16_t *>(ws + p.w_dh);
    float *dgp = reinterpret_cast<float *>(ws + p.w_dgp);
    uint8_t *dhq = reinterpret_cast<uint8_t *>(ws + p.w_dhq);
    uint8_t *dhqs = reinterpret_cast<uint8_t *>(ws + p.w_dhq_scales);
    hipError_t err;
    const int nta = (int)ceil_div(p.I, CfgA::BN), ntx = (int)ceil_div(p.H, CfgA::BN);
    DA8Args aa{v, g0, g1, nta, p.n_slots, p.MB, p.H, p.I, p.dg_slices, ring, w.down_elems, w.down_scales, h,
               topk_w, dh, dgp, dhq, dhqs};
    DX8Args xa{v, g0, g1, ntx, p.n_slots, p.H, p.I, p.k, (int)p.MT, p.nb_full, dhq, dhqs, w.gate_elems,
               w.gate_scales, w.up_elems, w.up_scales, dx, stage};
    // Separate launches: dW_down, on the side stream, fills dA's last partial
    // wave (528 tiles are 2.06 waves at the EP-64 share). In the persistent
    // pair (71 registers spilled around DA8's epilogue) dA + dX ran faster,
    // 1.13 against 1.36 ms, but dW_down then ran beside dW_gate | dW_up
    // instead: the step 2-6% slower.
    if ((err = launch_gemm8<DA8<CfgA>>("dA", seg_grid(nta, mt_bound), aa, st)) != hipSuccess) return err;
    return launch_gemm8<DX8<CfgA>>("dX", seg_grid(ntx, mt_bound), xa, st);
}

namespace {

// which: 0 x, 1 dh, 2 g * a (ga), 3 dy
QuantCols quant_cols(const Plan &p, const SchedView &v, char *ws, int which, const uint16_t *x,
                     const uint16_t *dy, const uint16_t *ga = nullptr) {
    int32_t *po = reinterpret_cast<int32_t *>(ws + p.w_po);
    auto B = [&](size_t off) { return reinterpret_cast<uint8_t *>(ws + off); };
    switch (which) {
    case 0: return QuantCols{v, po, x, p.H, p.H, true, p.Kp, B(p.w_qx), B(p.w_qxs)};
    case 1: return QuantCols{v, po, reinterpret_cast<const uint16_t *>(ws + p.w_dh), 2 * (int64_t)p.I, 2 * p.I,
                             false, p.Kp, B(p.w_qdh), B(p.w_qdhs)};
    case 2: return QuantCols{v, po, ga, p.I, p.I, false, p.Kp, B(p.w_qga), B(p.w_qgas)};
    default: return QuantCols{v, po, dy, p.H, p.H, true, p.Kp, B(p.w_qdy), B(p.w_qdys)};
    }
}

void launch_quant(const QuantCols &q, const Plan &p, const char *name, hipStream_t st) {
    KernelTimer tm(name, st);
    quantize_cols<<<dim3((unsigned)(p.Kp / kQRows), (unsigned)ceil_div(q.ncols, kQCols)), 256, 0, st>>>(q);
}

}  // namespace

hipError_t mx_wgrad_begin(const Plan &p, const SchedView &v, char *ws, const uint16_t *x, const uint16_t *dy,
                          hipStream_t st, hipStream_t *side) {
    *side = st;
    if (p.R == 0) {   // every count is 0: po all 0, so each weight-gradient tile has K = 0 and writes zeros
        KernelTimer tm("wq_offsets", st);
        wq_offsets<<<1, 256, 0, st>>>(v, reinterpret_cast<int32_t *>(ws + p.w_po));
        return hipGetLastError();
    }
    // x and dy are inputs: their quantizers run beside the backward rounds,
    // which are bound by the matrix cores while the quantizers are bound by memory
    const hipStream_t q = side_fork(st);
    *side = q;
    {
        KernelTimer tm("wq_offsets", q);
        wq_offsets<<<1, 256, 0, q>>>(v, reinterpret_cast<int32_t *>(ws + p.w_po));
    }
    launch_quant(quant_cols(p, v, ws, 0, x, dy), p, "wgrad_quantize_x_dy", q);
    launch_quant(quant_cols(p, v, ws, 3, x, dy), p, "wgrad_quantize_x_dy", q);
    return hipGetLastError();
}

hipError_t mx_wgrad_finish(const Plan &p, const SchedView &v, char *ws, const uint16_t *ga, hipStream_t side,
                           bool compute, uint16_t *dw_gate, uint16_t *dw_up, uint16_t *dw_down, hipStream_t st) {
    hipError_t err = side_join(st, side);
    if (err != hipSuccess || !compute) return err;
    if (p.R > 0) {
        launch_quant(quant_cols(p, v, ws, 1, nullptr, nullptr), p, "wgrad_quantize_dh_ga", st);
        launch_quant(quant_cols(p, v, ws, 2, nullptr, nullptr, ga), p, "wgrad_quantize_dh_ga", st);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    auto B = [&](size_t off) { return reinterpret_cast<uint8_t *>(ws + off); };
    const int32_t *po = reinterpret_cast<const int32_t *>(ws + p.w_po);
    const WGU8Args gu{v, p.H, p.I, p.Kp, po, B(p.w_qx), B(p.w_qxs), B(p.w_qdh), B(p.w_qdhs), dw_gate, dw_up};
    const WD8Args wd{v, p.H, p.I, p.Kp, po, B(p.w_qga), B(p.w_qgas), B(p.w_qdy), B(p.w_qdys), dw_down};
    err = launch_gemm8<WGU8<CfgA>>(
        "wgrad_gate_up", dim3((unsigned)(ceil_div(2 * p.I, CfgA::BN) * ceil_div(p.H, CfgA::BM) * p.E)), gu, st);
    if (err != hipSuccess) return err;
    return launch_gemm8<WD8<CfgA>>(
        "wgrad_down", dim3((unsigned)(ceil_div(p.H, CfgA::BN) * ceil_div(p.I, CfgA::BM) * p.E)), wd, st);
}

}  // namespace mok
