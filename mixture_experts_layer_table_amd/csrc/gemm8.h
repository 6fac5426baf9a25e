// Block-scaled FP8 tile GEMM for gfx950 (MXFP8: E4M3 elements, one E8M0 scale
// per 32 contiguous values along K), on v_mfma_scale_f32_32x32x64_f8f6f4.
//
// Same data path as the bf16 core in gemm.h: direct-to-LDS buffer loads into
// an NSTAGE-deep ring, Row tiles of 64-byte rows with 16-byte chunks
// swizzled, so one stage holds K = 64 fp8 values per row (the bytes of a
// K = 32 bf16 stage; the byte-row loaders of gemm.h are reused by viewing fp8
// rows as rows of byte pairs). Both operands are K-contiguous: the caller
// provides weights quantized along K in the orientation each GEMM needs.
//
// Scales: per stage each tile row needs the scale bytes of its two 32-blocks.
// Scale rows are [rows][K/32] bytes, so the bytes of consecutive blocks of a
// row are contiguous: they are loaded a chunk of CB blocks at a time (16
// bytes, 8 stages, where the rows allow 16-byte loads; else 4 bytes, K a
// multiple of 128), one row per lane, into chunk buffers after the operand
// stages (X rows by waves 0-3, W rows by waves 4-7, one load per wave on
// the first stage of each chunk). Loading every stage's two bytes per row
// would cost one memory request per row and stage, as many as the operand
// rows themselves, for a 32nd of the bytes.
//
// MFMA operand layout (measured): lane l supplies 32 bytes of row l%32; its
// bytes 0..15 belong to K-block 0 and bytes 16..31 to K-block 1 of the
// 64-wide step, and the scale of (row r, block b) is taken from lane r + 32b.
// Here lane half h = l/32 supplies 16-byte chunk h of block 0 (tile chunk h)
// and chunk h of block 1 (tile chunk 2 + h), and the scale of block h.
#pragma once
#include <type_traits>

#include "gemm.h"

namespace mok {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <class C>
struct Fp8Stage {
    static_assert(C::BM == 256 && C::BN == 256 && C::NW == 8, "scale loads assume 256 x 256 tiles, 8 waves");
    static constexpr int BYTES = C::STAGE_BYTES;
    static constexpr int NSCBUF = 3;                         // scale chunk buffers per operand (see ScaleLoader)
    static constexpr int SCBUF_BYTES = 256 * 16;             // one chunk: [256 rows][CB <= 16 bytes]
    static constexpr int SC_OFF = C::NSTAGE * BYTES;         // X chunk buffers, then W chunk buffers
    static constexpr size_t LDS_BYTES = (size_t)SC_OFF + 2 * NSCBUF * SCBUF_BYTES;
    static constexpr int BK8 = 64;                           // fp8 values per row and stage
};

// Scale chunks of one operand's 256 tile rows. Blocks are counted from the
// start of the source array they come from (a W operand may switch arrays at
// K = ksplit); chunk q of a source holds its blocks [CB q, CB q + CB), and
// chunks are numbered in K order across sources (seq), each in buffer
// seq % NSCBUF. The chunk is loaded with the operand loads of its first
// stage, ahead of them, so the wait for that stage covers it.
//
// Buffer reuse: chunk seq + NSCBUF overwrites chunk seq's buffer. Its load
// goes out with the loads of stage y = (first stage of chunk seq + NSCBUF),
// at the earliest after barrier y - 4 (group 1 issues stage y at the start of
// iteration y - 3, group 0 after barrier y - 3), and every read of stage x
// has landed before barrier x. So chunk seq's last stage must be at most
// y - 4: the NSCBUF - 1 = 2 chunks in between must span at least 3 stages.
// A full chunk spans CB / 2 >= 2 stages; only the last chunk of the first
// source (a W operand switching arrays) can be shorter, at least 1 stage,
// and never two of those in a row: 2 + 1 >= 3.
struct ScaleChunk {
    uint32_t seq, pos;   // chunk number, and block of the stage's first 32-block inside it
};
template <class C>
struct ScaleLoader {
    rsrc_t res, res2;
    uint32_t voff;   // byte offset of the lane's row in its source
    int ksplit;      // K (elements) from which res2 holds the blocks, at K - ksplit
    int cbx, cbw;    // blocks per chunk of the X and the W operand (16 or 4)
    int nq0w;        // W chunks of source 0 (before ksplit)

    // x/w: scale rows of the X / W operand ([rows][kbx or kbw] bytes, kb = K/32
    // of that array), nx/nw valid rows. w_hi: W rows [BN/2, BN) come from w_hi
    // instead (row - BN/2), each half with nw valid rows. w2: W blocks for
    // K >= wsplit come from w2, at K - wsplit.
    __device__ void init(const uint8_t *x, int nx, int kbx, const uint8_t *w, int nw, int kbw,
                         const uint8_t *w_hi = nullptr, const uint8_t *w2 = nullptr, int wsplit = 1 << 30) {
        const int wave = wave_id(), L = threadIdx.x & 63;
        const bool is_w = wave >= 4;
        int r = (wave & 3) * 64 + L;
        const uint8_t *base = x;
        int n = nx, kb = kbx;
        if (is_w) {
            base = w;
            n = nw;
            kb = kbw;
            if (w_hi && r >= C::BN / 2) {
                base = w_hi;
                r -= C::BN / 2;
            }
        }
        const uint32_t bytes = (uint32_t)((int64_t)max(n, 0) * kb);
        res = make_rsrc(base, bytes);
        res2 = make_rsrc(is_w && w2 ? w2 : base, bytes);
        ksplit = w2 ? wsplit : (1 << 30);
        voff = (uint32_t)r * (uint32_t)kb;
        // 16-byte chunks where every row of every source starts 16-byte aligned
        auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
        cbx = (kbx % 16 == 0 && a16(x)) ? 16 : 4;
        cbw = (kbw % 16 == 0 && a16(w) && (!w_hi || a16(w_hi)) && (!w2 || a16(w2))) ? 16 : 4;
        nq0w = w2 ? (wsplit / 32 + cbw - 1) / cbw : 0;
    }
    __device__ __forceinline__ ScaleChunk chunk_x(int kt) const {
        const uint32_t b = (uint32_t)kt * 2u;
        return ScaleChunk{b / (uint32_t)cbx, b % (uint32_t)cbx};
    }
    __device__ __forceinline__ ScaleChunk chunk_w(int kt) const {
        const int k0 = kt * Fp8Stage<C>::BK8;
        if (k0 < ksplit) {
            const uint32_t b = (uint32_t)k0 / 32u;
            return ScaleChunk{b / (uint32_t)cbw, b % (uint32_t)cbw};
        }
        const uint32_t b = (uint32_t)(k0 - ksplit) / 32u;
        return ScaleChunk{(uint32_t)nq0w + b / (uint32_t)cbw, b % (uint32_t)cbw};
    }
    // LDS address of chunk c's buffer for the X (w = false) or W operand
    static __device__ __forceinline__ uint32_t buffer(uint32_t lds, bool w, uint32_t seq) {
        return lds + (uint32_t)Fp8Stage<C>::SC_OFF +
               ((w ? (uint32_t)Fp8Stage<C>::NSCBUF : 0u) + seq % (uint32_t)Fp8Stage<C>::NSCBUF) *
                   (uint32_t)Fp8Stage<C>::SCBUF_BYTES;
    }
    // Before the operand loads of stage kt: this wave's rows of the chunk that
    // starts at kt, if one does. lds: the tile's LDS base.
    __device__ void issue(int kt, uint32_t lds) const {
        const bool is_w = wave_id() >= 4;
        const ScaleChunk c = is_w ? chunk_w(kt) : chunk_x(kt);
        if (c.pos != 0) return;
        const int cb = is_w ? cbw : cbx;
        const int k0 = kt * Fp8Stage<C>::BK8;
        const bool second = is_w && k0 >= ksplit;
        const uint32_t soff = (uint32_t)((second ? k0 - ksplit : k0) >> 5);   // first block of the chunk
        const uint32_t dst = buffer(lds, is_w, c.seq) + (uint32_t)((wave_id() & 3) * 64 * cb);
        if (cb == 16) load_lds16(second ? res2 : res, voff, soff, dst);
        else load_lds4(second ? res2 : res, voff, soff, dst);
    }
};

// 32 bytes of row `row` of a Row tile for the 64-wide step (see the layout note).
__device__ __forceinline__ i32x8_t frag8(uint32_t tile, int row) {
    const int l = threadIdx.x & 63, h = l >> 5, r = row + (l & 31);
    typedef __attribute__((address_space(3))) i32x4_t lds_i32x4_t;
    const i32x4_t lo = *(const lds_i32x4_t *)(uintptr_t)(tile + row_off(r, h));
    const i32x4_t hi = *(const lds_i32x4_t *)(uintptr_t)(tile + row_off(r, 2 + h));
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Scale byte of (tile row `row` + l%32, block l/32 of the stage) from the
// chunk buffer `buf` of CB-byte rows, the stage's first block at `pos`.
__device__ __forceinline__ int scale8(uint32_t buf, int cb, uint32_t pos, int row) {
    const int l = threadIdx.x & 63;
    const uint32_t a = buf + (uint32_t)((row + (l & 31)) * cb) + pos + (uint32_t)(l >> 5);
    return (int)*(const __attribute__((address_space(3))) uint8_t *)(uintptr_t)a;
}

// Block-scaled tile. P provides what gemm_tile's problems provide (C, Args,
// nk counted in 64-wide stages, issue(kt, stage) which also issues the scale
// chunk a stage starts, ahead of its operand loads, wrow, epilogue) and a
// ScaleLoader sl; LOADS_PER_STAGE counts the operand loads only (a stage
// that also loads a scale chunk only makes the waits stricter).
// Same ping-pong schedule as gemm_tile: the two waves of a SIMD (wm = 0, 1)
// run half a stage apart around one barrier per stage, so one group's MFMAs
// cover the other's barrier wait and fragment reads.
// between() runs after the K loop and publish() after the epilogue, as in
// gemm_tile (a persistent workgroup's ticket and a producer's release).
// Returns the constant-clock time at which the K loop ended (item trace).
template <class P, class F, class G>
__device__ __forceinline__ uint64_t gemm8_tile(P &p, uint32_t lds, F &&between, G &&publish) {
    using C = typename P::C;
    using S = Fp8Stage<C>;
    constexpr int FM = C::FM, FN = C::FN, L = P::LOADS_PER_STAGE;
    static_assert(C::WAVES_M == 2 && C::NSTAGE == 4, "two wave groups, 4-stage ring");
    f32x16_t acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
    const int wave = wave_id();
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int nk = __builtin_amdgcn_readfirstlane(p.nk);
    auto stage = [&](int kt) { return lds + (uint32_t)((kt % C::NSTAGE) * S::BYTES); };

    i32x8_t wa[FN], xb[FM];
    int swa[FN], sxb[FM];
    auto read_stage = [&](int kt) {
        const uint32_t st = stage(kt);
        const ScaleChunk cw = p.sl.chunk_w(kt), cx = p.sl.chunk_x(kt);
        const uint32_t bw = ScaleLoader<C>::buffer(lds, true, cw.seq), bx = ScaleLoader<C>::buffer(lds, false, cx.seq);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            wa[fn] = frag8(st + C::X_BYTES, p.wrow(wn, fn));
            swa[fn] = scale8(bw, p.sl.cbw, cw.pos, p.wrow(wn, fn));
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            xb[fm] = frag8(st, wm * C::WM + fm * 32);
            sxb[fm] = scale8(bx, p.sl.cbx, cx.pos, wm * C::WM + fm * 32);
        }
    };
    // The empty asm after each MFMA takes its accumulator as an operand, which
    // pins the MFMA phase where the schedule puts it. Without it the compiler
    // sank wave group 0's MFMAs past the barrier and the next stage's fragment
    // reads (the MFMAs touch no memory, so neither the barrier's memory clobber
    // nor s_setprio holds them), read those fragments into a second register
    // set and copied it back after every stage: both groups then ran their
    // MFMAs right after the same barrier, and the dense fp8 loop took 16% longer.
    auto mma_stage = [&]() {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[fn], xb[fm], acc[fm][fn], 0, 0, 0,
                                                                              swa[fn], 0, sxb[fm]);
                asm volatile("" : "+v"(acc[fm][fn]));
            }
    };
#pragma unroll
    for (int s = 0; s < 3; ++s)
        if (s < nk) p.issue(s, stage(s));
    if (nk > 0) {
        if (nk >= 3) wait_vmcnt<2 * L>();
        else if (nk == 2) wait_vmcnt<L>();
        else wait_vmcnt<0>();
        lds_barrier();
    }
    if (wm == 0) {
        if (nk > 0) read_stage(0);
        for (int kt = 0; kt < nk; ++kt) {
            __builtin_amdgcn_sched_barrier(0);
            mma_stage();
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 2 < nk) wait_vmcnt<L>();
            else wait_vmcnt<0>();
            lds_barrier();
            if (kt + 3 < nk) p.issue(kt + 3, stage(kt + 3));
            if (kt + 1 < nk) read_stage(kt + 1);
        }
    } else {
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 3 < nk) p.issue(kt + 3, stage(kt + 3));
            read_stage(kt);
            if (kt + 3 < nk) wait_vmcnt<2 * L>();
            else if (kt + 2 < nk) wait_vmcnt<L>();
            else wait_vmcnt<0>();
            wait_lgkm0();   // fragment reads of stage kt landed: the slot is refilled right after this barrier
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mma_stage();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const uint64_t t_kloop = __builtin_amdgcn_s_memrealtime();
    between();
    p.epilogue(acc, wm, wn);
    publish();
    return t_kloop;
}
template <class P>
__device__ __forceinline__ void gemm8_tile(P &p, uint32_t lds) {
    gemm8_tile(p, lds, [] {}, [] {});
}

template <class P>
__global__ __launch_bounds__(P::C::NT) void gemm8_kernel(typename P::Args args) {
    extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_raw;
    P p;
    if (!p.setup(args, Blk{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z})) return;
    gemm8_tile(p, lds);
}

}  // namespace mok
