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
// Scale rows are [rows][K/32] bytes with K a multiple of 128, so the 4 bytes
// of blocks 4s .. 4s+3 of a row form one aligned dword; every stage loads that
// dword for each of the 2 x 256 tile rows (waves 0-3: X rows, waves 4-7: W
// rows, one direct-to-LDS dword load per wave and stage) into a [rows][4]
// byte area after the operand tiles. Stage kt reads bytes 2*(kt%2) + 0/1.
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
    static constexpr int SC_OFF = C::X_BYTES + C::W_BYTES;   // [BM][4] X scales, then [BN][4] W scales
    static constexpr int SC_BYTES = (C::BM + C::BN) * 4;
    static constexpr int BYTES = C::STAGE_BYTES + SC_BYTES;
    static constexpr size_t LDS_BYTES = (size_t)C::NSTAGE * BYTES;
    static constexpr int BK8 = 64;                           // fp8 values per row and stage
};

// One direct-to-LDS dword load per wave and stage: the scale dwords of 64
// tile rows. Waves 0-3 load X rows 64w .. 64w+63, waves 4-7 W rows.
template <class C>
struct ScaleLoader {
    rsrc_t res, res2;
    uint32_t voff, lds0;
    int ksplit;   // K (elements) from which res2 holds the blocks, at K - ksplit

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
        ksplit = is_w && w2 ? wsplit : (1 << 30);
        voff = (uint32_t)r * (uint32_t)kb;
        lds0 = (uint32_t)(Fp8Stage<C>::SC_OFF + (is_w ? C::BM * 4 : 0) + (wave & 3) * 256);
    }
    __device__ void issue(int k0, uint32_t stage) const {
        const bool second = k0 >= ksplit;
        const uint32_t soff = (uint32_t)(((second ? k0 - ksplit : k0) >> 7) << 2);
        load_lds4(second ? res2 : res, voff, soff, stage + lds0);
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

// Scale byte of (tile row `row` + l%32, block l/32) for stage kt.
__device__ __forceinline__ int scale8(uint32_t area, int row, int kt) {
    const int l = threadIdx.x & 63;
    const uint32_t a = area + (uint32_t)((row + (l & 31)) * 4 + 2 * (kt & 1) + (l >> 5));
    return (int)*(const __attribute__((address_space(3))) uint8_t *)(uintptr_t)a;
}

// Block-scaled tile. P provides what gemm_tile's problems provide (C, Args,
// nk counted in 64-wide stages, issue(kt, stage) which also issues the scale
// load, wrow, epilogue), with LOADS_PER_STAGE counting the scale load.
// Same ping-pong schedule as gemm_tile: the two waves of a SIMD (wm = 0, 1)
// run half a stage apart around one barrier per stage, so one group's MFMAs
// cover the other's barrier wait and fragment reads.
template <class P>
__device__ __forceinline__ void gemm8_tile(P &p, uint32_t lds) {
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
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            wa[fn] = frag8(st + C::X_BYTES, p.wrow(wn, fn));
            swa[fn] = scale8(st + S::SC_OFF + C::BM * 4, p.wrow(wn, fn), kt);
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            xb[fm] = frag8(st, wm * C::WM + fm * 32);
            sxb[fm] = scale8(st + S::SC_OFF, wm * C::WM + fm * 32, kt);
        }
    };
    auto mma_stage = [&]() {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[fn], xb[fm], acc[fm][fn], 0, 0, 0,
                                                                              swa[fn], 0, sxb[fm]);
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
    p.epilogue(acc, wm, wn);
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
