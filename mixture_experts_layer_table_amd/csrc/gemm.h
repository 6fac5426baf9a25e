// Tile GEMM core for gfx950: C[m][n] = sum_k X[m][k] * W[k][n], bf16 inputs,
// fp32 accumulation on v_mfma_f32_32x32x16_bf16.
//
// The MFMA computes transposed 32x32 blocks of C: its A operand is a block of
// W^T (rows = n), its B operand a block of X (columns = m). A lane of the
// accumulator then holds one row m of C and four consecutive columns n, so
// epilogues store 8-byte runs along n and reduce along n inside a lane.
//
// Data path, per workgroup tile BM x BN and K-step BK = 32:
//  * global -> LDS with direct loads (buffer_load ... lds, 16 bytes per lane,
//    lane l lands at the instruction's LDS base + 16*l): no register staging;
//  * an NSTAGE-deep LDS ring: while the MFMAs consume stage kt, the loads of
//    k-steps kt+1 .. kt+NSTAGE-1 are in flight;
//  * two LDS tile layouts, one per operand kind:
//      Row   — tile rows whose k-values are contiguous in memory (activations,
//              W^T with k contiguous): [rows][32] bf16, 16-byte chunks swizzled;
//              fragments read with ds_read_b128;
//      Trans — tile columns contiguous in memory, k strided (weights stored
//              [K][N], token rows of the weight gradients): [32][cols] bf16 in
//              sub-tiles of 128 columns, chunks swizzled by k; fragments read
//              with two ds_read_b64_tr_b16 (the LDS transpose read), which
//              deliver 4 consecutive k of one column to each lane.
//  * buffer loads past a tile's valid range return zeros (hardware range
//    check), which masks ragged edges without branches.
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"
#include "../../include/mok.h"

namespace mok {

// OCC: waves per SIMD the kernel is built for (2: up to 256 registers per
// lane; 4: up to 128, two 8-wave workgroups per compute unit).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_, int OCC_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 32, OCC = OCC_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = 64 * NW;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int NSTAGE = NSTAGE_;
    static constexpr int X_BYTES = BM * BK * 2;   // one stage of the X tile
    static constexpr int W_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = X_BYTES + W_BYTES;
    static constexpr size_t LDS_BYTES = (size_t)NSTAGE * STAGE_BYTES;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must hold whole 32x32 blocks");
    static_assert(BM % 128 == 0 && BN % 128 == 0, "tiles are made of 128-wide sub-tiles");
    // The ping-pong K loop needs loads D = NSTAGE - 1 >= 2 stages ahead: wave
    // group 0 reads stage kt+1 right after barrier kt, and group 1 reads stage
    // kt+1 before barrier kt+1, so every load of stage kt+1 must have been
    // issued, and waited for by its wave, before barrier kt. With D = 1 stage
    // kt+1 would be issued only after barrier kt.
    static_assert(NSTAGE >= 3, "loads must run at least two stages ahead");
};

// ----------------------------------------------------------------------------- buffer loads

// Buffer descriptor (SGPR quad): base address, size in bytes; word 3 selects
// 32-bit data format, the gfx9 value for raw loads.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;    // a voffset past any buffer used here (all < 2 GiB)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    rsrc_t d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    d[3] = kBufWord3;
    return d;
}

// 16 bytes per lane from r at voff + soff into LDS at `dst` + 16 * lane
// (buffer_load_dwordx4 ... lds; M0 holds the LDS base). Issued as inline asm so
// that the compiler does not track these LDS writes: ordering against LDS
// reads is explicit (wait_vmcnt + lds_barrier in the kernel loop).
// The descriptor is wave-uniform by construction; readfirstlane states it to
// the compiler (a no-op when the value already sits in scalar registers).
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ rsrc_t uniform(rsrc_t r) {
    rsrc_t u;
    u.x = __builtin_amdgcn_readfirstlane(r.x);
    u.y = __builtin_amdgcn_readfirstlane(r.y);
    u.z = __builtin_amdgcn_readfirstlane(r.z);
    u.w = __builtin_amdgcn_readfirstlane(r.w);
    return u;
}

__device__ __forceinline__ void load_lds16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t dst) {
    // one wait state between the SALU write of M0 and the LDS-DMA read of it (GFX9 hazard)
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(uniform(r)), "s"(uniform(soff)), "s"(uniform(dst))
                 : "memory", "m0");
}

// 4-byte direct-to-LDS load: lane l's dword lands at LDS address dst + 4*l.
__device__ __forceinline__ void load_lds4(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(uniform(r)), "s"(uniform(soff)), "s"(uniform(dst))
                 : "memory", "m0");
}

// Four consecutive int32 at a uniform address, read through the constant
// address space so that the compiler emits a scalar load (s_load_dwordx4,
// counted by lgkmcnt rather than vmcnt) and places its wait before the first
// use itself. (A load written as inline asm would not do: the compiler takes
// an asm output as ready when the statement ends and may copy the registers
// before the data has arrived.)
struct sidx4_t {
    int32_t v[4];
};
__device__ __forceinline__ sidx4_t sload4(const int32_t *p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const auto *c = reinterpret_cast<const __attribute__((address_space(4))) int32_t *>(((uint64_t)hi << 32) | lo);
    return sidx4_t{{c[0], c[1], c[2], c[3]}};
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wave index as a provably uniform value (keeps descriptors and M0 in SGPRs).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those would wait for every outstanding direct-to-LDS load. Callers first
// wait (vmcnt) for the loads whose data the barrier publishes; LDS writes by
// those loads are complete once the counter has passed them.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ----------------------------------------------------------------------------- LDS layouts (byte offsets)

// Row layout: [rows][32] bf16, 64-byte rows of four 16-byte chunks; chunk c of
// row r sits at c ^ ((r >> 2) & 3). The LDS serves 256 bytes (64 banks) per
// cycle, 16 lanes of a 16-byte read: 16 lanes reading one chunk of 16
// consecutive rows then hit 16 distinct 16-byte bank groups (r % 4 picks the
// 64-byte quarter, (r >> 2) & 3 the group inside it).
__device__ __forceinline__ uint32_t row_off(int r, int c) {
    return (uint32_t)(r * 64 + ((c ^ ((r >> 2) & 3)) << 4));
}

// Trans layout: sub-tiles of 128 columns, each [32 k][128] bf16 with 256-byte
// k-rows; 16-byte chunk c of k-row k sits at c ^ (4 * (k & 3)). The 32 lanes
// the LDS serves per cycle of a transpose read cover 4 consecutive k-rows x 4
// chunks of one 32-column block: the XOR moves each k-row's 4 chunks to its
// own quarter of the 256-byte bank window, so they hit 16 distinct groups.
__device__ __forceinline__ uint32_t trans_off(int k, int col) {
    return (uint32_t)((col >> 7) * (32 * 256) + k * 256 + (((((col & 127) >> 3) ^ ((k & 3) << 2))) << 4) +
                      ((col & 7) << 1));
}

// ----------------------------------------------------------------------------- direct loaders

// Row tile: rows [0, nrows) of a row-major array with ld elements per row
// starting at `base`, k-step columns [k0, k0 + 32). Optional second array for
// k >= ksplit (at k - ksplit). Each wave issues ROWS / 16 / NW instructions of
// 16 rows each.
//
// K-tiled arrays (init_tiled): blocks of 32 columns, each [rows][32] (64-byte
// rows, rows contiguous), one block after the other. A stage's tile is then
// one contiguous run of ROWS x 64 bytes: whole 128-byte lines, where rows of
// a row-major array are 64-byte pieces of ROWS different lines.
template <class C, int ROWS>
struct RowLoader {
    static constexpr int IPW = ROWS / 16 / C::NW;     // instructions per wave per stage
    static_assert(IPW >= 1 && ROWS % (16 * C::NW) == 0, "row tile must split over the waves");
    rsrc_t res, res2;
    uint32_t voff, ldb, lds0;
    int ksplit;
    uint32_t kblock = 0;   // K-tiled: bytes from one 32-column block to the next (0: row-major)

    __device__ void init(const uint16_t *base, int64_t ld, int nrows, const uint16_t *base2 = nullptr,
                         int ksplit_ = 1 << 30) {
        const uint32_t bytes = (uint32_t)((int64_t)max(nrows, 0) * ld * 2);
        res = make_rsrc(base, bytes);
        res2 = make_rsrc(base2 ? base2 : base, bytes);
        ldb = (uint32_t)(ld * 2);
        const int wave = wave_id(), L = threadIdx.x & 63;
        const int r = wave * IPW * 16 + (L >> 2);
        const int c = (L & 3) ^ ((L >> 4) & 3);      // (r >> 2) & 3 == (L >> 4) & 3 (16-row blocks)
        voff = (uint32_t)r * ldb + (uint32_t)(c << 4);
        lds0 = (uint32_t)(wave * IPW * 1024);
        ksplit = ksplit_;
    }
    // K-tiled array: `base` is the tile's first row in the first block; rows
    // past the tile's valid ones read the array's other rows (their outputs
    // are discarded) or, past `bytes` (what the array holds from `base` on),
    // zeros.
    __device__ void init_tiled(const void *base, uint32_t block_bytes, uint32_t bytes) {
        res = make_rsrc(base, bytes);
        res2 = res;
        ldb = 64;
        kblock = block_bytes;
        const int wave = wave_id(), L = threadIdx.x & 63;
        const int r = wave * IPW * 16 + (L >> 2);
        const int c = (L & 3) ^ ((L >> 4) & 3);
        voff = (uint32_t)r * 64u + (uint32_t)(c << 4);
        lds0 = (uint32_t)(wave * IPW * 1024);
        ksplit = 1 << 30;
    }
    // Rows [0, ROWS/2) of the tile from `lo`, rows [ROWS/2, ROWS) from `hi`
    // (nrows_each valid rows in each; every wave's rows lie in one half).
    __device__ void init_split_rows(const uint16_t *lo, const uint16_t *hi, int64_t ld, int nrows_each) {
        static_assert((ROWS / 2) % (IPW * 16) == 0, "a wave's rows must lie in one half");
        const int wave = wave_id();
        const bool upper = wave * IPW * 16 >= ROWS / 2;
        const uint32_t bytes = (uint32_t)((int64_t)max(nrows_each, 0) * ld * 2);
        res = make_rsrc(upper ? hi : lo, bytes);
        res2 = res;
        ldb = (uint32_t)(ld * 2);
        const int L = threadIdx.x & 63;
        const int r = wave * IPW * 16 + (L >> 2) - (upper ? ROWS / 2 : 0);
        const int c = (L & 3) ^ ((L >> 4) & 3);
        voff = (uint32_t)r * ldb + (uint32_t)(c << 4);
        lds0 = (uint32_t)(wave * IPW * 1024);
        ksplit = 1 << 30;
    }
    __device__ void issue(int k0, uint32_t tile) const {
        const bool second = k0 >= ksplit;
        const rsrc_t r = second ? res2 : res;
        if (kblock) {   // the whole offset in voffset: the range check leaves soffset out
            const uint32_t kb = (uint32_t)(k0 >> 5) * kblock;
#pragma unroll
            for (int i = 0; i < IPW; ++i) load_lds16(res, voff + kb + (uint32_t)(i * 1024), 0, tile + lds0 + i * 1024);
            return;
        }
        const uint32_t kofs = (uint32_t)((second ? k0 - ksplit : k0) * 2);
#pragma unroll
        for (int i = 0; i < IPW; ++i) load_lds16(r, voff, kofs + (uint32_t)(i * 16) * ldb, tile + lds0 + i * 1024);
    }
};

// Trans tile: k-rows [k0, k0 + 32) x COLS columns of a row-major [K][ld] array
// whose columns are contiguous; element (k, c) at base + k*ld + c with k-rows
// [0, nrows) valid (later k-rows read as zeros). With a second base, columns
// [COLS/2, COLS) come from it instead (the gate | up pairing). Columns past
// the array's width read neighbouring data or zeros: they only feed output
// rows/columns the epilogue discards.
template <class C, int COLS>
struct TransLoader {
    static constexpr int NINST = COLS / 128 * 8;      // 8 instructions (4 k-rows each) per sub-tile
    static constexpr int IPW = NINST / C::NW;
    static_assert(IPW >= 1 && NINST % C::NW == 0, "trans tile must split over the waves");
    rsrc_t res, res2;
    uint32_t voff, ldb, lds0;
    int inst0;
    bool split;

    __device__ void init(const uint16_t *base, int64_t ld, int nrows, int ncols, const uint16_t *base2 = nullptr) {
        const int64_t bytes = nrows > 0 ? ((int64_t)(nrows - 1) * ld + ncols) * 2 : 0;
        res = make_rsrc(base, (uint32_t)bytes);
        res2 = make_rsrc(base2 ? base2 : base, (uint32_t)bytes);
        split = base2 != nullptr;
        ldb = (uint32_t)(ld * 2);
        const int wave = wave_id(), L = threadIdx.x & 63;
        const int c = (L & 15) ^ ((L >> 4) << 2);    // k & 3 == L >> 4
        voff = (uint32_t)(L >> 4) * ldb + (uint32_t)(c << 4);
        inst0 = wave * IPW;
        lds0 = (uint32_t)(inst0 * 1024);
    }
    __device__ void issue(int k0, uint32_t tile) const {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int inst = inst0 + i, sub = inst >> 3, kq = inst & 7;
            constexpr int SUBS = COLS >= 256 ? COLS / 256 : 1;   // 256-column sub-tiles per source
            const bool second = split && sub >= SUBS;
            const uint32_t colb = split ? (uint32_t)((sub % SUBS) * 256) : (uint32_t)(sub * 256);
            load_lds16(second ? res2 : res, voff, (uint32_t)(k0 + kq * 4) * ldb + colb, tile + lds0 + i * 1024);
        }
    }
};

// Trans tile whose k-rows are gathered through an index: k-row k lives at
// base + idx[k]*ld (k >= n: zeros), tile columns start at col0. The indices a
// wave needs for one issue (4 consecutive k-rows per instruction) are read
// with scalar loads, whose counter is separate from the vector-memory counter
// that tracks the direct-to-LDS loads; each lane then picks the index of its
// own k-row. fetch(k0) must precede issue(k0), in k order; the K loop places
// each fetch where no wait on LDS reads follows soon: scalar loads return out
// of order, so while one is in flight every wait for an LDS fragment becomes
// a wait for all of them, the scalar load's memory round trip included.
// init loads the indices of the first two issues together, so that the
// prologue's second issue does not wait for a round trip of its own (with a
// few k-steps per tile, as for many small experts, that wait is a large part
// of the tile).
template <class C, int COLS>
struct TransIdxLoader {
    static constexpr int NINST = COLS / 128 * 8;
    static constexpr int IPW = NINST / C::NW;
    static_assert(IPW >= 1 && NINST % C::NW == 0, "trans tile must split over the waves");
    rsrc_t res;
    uint32_t coff, ldb, lds0;
    const int32_t *idx;
    int n, inst0, krow;
    sidx4_t nid[IPW];   // indices of the next issue's k-rows (loaded one issue ahead)
    sidx4_t nid1[IPW];  // indices of the second issue (k0 = BK), loaded by init

    __device__ void init(const int32_t *idx_, int n_, const uint16_t *base, int64_t ld, int64_t total_rows,
                         int col0) {
        idx = idx_;
        n = n_;
        res = make_rsrc(base, (uint32_t)(total_rows * ld * 2));
        ldb = (uint32_t)(ld * 2);
        const int wave = wave_id(), L = threadIdx.x & 63;
        const int c = (L & 15) ^ ((L >> 4) << 2);
        coff = (uint32_t)((col0 + c * 8) * 2);
        krow = L >> 4;
        inst0 = wave * IPW;
        lds0 = (uint32_t)(inst0 * 1024);
        load(0, nid);
        load(C::BK, nid1);
    }
    // Scalar loads of the indices of k-rows [k0, k0 + 32) this wave issues;
    // reads at most 3 ints past the expert's rows (inside the index array's buffer).
    __device__ void load(int k0, sidx4_t (&dst)[IPW]) const {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int kb = min(k0 + ((inst0 + i) & 7) * 4, max(n - 1, 0));
            dst[i] = sload4(idx + kb);
        }
    }
    __device__ void fetch(int k0) {
        if (k0 == C::BK) {
#pragma unroll
            for (int i = 0; i < IPW; ++i) nid[i] = nid1[i];
        } else {
            load(k0, nid);
        }
    }
    // issue(k0) uses the indices fetched for k0 (init fetches those of k0 = 0).
    __device__ void issue(int k0, uint32_t tile) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int inst = inst0 + i, sub = inst >> 3, kb = k0 + (inst & 7) * 4;
            const int32_t r0 = nid[i].v[0], r1 = nid[i].v[1], r2 = nid[i].v[2], r3 = nid[i].v[3];
            const int32_t mine = krow == 0 ? r0 : krow == 1 ? r1 : krow == 2 ? r2 : r3;
            const uint32_t v = kb + krow < n ? (uint32_t)mine * ldb + coff + (uint32_t)(sub * 256) : kOutOfRange;
            load_lds16(res, v, 0, tile + lds0 + i * 1024);
        }
    }
};

// ----------------------------------------------------------------------------- fragments

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// MFMA operand for 32 tile rows starting at `row` of a Row tile, k-step kk:
// lane l holds row + l%32, k = 16*kk + 8*(l/32) + 0..7.
__device__ __forceinline__ bf16x8_t frag_row(uint32_t tile, int row, int kk) {
    const int l = threadIdx.x & 63;
    const uint32_t a = tile + row_off(row + (l & 31), kk * 2 + (l >> 5));
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
        (const __attribute__((address_space(3))) char *)(uintptr_t)a);
}

// MFMA operand for 32 tile columns starting at `col` of a Trans tile, k-step kk:
// lane l holds column col + l%32, k = 16*kk + 8*(l/32) + 0..7. Within each
// group of 16 lanes the transpose read hands lane i the 4 values at
// (k0 + j, c0 + i), j = 0..3, when source lane 4j + q points at (k0 + j, c0 + 4q).
__device__ __forceinline__ bf16x8_t frag_trans(uint32_t tile, int col, int kk) {
    const int l = threadIdx.x & 63;
    const int g = l >> 4, s = l & 15;
    const int k = kk * 16 + (g >> 1) * 8 + (s >> 2);
    const int c = col + (g & 1) * 16 + (s & 3) * 4;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(uintptr_t)(tile + trans_off(k, c)));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(uintptr_t)(tile + trans_off(k + 4, c)));
    typedef short v8i16_t __attribute__((ext_vector_type(8)));
    const v8i16_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

template <bool TRANS>
__device__ __forceinline__ bf16x8_t frag(uint32_t tile, int rc, int kk) {
    if constexpr (TRANS)
        return frag_trans(tile, rc, kk);
    else
        return frag_row(tile, rc, kk);
}

// Fragments and MFMAs of one 16-wide k-step (kk = 0, 1 of a BK = 32 stage).
// FULL: every 32-row block of the wave's rows holds valid rows; otherwise only
// the first `live` blocks do, and the others (zeros from the range-checked
// loads, discarded by the epilogue) are neither read nor multiplied.
template <class C, class P, bool FULL>
struct Frags {
    bf16x8_t a[C::FN], b[C::FM];
    __device__ __forceinline__ void read(uint32_t stage, int kk, int wm, int wn, const P &p, int live) {
        if (!FULL && live == 0) return;
        const uint32_t xs = stage, ws = stage + C::X_BYTES;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) a[fn] = frag<P::W_TRANS>(ws, p.wrow(wn, fn), kk);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            if (FULL || fm < live) b[fm] = frag<P::X_TRANS>(xs, wm * C::WM + fm * 32, kk);
    }
    __device__ __forceinline__ void mma(f32x16_t (&acc)[C::FM][C::FN], int live) const {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            if (FULL || fm < live)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fn], b[fm], acc[fm][fn], 0, 0, 0);
    }
};

// Wait for every LDS read (and scalar load) of this wave. The asm form keeps
// memory accesses from moving across it; the builtin that follows tells the
// compiler's own wait tracking that nothing is pending any more, so that it
// does not wait again (then also for scalar loads issued later) before the
// next use of the fragments.
__device__ __forceinline__ void wait_lgkm0() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt left at their maxima (gfx9 encoding)
}

// Block coordinates of a tile (the launch grid's, or a persistent kernel's
// virtual grid).
struct Blk {
    int x, y, z;
};

// One output tile. P provides: C, Args, X_TRANS, W_TRANS, LOADS_PER_STAGE
// (vector-memory instructions one wave issues per stage), nk, mvalid() (valid
// rows of the X tile),
// issue(kt, stage_lds_address), wrow(wn, fn), epilogue(acc, wm, wn), and
// for gemm_kernel setup(args) -> bool.
//
// Ping-pong schedule. The two wave groups (wm = 0 and wm = 1) run half a
// stage apart around one barrier per stage (stage = kt % NSTAGE; loads run
// D = NSTAGE - 1 stages ahead):
//   group 0: MFMAs(stage kt) | wait own loads of kt+1 | barrier | issue kt+D, read fragments(kt+1)
//   group 1: issue kt+D, read fragments(kt) | wait own loads of kt+1 | barrier | MFMAs(stage kt)
// While one group waits at the barrier or for its fragment reads, the other
// group's MFMAs keep the matrix cores busy.
// Ordering: every wave waits for its own loads of stage kt+1 before barrier
// kt, so stage kt+1 is visible after it (group 0 reads it right away, group 1
// in its next iteration). Slot kt-1 is refilled (with stage kt+D) after
// barrier kt-1 by group 1 and after barrier kt by group 0; every read of stage
// kt-1 has landed before barrier kt-1: group 0 consumed its fragments in the
// MFMAs before that barrier, and group 1 waits for its reads (lgkmcnt) right
// before it.
// s_waitcnt for "at most n stages of L loads still in flight" (n wave-uniform, 0 <= n).
template <int L, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            wait_vmcnt<MAXN * L>();
            return;
        }
        wait_stages<L, MAXN - 1>(n);
    } else {
        wait_vmcnt<0>();
    }
}

// P::fetch(kt), where a problem has it, prepares what issue(kt) needs (the
// scalar index loads of a gathered operand); fetch(0) is part of setup.
template <class P, class = void>
struct has_fetch : std::false_type {};
template <class P>
struct has_fetch<P, std::void_t<decltype(std::declval<P &>().fetch(0))>> : std::true_type {};
template <class P>
__device__ __forceinline__ void fetch_stage(P &p, int kt) {
    if constexpr (has_fetch<P>::value) p.fetch(kt);
}

// K loop of one tile into acc (acc zeroed by the caller). live: the wave's
// 32-row blocks that hold valid rows (FM when FULL).
template <class P, bool FULL>
__device__ __forceinline__ void gemm_kloop(P &p, uint32_t lds, f32x16_t (&acc)[P::C::FM][P::C::FN], int live) {
    using C = typename P::C;
    constexpr int L = P::LOADS_PER_STAGE, D = C::NSTAGE - 1;
    const int wave = wave_id();
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int nk = __builtin_amdgcn_readfirstlane(p.nk);
    auto stage = [&](int kt) { return lds + (uint32_t)((kt % C::NSTAGE) * C::STAGE_BYTES); };
    Frags<C, P, FULL> f0, f1;
    auto read_stage = [&](int kt) {
        f0.read(stage(kt), 0, wm, wn, p, live);
        f1.read(stage(kt), 1, wm, wn, p, live);
    };
    auto mma_stage = [&]() {
        f0.mma(acc, live);
        f1.mma(acc, live);
    };
#pragma unroll
    for (int s = 0; s < D; ++s)
        if (s < nk) {
            if (s > 0) fetch_stage(p, s);
            p.issue(s, stage(s));
        }
    if (nk > 0) {
        wait_stages<L, D - 1>(min(D, nk) - 1);   // stage 0 landed
        lds_barrier();
    }
    // Index fetches (fetch_stage) go where no LDS wait follows soon: group 0
    // right after issuing its MFMAs (the next LDS wait is after the barrier),
    // group 1 right after the barrier (its MFMA phase reads no LDS).
    if (wm == 0) {
        if (nk > 0) read_stage(0);
        for (int kt = 0; kt < nk; ++kt) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
            mma_stage();
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            if (kt + D < nk) fetch_stage(p, kt + D);
            // own loads issued so far: up to stage kt + D - 1; stage kt + 1 must have landed
            if constexpr (D >= 2) wait_stages<L, D - 2>(max(0, min(D - 2, nk - 2 - kt)));
            else wait_vmcnt<0>();
            lds_barrier();
            if (kt + D < nk) p.issue(kt + D, stage(kt + D));
            if (kt + 1 < nk) read_stage(kt + 1);
        }
    } else {
        if (D < nk) fetch_stage(p, D);
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + D < nk) p.issue(kt + D, stage(kt + D));
            read_stage(kt);
            // own loads issued so far: up to stage kt + D; stage kt + 1 must have landed
            wait_stages<L, D - 1>(max(0, min(D - 1, nk - 2 - kt)));
            wait_lgkm0();   // fragment reads of stage kt landed: the slot is refilled right after this barrier
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (kt + D + 1 < nk) fetch_stage(p, kt + D + 1);
            __builtin_amdgcn_s_setprio(1);
            mma_stage();
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// K loop of one tile into acc. P::mvalid() gives the tile's valid X rows: a
// wave whose rows are partly or wholly past them takes the K loop that skips
// the empty 32-row blocks (both loops run the same barriers). Grouped GEMMs
// whose groups hold fewer rows than the tile (many small experts) then spend
// matrix-core time on real rows only.
template <class P>
__device__ __forceinline__ void gemm_mainloop(P &p, uint32_t lds, f32x16_t (&acc)[P::C::FM][P::C::FN]) {
    using C = typename P::C;
    static_assert(C::WAVES_M == 2, "two wave groups");
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
    const int wm = wave_id() / C::WAVES_N;
    const int d = __builtin_amdgcn_readfirstlane(p.mvalid() - wm * C::WM);
    const int live = d <= 0 ? 0 : min(C::FM, (d + 31) / 32);
    if (live == C::FM)
        gemm_kloop<P, true>(p, lds, acc, C::FM);
    else
        gemm_kloop<P, false>(p, lds, acc, live);
}

// A tile pipeline whose epilogue takes a `publish` callable (P::SPLIT_EPILOGUE
// true) stores first what consumer tiles of the same launch read, calls
// publish() from every wave, then stores the rest.
template <class P, class = void>
struct split_epilogue : std::false_type {};
template <class P>
struct split_epilogue<P, std::void_t<decltype(P::SPLIT_EPILOGUE)>> : std::bool_constant<P::SPLIT_EPILOGUE> {};

// One tile: prologue, K loop, `between()` (e.g. a persistent workgroup's
// claim of its next item), epilogue, and `publish()` (a persistent producer's
// completion: barrier and release), inside the epilogue for split epilogues,
// after it otherwise. Returns the constant-clock time (s_memrealtime,
// 100 MHz) at which the K loop ended, for the item trace.
template <class P, class F, class G>
__device__ __forceinline__ uint64_t gemm_tile(P &p, uint32_t lds, F &&between, G &&publish) {
    using C = typename P::C;
    f32x16_t acc[C::FM][C::FN];
    gemm_mainloop(p, lds, acc);
    const uint64_t t_kloop = __builtin_amdgcn_s_memrealtime();
    between();
    const int wave = wave_id();
    if constexpr (split_epilogue<P>::value) {
        p.epilogue(acc, wave / C::WAVES_N, wave % C::WAVES_N, publish);
    } else {
        p.epilogue(acc, wave / C::WAVES_N, wave % C::WAVES_N);
        publish();
    }
    return t_kloop;
}
template <class P>
__device__ __forceinline__ uint64_t gemm_tile(P &p, uint32_t lds) {
    return gemm_tile(p, lds, [] {}, [] {});
}

// ----------------------------------------------------------------------------- item trace

// Destination of the optional per-item trace (mok_item_trace_enable): null
// when tracing is off, which costs one scalar branch per tile.
struct TraceArgs {
    mok_item_record *rec;
    int *count;
    int cap;
    uint32_t launch;
    int kernel;
};

// Thread 0 of a workgroup: append one record (dropped once the buffer is full).
__device__ __forceinline__ void trace_item(const TraceArgs &tr, uint64_t t_claim, uint64_t t_start, uint64_t t_kloop,
                                           int cls, int item) {
    if (!tr.rec) return;
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    const int slot = atomicAdd(tr.count, 1);
    if (slot >= tr.cap) return;
    mok_item_record r;
    r.t_claim = t_claim;
    r.t_start = t_start;
    r.t_kloop = t_kloop;
    r.t_end = t_end;
    r.launch = tr.launch;
    r.kernel = (uint8_t)tr.kernel;
    r.item_class = (uint8_t)cls;
    r.xcd = (uint16_t)(blockIdx.x % 8);
    r.item = (uint32_t)item;
    r.workgroup = blockIdx.x;
    tr.rec[slot] = r;
}

// One tile per workgroup; P::setup(args, block) picks the tile (false: no tile).
// C::OCC waves per SIMD: with OCC = 2, one 8-wave workgroup per compute unit;
// with OCC = 4 (and at most 80 KiB of LDS), two.
template <class P>
__global__ __launch_bounds__(P::C::NT, P::C::OCC) void gemm_kernel(typename P::Args args, TraceArgs tr) {
    extern __shared__ __attribute__((aligned(1024))) char lds_raw[];
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds_raw;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    P p;
    if (!p.setup(args, Blk{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z})) return;
    const uint64_t t_kloop = gemm_tile(p, lds);
    if (tr.rec) {
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0) trace_item(tr, t0, t0, t_kloop, 0, (int)blockIdx.x);
    }
}

}  // namespace mok
