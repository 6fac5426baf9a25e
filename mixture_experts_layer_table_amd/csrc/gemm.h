// Tile GEMM core for gfx950: C[m][n] = sum_k X[m][k] * W[k][n], bf16 inputs,
// fp32 accumulation on v_mfma_f32_32x32x16_bf16.
//
// The MFMA computes transposed 32x32 blocks of C: its A operand is a block of
// W^T (rows = n), its B operand a block of X (columns = m). With that choice a
// lane of the accumulator holds one row m of C and four consecutive columns n,
// so epilogues store 8-byte runs along n and reduce along n inside a lane.
//
// Both operands are staged in LDS as [rows][BK] bf16 (k contiguous), double
// buffered, with 16-byte chunks XOR-swizzled per row. Two loaders fill a stage:
//   RowTile   — tile rows whose k-values are contiguous in memory (activations
//               in processing order, W^T stored with k contiguous);
//   TransTile — tile columns contiguous in memory along m or n, k strided
//               (weights stored [K][N], token rows for the weight gradients):
//               each thread loads an 8(k) x 8(col) block with 16-byte loads and
//               transposes it in registers before writing LDS.
#pragma once
#include "common.h"

namespace mok {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int KCH = BK / 8;
    static constexpr int STAGE = (BM + BN) * BK;             // bf16 elements per stage
    static constexpr size_t LDS_BYTES = 2 * (size_t)STAGE * 2;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must hold whole 32x32 blocks");
    static_assert(KCH == 8, "LDS swizzle assumes 8 chunks of 16 bytes per row");
};

// chunk c of row r lives at chunk c ^ swz(r): conflict-free for 8 lanes reading
// one chunk of 8 consecutive rows, writing 8 chunks of one row, or writing one
// chunk of rows 8 apart (the transposing loader).
__device__ __forceinline__ int lds_off(int r, int c, int BK) {
    return r * BK + ((c ^ ((r ^ (r >> 3)) & 7)) << 3);
}

// Raw buffer loads: base address and size in SGPRs, one 32-bit VGPR offset per
// thread, plus a uniform scalar offset. Reads at or past `bytes` return zeros
// (the hardware range check), which masks ragged tile edges without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3: 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // a voffset past any buffer used here (all < 2 GiB)

// Tile rows [0, nrows) of a row-major array (ld elements per row), k contiguous.
// An optional second array supplies k >= ksplit (at k - ksplit).
template <class C, int ROWS>
struct RowTile {
    static constexpr int PER = ROWS * C::KCH / C::NT;
    static_assert(PER >= 1 && (ROWS * C::KCH) % C::NT == 0, "row tile must split evenly");
    static constexpr int ROWS_PER_PASS = C::NT / C::KCH;
    rsrc_t res, res2;
    uint32_t voff, rowstep;
    int ksplit;
    uint4 buf[PER];

    __device__ static int row(int i) { return (int)(threadIdx.x + i * C::NT) / C::KCH; }
    __device__ static int chunk() { return (int)threadIdx.x % C::KCH; }

    __device__ void init(const uint16_t *base, int64_t ld, int nrows, const uint16_t *base2 = nullptr,
                         int ksplit_ = 1 << 30) {
        const uint32_t bytes = (uint32_t)((int64_t)max(nrows, 0) * ld * 2);
        res = make_rsrc(base, bytes);
        res2 = make_rsrc(base2 ? base2 : base, bytes);
        voff = (uint32_t)((row(0) * ld + chunk() * 8) * 2);
        rowstep = (uint32_t)(ROWS_PER_PASS * ld * 2);
        ksplit = ksplit_;
    }
    __device__ void load(int k0) {
        const bool second = k0 >= ksplit;
        const rsrc_t r = second ? res2 : res;
        const uint32_t kofs = (uint32_t)((second ? k0 - ksplit : k0) * 2);
#pragma unroll
        for (int i = 0; i < PER; ++i) buf[i] = bload(r, voff, kofs + i * rowstep);
    }
    __device__ void store(uint16_t *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            *reinterpret_cast<uint4 *>(lds + lds_off(row(i), chunk(), C::BK)) = buf[i];
    }
};

// 8 k-rows x 8 columns held by one thread (one uint4 per k-row) -> LDS rows
// cb*8 + c (one per column), k-chunk kb.
template <class C>
__device__ __forceinline__ void trans_block_store(const uint4 (&blk)[8], int kb, int cb, uint16_t *lds) {
    const uint32_t *in = reinterpret_cast<const uint32_t *>(blk);   // [8 k][4 dwords]
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint4 o;
        uint32_t *w = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = in[(2 * j) * 4 + (c >> 1)], b = in[(2 * j + 1) * 4 + (c >> 1)];
            w[j] = (c & 1) ? pack_hi16(a, b) : pack_lo16(a, b);
        }
        *reinterpret_cast<uint4 *>(lds + lds_off(cb * 8 + c, kb, C::BK)) = o;
    }
}

// Tile of BK k-rows x COLS columns of a row-major [rows][ld] array whose
// columns are contiguous (k strided): element (k, c) at base + k*ld + c, k-rows
// [0, nrows) valid (later k-rows read as zeros). Columns past the array's width
// read neighbouring data or zeros; they only feed output rows/columns the
// epilogue discards.
template <class C, int COLS>
struct TransTile {
    static constexpr int CB = COLS / 8;
    static constexpr int NBLK = (C::BK / 8) * CB;
    static constexpr int PER = (NBLK + C::NT - 1) / C::NT;
    rsrc_t res;
    uint32_t voff, ldb;
    uint4 buf[PER][8];

    __device__ static int blk(int i) { return (int)threadIdx.x + i * C::NT; }
    __device__ static bool has(int i) { return NBLK % C::NT == 0 || blk(i) < NBLK; }

    __device__ void init(const uint16_t *base, int64_t ld, int nrows, int ncols) {
        const int64_t bytes = nrows > 0 ? ((int64_t)(nrows - 1) * ld + ncols) * 2 : 0;
        res = make_rsrc(base, (uint32_t)bytes);
        ldb = (uint32_t)(ld * 2);
        const int b = blk(0);
        voff = (uint32_t)(((int64_t)(b / CB) * 8 * ld + (b % CB) * 8) * 2);
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!has(i)) continue;
            const uint32_t v = voff + (uint32_t)(i * C::NT / CB) * 8 * ldb;   // PER > 1 only when NT divides CB
#pragma unroll
            for (int r = 0; r < 8; ++r) buf[i][r] = bload(res, v, (uint32_t)(k0 + r) * ldb);
        }
    }
    __device__ void store(uint16_t *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (has(i)) trans_block_store<C>(buf[i], blk(i) / CB, blk(i) % CB, lds);
    }
};

// TransTile whose first COLS/2 columns come from one array and the rest from
// another (the gate | up pairing). Each half of the workgroup's waves loads one
// half, so every wave's buffer descriptor stays uniform.
template <class C, int COLS>
struct TransTileSplit {
    static constexpr int CB = COLS / 8, HCB = CB / 2;
    static_assert((C::BK / 8) * CB == C::NT, "one 8x8 block per thread");
    rsrc_t res;
    uint32_t voff, ldb;
    int kb, cb;
    uint4 buf[8];

    // element (k, c) of half h at base_h + k*ld + c, k-rows [0, nrows), ncols
    // columns from each base
    __device__ void init(const uint16_t *base0, const uint16_t *base1, int64_t ld, int nrows, int ncols) {
        const int half = __builtin_amdgcn_readfirstlane((int)threadIdx.x / (C::NT / 2));
        const int lt = (int)threadIdx.x % (C::NT / 2);
        kb = lt / HCB;
        cb = half * HCB + lt % HCB;
        const int64_t bytes = nrows > 0 ? ((int64_t)(nrows - 1) * ld + ncols) * 2 : 0;
        res = make_rsrc(half ? base1 : base0, (uint32_t)bytes);
        ldb = (uint32_t)(ld * 2);
        voff = (uint32_t)(((int64_t)kb * 8 * ld + (lt % HCB) * 8) * 2);
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int r = 0; r < 8; ++r) buf[r] = bload(res, voff, (uint32_t)(k0 + r) * ldb);
    }
    __device__ void store(uint16_t *lds) const { trans_block_store<C>(buf, kb, cb, lds); }
};

// As TransTile, for k-rows gathered through an index: k-row k lives at
// base + idx[k]*ld (k >= n: zeros). Each thread keeps the row indices of its
// next tile in registers, fetched one tile ahead so that data loads never wait
// on an index load.
template <class C, int COLS>
struct TransTileIdx {
    static constexpr int CB = COLS / 8;
    static constexpr int NBLK = (C::BK / 8) * CB;
    static constexpr int PER = (NBLK + C::NT - 1) / C::NT;
    rsrc_t res;
    uint32_t coloff, ldb;
    const int32_t *idx;
    int n;
    int32_t nid[PER][8];
    uint4 buf[PER][8];

    __device__ static int blk(int i) { return (int)threadIdx.x + i * C::NT; }
    __device__ static bool has(int i) { return NBLK % C::NT == 0 || blk(i) < NBLK; }

    // base points at column 0 of row 0 of an array of `total_rows` rows; the
    // tile's columns start at col0 and the array has ncols columns.
    __device__ void init(const int32_t *idx_, int n_, const uint16_t *base, int64_t ld, int64_t total_rows,
                         int col0, int ncols) {
        (void)ncols;
        idx = idx_;
        n = n_;
        res = make_rsrc(base, (uint32_t)(total_rows * ld * 2));
        ldb = (uint32_t)(ld * 2);
        coloff = (uint32_t)((col0 + (blk(0) % CB) * 8) * 2);
        fetch(0);
    }
    __device__ void fetch(int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!has(i)) continue;
            const int kb = blk(i) / CB;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int k = k0 + kb * 8 + r;
                nid[i][r] = k < n ? idx[k] : -1;
            }
        }
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!has(i)) continue;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const uint32_t v = nid[i][r] >= 0 ? (uint32_t)nid[i][r] * ldb + coloff : kOutOfRange;
                buf[i][r] = bload(res, v, 0);
            }
        }
        fetch(k0 + C::BK);
    }
    __device__ void store(uint16_t *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (has(i)) trans_block_store<C>(buf[i], blk(i) / CB, blk(i) % CB, lds);
    }
};

// One BK stage of MFMAs, LDS fragments double buffered across the 16-wide
// k-steps. wrow(wn, fn) gives the LDS W row of n-block fn of wave wn.
template <class C, class P>
__device__ __forceinline__ void mma_stage(const uint16_t *stage, f32x16_t (&acc)[C::FM][C::FN], int wm,
                                          int wn, const P &p) {
    const uint16_t *xs = stage;
    const uint16_t *ws = stage + C::BM * C::BK;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5;
    constexpr int KS = C::BK / 16;
    bf16x8_t a[2][C::FN], b[2][C::FM];
    auto frags = [&](int kk, int s) {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
            a[s][fn] = *reinterpret_cast<const bf16x8_t *>(ws + lds_off(p.wrow(wn, fn) + lr, kk * 2 + lh, C::BK));
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            b[s][fm] = *reinterpret_cast<const bf16x8_t *>(xs + lds_off(wm * C::WM + fm * 32 + lr, kk * 2 + lh, C::BK));
    };
    frags(0, 0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) frags(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][fn], b[kk & 1][fm], acc[fm][fn], 0, 0, 0);
    }
}

// Generic tile kernel body. P provides: setup(args) -> bool, nk, load(kt),
// store(stage), wrow(wn, fn), epilogue(acc, wm, wn).
template <class P>
__global__ __launch_bounds__(P::C::NT) void gemm_kernel(typename P::Args args) {
    using C = typename P::C;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    P p;
    if (!p.setup(args)) return;
    f32x16_t acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int nk = p.nk;
    if (nk > 0) {
        p.load(0);
        p.store(lds);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const uint16_t *cur = lds + (kt & 1) * C::STAGE;
            uint16_t *nxt = lds + ((kt + 1) & 1) * C::STAGE;
            if (kt + 1 < nk) p.load(kt + 1);
            mma_stage<C>(cur, acc, wm, wn, p);
            if (kt + 1 < nk) p.store(nxt);
            __syncthreads();
        }
    }
    p.epilogue(acc, wm, wn);
}

}  // namespace mok
