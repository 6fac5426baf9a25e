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

template <class C, int ROWS>
struct RowTile {
    static constexpr int PER = ROWS * C::KCH / C::NT;
    static_assert(PER >= 1 && (ROWS * C::KCH) % C::NT == 0, "row tile must split evenly");
    const uint16_t *ptr[PER];
    uint4 buf[PER];

    __device__ static int row(int i) { return (int)(threadIdx.x + i * C::NT) / C::KCH; }
    __device__ static int chunk() { return (int)threadIdx.x % C::KCH; }

    // f(r) -> pointer to element (r, k = 0) of tile row r, or nullptr for a zero row
    template <class F>
    __device__ void init(F &&f) {
#pragma unroll
        for (int i = 0; i < PER; ++i) ptr[i] = f(row(i));
    }
    __device__ void load(int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            buf[i] = ptr[i] ? *reinterpret_cast<const uint4 *>(ptr[i] + k0 + chunk() * 8)
                            : make_uint4(0, 0, 0, 0);
    }
    // k in [0, ksplit) from the primary rows, k >= ksplit from rows `delta` elements away
    __device__ void load_split(int k0, int ksplit, ptrdiff_t delta) {
        const ptrdiff_t o = k0 < ksplit ? (ptrdiff_t)k0 : delta + (k0 - ksplit);
#pragma unroll
        for (int i = 0; i < PER; ++i)
            buf[i] = ptr[i] ? *reinterpret_cast<const uint4 *>(ptr[i] + o + chunk() * 8)
                            : make_uint4(0, 0, 0, 0);
    }
    __device__ void store(uint16_t *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            *reinterpret_cast<uint4 *>(lds + lds_off(row(i), chunk(), C::BK)) = buf[i];
    }
};

template <class C, int COLS>
struct TransTile {
    static constexpr int CB = COLS / 8;
    static constexpr int NBLK = (C::BK / 8) * CB;
    static constexpr int PER = (NBLK + C::NT - 1) / C::NT;
    uint4 buf[PER][8];

    __device__ static int blk(int i) { return (int)threadIdx.x + i * C::NT; }

    // f(k, c) -> pointer to element (k-row k, tile column c), c a multiple of 8,
    // or nullptr for zeros
    template <class F>
    __device__ void load(F &&f, int k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            if (NBLK % C::NT == 0 || b < NBLK) {
                const int kb = b / CB, cb = b % CB;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const uint16_t *p = f(k0 + kb * 8 + r, cb * 8);
                    buf[i][r] = p ? *reinterpret_cast<const uint4 *>(p) : make_uint4(0, 0, 0, 0);
                }
            }
        }
    }
    __device__ void store(uint16_t *lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = blk(i);
            if (NBLK % C::NT == 0 || b < NBLK) {
                const int kb = b / CB, cb = b % CB;
                const uint32_t *in = reinterpret_cast<const uint32_t *>(buf[i]);  // [8 k][4 dw]
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    uint4 o;
                    uint32_t *w = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t a = in[(2 * j) * 4 + (c >> 1)], bb = in[(2 * j + 1) * 4 + (c >> 1)];
                        w[j] = (c & 1) ? pack_hi16(a, bb) : pack_lo16(a, bb);
                    }
                    *reinterpret_cast<uint4 *>(lds + lds_off(cb * 8 + c, kb, C::BK)) = o;
                }
            }
        }
    }
};

// One BK stage of MFMAs. wrow(wn, fn) gives the LDS W row of n-block fn of wave wn.
template <class C, class P>
__device__ __forceinline__ void mma_stage(const uint16_t *stage, f32x16_t (&acc)[C::FM][C::FN], int wm,
                                          int wn, const P &p) {
    const uint16_t *xs = stage;
    const uint16_t *ws = stage + C::BM * C::BK;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
        bf16x8_t a[C::FN], b[C::FM];
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
            a[fn] = *reinterpret_cast<const bf16x8_t *>(ws + lds_off(p.wrow(wn, fn) + lr, kk * 2 + lh, C::BK));
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
            b[fm] = *reinterpret_cast<const bf16x8_t *>(xs + lds_off(wm * C::WM + fm * 32 + lr, kk * 2 + lh, C::BK));
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fn], b[fm], acc[fm][fn], 0, 0, 0);
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
