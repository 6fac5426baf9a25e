// GEMM tile family, chosen from the layer shape only (never from a knob), so
// that the bits of every result are independent of the mini-batch,
// macro-batch, ring and capacity settings.
#pragma once
#include <cstdint>

namespace mok {

constexpr int kMaxExperts = 4096;
// Output columns per tile of every segment GEMM (BF16 and MXFP8 alike).
constexpr int kTileN = 256;

struct TileChoice {
    int BM;      // routed rows per m-tile of the segment GEMMs
    int da_wn;   // columns of I summed into one router-grad partial
};

// BF16 layers whose experts average at most 128 routed rows (many small
// groups) take 128-row m-tiles: their grouped GEMMs stream each expert's
// weights once at low arithmetic intensity, so they are bound by HBM, and the
// smaller row tile leaves LDS for a deeper weight pipeline. Larger groups keep
// 256-row tiles (bound by the matrix cores). No result depends on the choice:
// every output element sums its K products in the same order either way.
inline TileChoice choose_tiles(int H, int I, int E, int k, int64_t T, int precision) {
    (void)H; (void)I;
    const bool small_groups = T * (int64_t)k <= 128 * (int64_t)E;
    return TileChoice{precision == 0 && small_groups ? 128 : 256, 64};
}

}  // namespace mok
