// Tile lists of the bf16 grouped GEMM, built by one wave64 from the expert
// counts and offsets it holds (4 consecutive experts per lane, E <= 256).
// Used by the standalone plan kernel and at the end of the dispatch kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

constexpr int kMfmaBigRows = 256;

// List layout (ints): big tiles expert[max_mt], row0[max_mt], rows[max_mt],
// count; then the same for the 64-row tiles with max_st entries.
struct MfmaPlanArgs {
    int32_t* tiles;     // null: no plan
    int tau, tile_mode, max_mt, max_st;
};

// Per expert with more than tau rows: 256-row tiles when the tile mode says
// so (BIG, or BOTH with more than 128 rows), else 64-row tiles; exclusive
// scans over the experts place them, in expert order.
__device__ __forceinline__ void mfma_plan_wave(int lane, const int (&c)[4], const int (&o)[4], int E,
                                               const MfmaPlanArgs& p) {
    int nb[4], ns[4], sb = 0, ss = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        nb[j] = 0;
        ns[j] = 0;
        if (e < E && c[j] > p.tau && c[j] > 0) {
            const bool big = p.tile_mode == MFMA_TILES_BIG ||
                             (p.tile_mode == MFMA_TILES_BOTH && c[j] > 2 * kMfmaSmallRows);
            if (big) nb[j] = (c[j] + kMfmaBigRows - 1) / kMfmaBigRows;
            else ns[j] = (c[j] + kMfmaSmallRows - 1) / kMfmaSmallRows;
        }
        sb += nb[j];
        ss += ns[j];
    }
    int ib = sb, is = ss;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int vb = __shfl_up(ib, d, 64), vs = __shfl_up(is, d, 64);
        if (lane >= d) { ib += vb; is += vs; }
    }
    int b = ib - sb, s = is - ss;
    int32_t* big = p.tiles;
    int32_t* small = p.tiles + 3 * p.max_mt + 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        for (int i = 0; i < nb[j]; ++i) {
            big[b + i] = e;
            big[p.max_mt + b + i] = o[j] + i * kMfmaBigRows;
            big[2 * p.max_mt + b + i] = min(kMfmaBigRows, c[j] - i * kMfmaBigRows);
        }
        for (int i = 0; i < ns[j]; ++i) {
            small[s + i] = e;
            small[p.max_st + s + i] = o[j] + i * kMfmaSmallRows;
            small[2 * p.max_st + s + i] = min(kMfmaSmallRows, c[j] - i * kMfmaSmallRows);
        }
        b += nb[j];
        s += ns[j];
    }
    if (lane == 63) {
        big[3 * p.max_mt] = ib;
        small[3 * p.max_st] = is;
    }
}

}  // namespace moe
