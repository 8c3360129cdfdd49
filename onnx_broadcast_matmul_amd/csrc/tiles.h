// tiles.h -- tile table of the tiled MFMA kernels (host and device).
//
// An entry is a block tile bm x bn run by wgm x wgn waves, each wave owning a
// (bm/wgm) x (bn/wgn) sub-tile; with kgroups > 1 there are kgroups such sets
// of waves, each taking every kgroups-th MFMA step of a stage, and their
// accumulators are added in group order before the epilogue.  Eight waves put two waves on every SIMD, so
// one wave's MFMAs cover the other's LDS and barrier waits.  The vectorized
// kernel stages bkb bytes of K per row (64 elements of a 16-bit type, 32 of
// FP32 for bkb = 128) in `stages` LDS buffers, filled by the first
// `producers` waves.  An entry marked persistent runs one workgroup per CU
// over many tiles (k_gemm_persist) where the shape allows it, and the
// one-tile kernel of the same shape elsewhere.  The element-wise fallback
// kernel uses the block tile only.  The selector picks an entry per shape;
// tests force each one.
#pragma once

#include "internal.h"

namespace mm {

// FLOAT16 / BFLOAT16 entries.
constexpr TileCfg kTiles16[] = {
    {256, 256, 2, 4, 128, 2, 4, 1},
    {256, 128, 2, 2, 128, 3, 4, 1},
    {128, 128, 2, 2, 128, 3, 4, 1},
    {128, 64, 2, 2, 128, 3, 4, 1},
    {64, 64, 2, 2, 128, 3, 4, 1},
    {128, 128, 2, 2, 128, 2, 4, 1},
    {128, 256, 2, 4, 128, 2, 4, 1},
    {256, 128, 4, 2, 128, 2, 4, 1},
    {64, 64, 2, 2, 128, 3, 4, 2},
    {128, 128, 2, 2, 128, 2, 4, 2},
    {256, 256, 2, 4, 128, 2, 4, 1, 1},
    // Entries for products of at most 64 rows, where one row tile spans M
    // and the kernel streams B: 128 or 256 columns per tile give each wave
    // longer contiguous B rows per stage than the 64-column tiles.
    {32, 128, 1, 4, 128, 3, 4, 1},
    {32, 256, 1, 4, 128, 3, 4, 1},
    {64, 128, 2, 2, 128, 3, 4, 1},
};

// FLOAT entries.
constexpr TileCfg kTiles32[] = {
    {128, 128, 2, 2, 128, 3, 4, 1},
    {128, 64, 2, 2, 128, 3, 4, 1},
    {64, 64, 2, 2, 128, 3, 4, 1},
    {256, 128, 2, 4, 128, 3, 4, 1},
    {128, 128, 2, 2, 128, 2, 4, 1},
    {64, 64, 2, 2, 128, 3, 4, 2},
    {128, 128, 2, 2, 128, 2, 4, 2},
    // For products of at most 32 rows: one row tile spans M, so the FP32
    // matrix-core work is not padded to 64 rows.
    {32, 128, 1, 4, 128, 3, 4, 2},
};

// DOUBLE entries (k_f64.hip: 4 waves, 16 doubles of K per stage, two
// register-staged LDS buffers; the wave, stage and producer fields are those
// of that kernel).
constexpr TileCfg kTiles64[] = {
    {128, 128, 2, 2, 128, 2, 4, 1},
    {64, 64, 2, 2, 128, 2, 4, 1},
    {32, 128, 2, 2, 128, 2, 4, 1},  // products of at most 32 rows
};

// Entries instantiated for Gemm (its epilogue and transA / transB).
constexpr int kTransTiles16[] = {0, 5, 4, 2, 1, 13};
constexpr int kTransTiles32[] = {4, 2, 6, 5, 7};

// INT8 entries (MatMulInteger; B rows need at least 128 bytes per stage row).
// The two 256 x 256 entries differ in wave layout: 2 x 4 waves hold two B
// fragments each, 4 x 2 waves two A fragments, so a UINT8 A (whose
// fragments are sign-flipped after every read) takes the second.
constexpr TileCfg kTiles8[] = {
    {256, 256, 2, 4, 128, 2, 4, 1},
    {128, 128, 2, 2, 128, 2, 4, 1},
    {256, 256, 4, 2, 128, 2, 4, 1},
    // Split-K (and few-row) entries: three stages deep for short K chunks.
    {64, 128, 2, 2, 128, 3, 4, 1},
    {128, 128, 2, 2, 128, 3, 4, 1},
};

constexpr int kNumTiles16 = sizeof(kTiles16) / sizeof(kTiles16[0]);
constexpr int kNumTiles32 = sizeof(kTiles32) / sizeof(kTiles32[0]);
constexpr int kNumTiles64 = sizeof(kTiles64) / sizeof(kTiles64[0]);
constexpr int kNumTiles8 = sizeof(kTiles8) / sizeof(kTiles8[0]);

// K granularity of split-K partitions: 128 bytes of K, a whole number of
// LDS stages of every tile entry.
inline int stage_k(int dtype) {
    if (dtype == MM_INT8 || dtype == MM_UINT8 || dtype == MM_INT32) return 128;  // MatMulInteger
    return dtype == MM_DOUBLE ? 16 : dtype == MM_FLOAT ? 32 : 64;
}
constexpr bool stages_divide_128() {
    for (const TileCfg &t : kTiles16)
        if (128 % t.bkb != 0) return false;
    for (const TileCfg &t : kTiles32)
        if (128 % t.bkb != 0) return false;
    return true;
}
static_assert(stages_divide_128(), "split-K granularity must be a whole number of stages");

}  // namespace mm
