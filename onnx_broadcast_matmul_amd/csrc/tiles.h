// tiles.h -- tile table of the tiled MFMA kernels (host and device).
//
// Every entry runs 4 waves (256 threads) in a 2 x 2 arrangement, each wave
// owning a (bm/2) x (bn/2) sub-tile.  One LDS stage holds 128 bytes of K per
// row (64 elements of a 16-bit type, 32 of FP32).  The selector picks an
// entry per shape; tests force each one.
#pragma once

#include "internal.h"

namespace mm {

// FLOAT16 / BFLOAT16 entries.
constexpr TileCfg kTiles16[] = {
    {256, 256, 128, 128},
    {256, 128, 128, 64},
    {128, 128, 64, 64},
    {128, 64, 64, 32},
    {64, 64, 32, 32},
};

// FLOAT entries.
constexpr TileCfg kTiles32[] = {
    {128, 128, 64, 64},
    {128, 64, 64, 32},
    {64, 64, 32, 32},
};

constexpr int kNumTiles16 = sizeof(kTiles16) / sizeof(kTiles16[0]);
constexpr int kNumTiles32 = sizeof(kTiles32) / sizeof(kTiles32[0]);

// K elements held per LDS stage (one 128-byte row segment).
inline int stage_k(int dtype) { return dtype == MM_FLOAT ? 32 : 64; }

}  // namespace mm
