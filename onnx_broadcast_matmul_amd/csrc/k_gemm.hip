// k_gemm.hip -- launch switch of the tiled GEMM over the tile table (A and
// B in their MatMul layouts); the kernels are in k_gemm_impl.h.
#include "k_gemm_impl.h"

namespace mm {

#define MM_TILE_CASE(DT, T, IDX)                                                                          \
    case IDX:                                                                                             \
        return launch_tile<DT, T[IDX].bm, T[IDX].bn, T[IDX].wgm, T[IDX].wgn, T[IDX].bkb, T[IDX].stages, \
                           T[IDX].producers, T[IDX].kgroups>(vec, split, a, s)

template <int DT>
static hipError_t launch_16(int tile, bool vec, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
        MM_TILE_CASE(DT, kTiles16, 0);
        MM_TILE_CASE(DT, kTiles16, 1);
        MM_TILE_CASE(DT, kTiles16, 2);
        MM_TILE_CASE(DT, kTiles16, 3);
        MM_TILE_CASE(DT, kTiles16, 4);
        MM_TILE_CASE(DT, kTiles16, 5);
        MM_TILE_CASE(DT, kTiles16, 6);
        MM_TILE_CASE(DT, kTiles16, 7);
        MM_TILE_CASE(DT, kTiles16, 8);
        MM_TILE_CASE(DT, kTiles16, 9);
    }
    return hipErrorInvalidValue;
}

static hipError_t launch_32(int tile, bool vec, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
        MM_TILE_CASE(MM_FLOAT, kTiles32, 0);
        MM_TILE_CASE(MM_FLOAT, kTiles32, 1);
        MM_TILE_CASE(MM_FLOAT, kTiles32, 2);
        MM_TILE_CASE(MM_FLOAT, kTiles32, 3);
        MM_TILE_CASE(MM_FLOAT, kTiles32, 4);
        MM_TILE_CASE(MM_FLOAT, kTiles32, 5);
        MM_TILE_CASE(MM_FLOAT, kTiles32, 6);
    }
    return hipErrorInvalidValue;
}
#undef MM_TILE_CASE

static_assert(kNumTiles16 == 10 && kNumTiles32 == 7, "launch switch must cover the tile table");

hipError_t launch_general(int dtype, int tile, const Align &al, bool split, const KArgs &a, hipStream_t s) {
    if (a.gemm_epi || a.ta || a.tb) return launch_general_t(dtype, tile, al, split, a, s);
    const bool vec = al.a && al.b;
    switch (dtype) {
    case MM_FLOAT: return launch_32(tile, vec, split, a, s);
    case MM_FLOAT16: return launch_16<MM_FLOAT16>(tile, vec, split, a, s);
    case MM_BFLOAT16: return launch_16<MM_BFLOAT16>(tile, vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
