// k_gemm_t.hip -- launch switch of the tiled GEMM for Gemm plans: the same
// kernels as k_gemm.hip, instantiated with the alpha / beta / C epilogue and
// with A staged from its [K][M] layout and/or B from its [N][K] layout when
// transposed, for the tile subset kTransTiles16 / kTransTiles32.  A separate
// translation unit so the two sets of instantiations compile in parallel.
#include "k_gemm_impl.h"

namespace mm {

template <int DT, const TileCfg *T, int IDX>
static hipError_t launch_t_tile(bool vec, bool split, const KArgs &a, hipStream_t s) {
    constexpr TileCfg c = T[IDX];
    if (a.ta && a.tb)
        return launch_tile<DT, c.bm, c.bn, c.wgm, c.wgn, c.bkb, c.stages, c.producers, c.kgroups, true, true, true>(vec, split, a, s);
    if (a.ta)
        return launch_tile<DT, c.bm, c.bn, c.wgm, c.wgn, c.bkb, c.stages, c.producers, c.kgroups, true, false, true>(vec, split, a, s);
    if (a.tb)
        return launch_tile<DT, c.bm, c.bn, c.wgm, c.wgn, c.bkb, c.stages, c.producers, c.kgroups, false, true, true>(vec, split, a, s);
    return launch_tile<DT, c.bm, c.bn, c.wgm, c.wgn, c.bkb, c.stages, c.producers, c.kgroups, false, false, true>(vec, split, a, s);
}

static_assert(sizeof(kTransTiles16) / sizeof(int) == 6 && kTransTiles16[0] == 0 && kTransTiles16[1] == 5 &&
                  kTransTiles16[2] == 4 && kTransTiles16[3] == 2 && kTransTiles16[4] == 1 && kTransTiles16[5] == 13,
              "launch switch must cover the transposed tile subset");
static_assert(sizeof(kTransTiles32) / sizeof(int) == 5 && kTransTiles32[0] == 4 && kTransTiles32[1] == 2 &&
                  kTransTiles32[2] == 6 && kTransTiles32[3] == 5 && kTransTiles32[4] == 7,
              "launch switch must cover the transposed tile subset");

template <int DT>
static hipError_t launch_t16(int tile, bool vec, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
    case 0: return launch_t_tile<DT, kTiles16, 0>(vec, split, a, s);
    case 5: return launch_t_tile<DT, kTiles16, 5>(vec, split, a, s);
    case 4: return launch_t_tile<DT, kTiles16, 4>(vec, split, a, s);
    case 2: return launch_t_tile<DT, kTiles16, 2>(vec, split, a, s);
    case 1: return launch_t_tile<DT, kTiles16, 1>(vec, split, a, s);
    case 13: return launch_t_tile<DT, kTiles16, 13>(vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

static hipError_t launch_t32(int tile, bool vec, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
    case 4: return launch_t_tile<MM_FLOAT, kTiles32, 4>(vec, split, a, s);
    case 2: return launch_t_tile<MM_FLOAT, kTiles32, 2>(vec, split, a, s);
    case 6: return launch_t_tile<MM_FLOAT, kTiles32, 6>(vec, split, a, s);
    case 5: return launch_t_tile<MM_FLOAT, kTiles32, 5>(vec, split, a, s);
    case 7: return launch_t_tile<MM_FLOAT, kTiles32, 7>(vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_general_t(int dtype, int tile, const Align &al, bool split, const KArgs &a, hipStream_t s) {
    const bool vec = al.a && al.b;
    switch (dtype) {
    case MM_FLOAT: return launch_t32(tile, vec, split, a, s);
    case MM_FLOAT16: return launch_t16<MM_FLOAT16>(tile, vec, split, a, s);
    case MM_BFLOAT16: return launch_t16<MM_BFLOAT16>(tile, vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
