// k_gemm.hip -- launch switch of the tiled GEMM over the tile table (A and
// B in their MatMul layouts); the kernels are in k_gemm_impl.h.
#include "k_gemm_impl.h"

namespace mm {

#define MM_TILE_CASE(DT, T, IDX)                                                                          \
    case IDX:                                                                                             \
        return launch_tile<DT, T[IDX].bm, T[IDX].bn, T[IDX].wgm, T[IDX].wgn, T[IDX].bkb, T[IDX].stages, \
                           T[IDX].producers, T[IDX].kgroups, false, false, false, T[IDX].persistent != 0>(vec, split, a, s)

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
        MM_TILE_CASE(DT, kTiles16, 10);
        MM_TILE_CASE(DT, kTiles16, 11);
        MM_TILE_CASE(DT, kTiles16, 12);
        MM_TILE_CASE(DT, kTiles16, 13);
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
        MM_TILE_CASE(MM_FLOAT, kTiles32, 7);
    }
    return hipErrorInvalidValue;
}
#undef MM_TILE_CASE

static_assert(kNumTiles16 == 14 && kNumTiles32 == 8, "launch switch must cover the tile table");

// Prepacked constant B: the 16-byte chunk (piece, lane) of the panel of
// matrix mi, tile column tn and K stage st is what lane `lane` of load
// `piece` of that stage puts in LDS: k-row piece * rpb + lane / cpr of the
// stage, chunk position lane % cpr, i.e. chunk (lane % cpr) ^
// kn_swizzle<2>(row, cpr) of the tile's columns in that row.
template <int BN>
__global__ __launch_bounds__(256) void k_pack_b(const uint16_t *__restrict__ B, int64_t nmat, int64_t mat_elems,
                                                int64_t K, int64_t ldb, int64_t col0, int64_t ncols,
                                                uint4 *__restrict__ dst) {
    constexpr int BK = 64, RBB = BN * 2, CPR = RBB / 16, RPB = 1024 / RBB;
    constexpr int64_t PANEL = (int64_t)BK * RBB / 16;  // chunks per panel
    const int64_t ntn = (ncols + BN - 1) / BN, nst = (K + BK - 1) / BK;
    const int64_t total = nmat * ntn * nst * PANEL;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t chunk = i % PANEL, panel = i / PANEL;
        const int64_t st = panel % nst, t = panel / nst;
        const int64_t tn = t % ntn, mi = t / ntn;
        const int piece = (int)(chunk / 64), lane = (int)(chunk % 64);
        const int row = piece * RPB + lane / CPR;
        const int c = (lane % CPR) ^ kn_swizzle<2>(row, CPR);
        const int64_t k = st * BK + row, n = tn * BN + (int64_t)c * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k < K && n < ncols) v = *(const uint4 *)(B + mi * mat_elems + k * ldb + col0 + n);
        dst[i] = v;
    }
}

int64_t packed_b_bytes(int64_t ncols, int64_t K, int bn) {
    return ((ncols + bn - 1) / bn) * ((K + 63) / 64) * 64 * (int64_t)bn * 2;
}

hipError_t launch_pack_b(int bn, const void *B, int64_t nmat, int64_t mat_elems, int64_t K, int64_t ldb, int64_t col0,
                         int64_t ncols, void *dst, hipStream_t s) {
    const int64_t chunks = nmat * packed_b_bytes(ncols, K, bn) / 16;
    if (chunks <= 0) return hipSuccess;
    int64_t g = (chunks + 255) / 256;
    if (g > 65536) g = 65536;
    const uint16_t *b = (const uint16_t *)B;
    uint4 *d = (uint4 *)dst;
    switch (bn) {
    case 256: hipLaunchKernelGGL(k_pack_b<256>, dim3((unsigned)g), dim3(256), 0, s, b, nmat, mat_elems, K, ldb, col0, ncols, d); break;
    case 128: hipLaunchKernelGGL(k_pack_b<128>, dim3((unsigned)g), dim3(256), 0, s, b, nmat, mat_elems, K, ldb, col0, ncols, d); break;
    case 64: hipLaunchKernelGGL(k_pack_b<64>, dim3((unsigned)g), dim3(256), 0, s, b, nmat, mat_elems, K, ldb, col0, ncols, d); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

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
