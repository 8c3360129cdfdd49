// internal.h -- structures shared by the host plan layer and the HIP kernels.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "mm.h"

namespace mm {

// Number of compute units the selector plans for (MI355X: 256 CUs in 8 XCDs).
constexpr int kNumCUs = 256;
constexpr int kNumXCDs = 8;

// Collapsed batch description: output batch index b is unravelled row-major
// over dim[0..nb); each operand's matrix starts at sum_d i_d * stride_d
// elements.  A zero stride reads the same matrix for every index along that
// dimension (broadcast without a copy).
struct BatchDesc {
    int32_t nb;
    int32_t pad_;
    int64_t dim[MM_MAX_BATCH_DIMS];
    int64_t sa[MM_MAX_BATCH_DIMS];
    int64_t sb[MM_MAX_BATCH_DIMS];
};

// Arguments of every kernel (passed by value).  M is the number of rows of
// one product as the kernels see it (batch*M when A's batch is folded into
// the rows).  Y is [batch][M][N] with rows ldy elements apart (batches M*ldy
// apart) and B's rows are ldb elements apart; both equal N except in the
// tiled kernels' column sub-launches, where N is the width of a column range
// of wider matrices.  W is the split-K workspace [split][batch][M][N] in
// FP32 (in double for DOUBLE products), always dense.
struct KArgs {
    const void *A;
    const void *B;
    void *Y;
    float *W;
    int64_t M, N, K;
    int64_t lda, ldb, ldy;  // row pitches of the stored A, stored B and Y, in elements
    int64_t batch;
    int64_t kchunk;
    int32_t split;
    int32_t y_vec;  // output rows (Y, or the workspace) are whole 16-byte chunks
    BatchDesc bd;
    // Gemm: A stored transposed ([K][M], lda = M) and/or B stored transposed
    // ([N][K], ldb = K); the kernels then read A'[m][k] = A[k][m] and
    // B'[k][n] = B[n][k].  The epilogue Y = alpha * acc + beta * C(m, n) is
    // applied when gemm_epi is set (C broadcast per c_mode, C's rows ldc
    // elements apart); MatMul leaves all of this zero.
    int32_t ta, tb;
    int32_t gemm_epi;
    int32_t c_mode;  // a GemmBias value
    float alpha, beta;
    const void *C;
    int64_t ldc;
    // MatMulInteger: UINT8 operands are fed to the signed INT8 matrix cores
    // with their sign bit flipped (x - 128); flip_a / flip_b are then
    // 0x80808080.  zpa / zpb are the zero points (a_signed / b_signed give
    // their type; zp_mode: 0 none, 1 scalar, 2 per row of A / per column of
    // B).  sum_a / sum_b ask the tiled kernel for the row sums of A' / the
    // column sums of B' (needed when the other operand's shifted zero point
    // can be non-zero); it forms them from the operand fragments it already
    // holds.
    uint32_t flip_a, flip_b;
    int32_t a_signed, b_signed;
    int32_t zpa_mode, zpb_mode;
    const void *zpa;
    const void *zpb;
    int32_t sum_a, sum_b;
    int64_t zp_rows;  // rows of one A matrix: a per-row zero point is indexed by row % zp_rows
    // Plan-owned constant B in the prepacked layout (b_packed = 1): for each
    // B matrix (bp_mat_bytes apart; matrix i starts at element i * bp_mat_elems
    // of the row-major B), for each tile column and K stage, the stage's B
    // panel exactly as the tiled kernel lays it out in LDS, zero-padded past
    // K and N.  Only the 16-bit MatMul tiles read it; other kernels read B.
    const void *Bp;
    int64_t bp_mat_bytes, bp_mat_elems;
    int32_t b_packed;
    int32_t pad1_;
};

// Layouts of the Gemm bias C, unidirectionally broadcast to (M, N).
enum GemmBias { kBiasNone = 0, kBiasScalar = 1, kBiasRow = 2, kBiasCol = 3, kBiasFull = 4 };

// Which operands allow 16-byte vector access: the base pointer is 16-byte
// aligned and every row starts on a 16-byte boundary (A: K elements per row;
// B and Y: N elements per row).
struct Align {
    bool a, b, y;
};

// Tile table entry of the tiled (MFMA) kernels.
struct TileCfg {
    int bm, bn;     // block tile
    int wgm, wgn;   // waves along M and N
    int bkb;        // bytes of K per row and LDS stage
    int stages;     // LDS stages
    int producers;  // waves that issue the global-to-LDS loads
    int kgroups;    // wave groups that split each stage's K steps (1: none)
    int persistent; // 1: one workgroup per CU walks the tiles (16-bit MatMul,
                    // two stages, one K group); other cases run the plain kernel
};

// Number of tile table entries and the entries, per element type.
int tile_count(int dtype);
const TileCfg *tile_entry(int dtype, int index);

// Kernel launchers (defined in the .hip files).  All return hipSuccess or
// the launch error.  `al` selects the 16-byte vectorized kernel variants
// where the operands they stream allow it.
hipError_t launch_direct(int dtype, const KArgs &a, hipStream_t s);
hipError_t launch_fill_zero(int dtype, void *Y, int64_t n, hipStream_t s);
hipError_t launch_general(int dtype, int tile, const Align &al, bool split, const KArgs &a, hipStream_t s);
// The same for Gemm plans (epilogue, transposed operands); only the
// kTransTiles entries.
hipError_t launch_general_t(int dtype, int tile, const Align &al, bool split, const KArgs &a, hipStream_t s);
hipError_t launch_splitk_reduce(int dtype, const KArgs &a, hipStream_t s);
// Prepack B columns [col0, col0 + ncols) of nmat row-major 16-bit [K][ldb]
// matrices (matrix i at element i * mat_elems) into the layout KArgs::Bp
// describes for a tile of bn columns (K stages of 64 elements); dst holds
// nmat * packed_b_bytes(ncols, K, bn) bytes.
hipError_t launch_pack_b(int bn, const void *B, int64_t nmat, int64_t mat_elems, int64_t K, int64_t ldb, int64_t col0,
                         int64_t ncols, void *dst, hipStream_t s);
int64_t packed_b_bytes(int64_t ncols, int64_t K, int bn);
hipError_t launch_skinny_m(int dtype, const Align &al, const KArgs &a, hipStream_t s);
hipError_t launch_skinny_n(int dtype, const Align &al, const KArgs &a, hipStream_t s);
// MatMulInteger kernels (k_int.hip): the direct kernel, the row / column
// sum passes (ra over a_rows rows of A, cb over b_mats B matrices; either
// may be NULL) and the INT8 tiled kernel for the kTiles8 entries.
hipError_t launch_int_direct(const KArgs &a, hipStream_t s);
hipError_t launch_general_int(int tile, bool split, const KArgs &a, hipStream_t s);
hipError_t launch_splitk_reduce_i32(const KArgs &a, hipStream_t s);
// DOUBLE kernels (k_f64.hip); W holds double partials for split-K.
hipError_t launch_direct_f64(const KArgs &a, hipStream_t s);
hipError_t launch_general_f64(int tile, const Align &al, bool split, const KArgs &a, hipStream_t s);
hipError_t launch_splitk_reduce_f64(const KArgs &a, hipStream_t s);

}  // namespace mm
