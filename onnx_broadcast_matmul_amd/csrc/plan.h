// plan.h -- the plan object behind mm_plan_t.
#pragma once

#include <stdarg.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

struct mm_plan_s {
    int dtype = 0;
    int a_rank = 0, b_rank = 0;
    int64_t a_shape[MM_MAX_RANK] = {};
    int64_t b_shape[MM_MAX_RANK] = {};
    int out_rank = 0;
    int64_t out_shape[MM_MAX_RANK] = {};
    int64_t out_numel = 0;
    int64_t M = 0, N = 0, K = 0;  // promoted sizes of one product
    int64_t total_batch = 0;      // broadcast batch count before folding
    int64_t batch = 0;            // products launched (1 when folded)
    int64_t kernel_m = 0;         // rows per launched product
    int folded = 0;
    mm::BatchDesc bd = {};
    int algo = MM_ALGO_EMPTY;
    int tile = -1;  // tile table index (tiled algorithms)
    // GENERAL only: when tail_col > 0, the tile `tile` covers output columns
    // [0, tail_col) in whole rounds of workgroups and a second launch with
    // tile `tail_tile` covers [tail_col, N).
    int64_t tail_col = 0;
    int tail_tile = -1;
    int32_t split = 1;
    int64_t kchunk = 0;
    int64_t workspace_bytes = 0;

    // Device workspace for split-K and a split skinny-M, allocated by plan
    // creation on the current device (by the first execution when creation
    // found no GPU).
    std::mutex ws_mutex;
    void *ws = nullptr;
    int ws_device = -1;

    // Gemm (mm_gemm_plan_create): transposed operands, epilogue, C layout.
    bool is_gemm = false;
    int ta = 0, tb = 0;
    float alpha = 1.0f, beta = 0.0f;
    int c_mode = 0;  // mm::GemmBias
    int64_t ldc = 0;

    // MatMulInteger (mm_int_plan_create): operand types, zero-point kinds and
    // the row / column sums the zero points need (formed by the tiled kernel).
    bool is_int = false;
    int a_type = 0, b_type = 0;
    int zpa_kind = 0, zpb_kind = 0;
    bool need_ra = false, need_cb = false;

    // Plan-owned constant B (mm_plan_set_constant_b).
    std::mutex cb_mutex;
    bool cb_set = false;
    void *cb = nullptr;
    int cb_device = -1;
    int64_t b_numel = 0;  // elements of the planned B tensor
    // The same B prepacked for the tiled 16-bit kernel (see KArgs::Bp): the
    // columns of `tile` (all of N, or [0, tail_col)) then those of
    // `tail_tile`, cbp_main and cbp_tail bytes per B matrix.
    void *cbp = nullptr;
    size_t cbp_bytes = 0;
    bool cbp_ok = false;
    int64_t cbp_main = 0, cbp_tail = 0;
};

namespace mm {
// Allocate the plan's split workspace on the current device (execute.cpp).
// At creation a host without a GPU is not an error: the first execution
// allocates instead.
mm_status alloc_workspace(mm_plan_s *p, bool at_create);
// Enqueue a MatMul or Gemm plan (C: the Gemm bias or NULL); split partial
// sums go to `ws` when it is not NULL, else to the plan's workspace.
// packed_b: read B's prepacked copy (the plan's constant B) where the tiled
// 16-bit kernel runs; B must then be the plan's row-major constant B.
mm_status execute_plan(mm_plan_s *p, const void *A, const void *B, const void *C, void *Y, void *stream, void *ws,
                       bool packed_b = false);
mm_status fail(mm_status st, const char *fmt, ...);
void clear_error();
int elem_size(int dtype);
}  // namespace mm
