/*
 * mm.h -- C ABI of the MI355X (gfx950) ONNX MatMul library (libmm.so).
 *
 * The operation is ONNX MatMul as described on the page "MatMul Kernel
 * Design" (sections "Shape and plan model", "Types and algorithm selection",
 * "Scheduling and invariants") and on the page "Gemm and MatMul Performance
 * Roadmap" (sections "Target computation algorithm", "Planning once, computing
 * many times", "Parallel execution", "Phase 4: complete MatMul"):
 *
 *   Y[i, m, n] = sum_k A[iA(i), m, k] * B[iB(i), k, n]
 *
 * with a rank-one A ([K], used as [1, K]) or B ([K], used as [K, 1]) promoted
 * for the product and its axis removed from the output, and the leading batch
 * dimensions broadcast NumPy style (right-aligned, 1 stretches, otherwise
 * equal).  Inputs and output share one element type; FLOAT16 and BFLOAT16
 * products accumulate in FP32 and are narrowed once, at the end, with
 * round-to-nearest-even.  DOUBLE products accumulate in double on the FP64
 * matrix cores (page "MatMul Kernel Design", section "Types and algorithm
 * selection": the adapter takes DOUBLE with the same shape rules).
 *
 * Usage: create a plan once per (A shape, B shape, type); execute it any
 * number of times on device buffers; destroy it.  Every shape/type error is
 * reported by plan creation, before compute.  Plan creation makes no GPU
 * call except for a plan that needs a workspace (below), which it allocates.
 *
 * Layout: A, B and Y are dense, contiguous, row-major device tensors with the
 * ONNX shapes given at plan creation (Y has the plan's output shape).
 * Broadcast operands are read in place through zero batch strides; nothing is
 * copied or widened.
 *
 * Ownership: the caller owns A, B and Y and keeps them alive until the work
 * enqueued on the stream has completed.  The plan owns its metadata and, for
 * the split-K algorithm and a skinny-M plan that cuts K (split_k > 1 in
 * mm_plan_info), an FP32 (DOUBLE: double) workspace of
 * mm_plan_workspace_bytes() bytes, allocated by plan creation on the current
 * device and freed by mm_plan_destroy (page "Gemm and MatMul Performance
 * Roadmap", section "Planning once, computing many times": what the chosen
 * algorithm and its parallel decomposition need is prepared with the plan,
 * and execution only invokes it).  On a host where
 * creation finds no GPU, the first execution allocates it instead.  Because
 * of that workspace, executions of such a plan must not overlap on different
 * streams; use one plan per stream.  A plan executes on the device that
 * holds its workspace (another device gives MM_ERR_HIP).  Executions
 * allocate nothing once the workspace exists, so a plan created before a
 * HIP graph capture may be executed inside it.
 *
 * Threading: plans are immutable after creation apart from a workspace that
 * the first execution allocates, which is guarded; mm_last_error() is per
 * thread.
 */
#ifndef MM_H
#define MM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Maximum number of broadcast batch dimensions; inputs may have rank up to
 * MM_MAX_BATCH_DIMS + 2. */
#define MM_MAX_BATCH_DIMS 8
#define MM_MAX_RANK (MM_MAX_BATCH_DIMS + 2)

/* Element types: the ONNX TensorProto codes.  DOUBLE has no skinny-M /
 * skinny-N kernels: the plan runs its skinny shapes on the tiled FP64 kernel,
 * and forcing SKINNY_M or SKINNY_N for DOUBLE gives MM_ERR_BAD_OPTION. */
typedef enum mm_dtype {
    MM_FLOAT = 1,
    MM_UINT8 = 2,  /* MatMulInteger inputs */
    MM_INT8 = 3,   /* MatMulInteger inputs */
    MM_INT32 = 6,  /* MatMulInteger output */
    MM_FLOAT16 = 10,
    MM_DOUBLE = 11,
    MM_BFLOAT16 = 16
} mm_dtype;

typedef enum mm_status {
    MM_OK = 0,
    MM_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
    MM_ERR_RANK = 2,         /* rank 0, or rank above MM_MAX_RANK */
    MM_ERR_NEG_DIM = 3,      /* a dimension is negative (dynamic) */
    MM_ERR_K_MISMATCH = 4,   /* A's last dim differs from B's second-to-last */
    MM_ERR_BROADCAST = 5,    /* batch dimensions cannot be broadcast */
    MM_ERR_DTYPE = 6,        /* unsupported or unknown element type */
    MM_ERR_BAD_OPTION = 7,   /* invalid mm_plan_options field */
    MM_ERR_TOO_LARGE = 8,    /* a size exceeds what the kernels index */
    MM_ERR_ALLOC = 9,        /* host or device allocation failed */
    MM_ERR_HIP = 10,         /* a HIP runtime call failed (see mm_last_error) */
    MM_ERR_SIZE = 11,        /* a constant B whose element count is not the planned B's */
    MM_ERR_NO_CONSTANT_B = 12 /* mm_execute_constant_b on a plan that owns no B */
} mm_status;

/* Algorithms (page "Gemm and MatMul Performance Roadmap", section "Target
 * computation algorithm", the shape-to-algorithm table; page "MatMul Kernel
 * Design", section "Types and algorithm selection"). */
typedef enum mm_algo {
    MM_ALGO_AUTO = 0,      /* let the plan choose (only valid as an option) */
    MM_ALGO_EMPTY = 1,     /* output has no element: nothing is launched */
    MM_ALGO_ZERO_FILL = 2, /* K == 0: the output is filled with zeros */
    MM_ALGO_DIRECT = 3,    /* tiny products: one thread per output */
    MM_ALGO_SKINNY_M = 4,  /* small M (GEMV): B streamed once along N; K may be cut
                              into chunks (FP32 partials + ordered reduce) */
    MM_ALGO_SKINNY_N = 5,  /* small N: A streamed once along K */
    MM_ALGO_SPLIT_K = 6,   /* tiny output, long K: FP32 (DOUBLE: double) partials + ordered reduce */
    MM_ALGO_GENERAL = 7    /* tiled MFMA GEMM with LDS double buffering */
} mm_algo;

typedef struct mm_plan_s *mm_plan_t;

/* Overrides for tests and tuning.  Zero-initialise for defaults. */
typedef struct mm_plan_options {
    int32_t force_algo; /* MM_ALGO_AUTO, or one of DIRECT..GENERAL; ignored
                           (EMPTY / ZERO_FILL kept) when the output is empty
                           or K == 0 */
    int32_t tile;       /* 0 = plan's choice; k >= 1 selects entry k-1 of the
                           GENERAL/SPLIT_K tile table for the element type
                           (see mm_tile_config) */
    int32_t split_k;    /* 0 = plan's choice; >= 1 number of K partitions for
                           SPLIT_K and SKINNY_M (clamped so every partition is
                           non-empty; SKINNY_M partitions hold whole 64-row
                           chunks of K) */
    int32_t reserved;   /* must be 0 */
} mm_plan_options;

/* Everything the plan resolved, for inspection and tests. */
typedef struct mm_plan_info {
    int32_t dtype;
    int32_t algo;             /* mm_algo actually selected */
    int64_t M, N, K;          /* promoted matrix sizes of one product */
    int64_t batch;            /* independent products launched (after collapse/fold) */
    int64_t kernel_m;         /* rows per product seen by the kernels (batch*M when folded) */
    int32_t folded;           /* 1 if A's batch was folded into M (B shared by every batch) */
    int32_t batch_rank;       /* number of collapsed batch dimensions */
    int64_t batch_dims[MM_MAX_BATCH_DIMS];
    int64_t a_batch_strides[MM_MAX_BATCH_DIMS]; /* elements; 0 = broadcast */
    int64_t b_batch_strides[MM_MAX_BATCH_DIMS]; /* elements; 0 = broadcast */
    int32_t tile;             /* tile table entry + 1 (0 if not a tiled algorithm) */
    int32_t split_k;          /* K partitions (1 unless SPLIT_K or a split SKINNY_M) */
    int64_t k_chunk;          /* K elements per partition */
    int64_t workspace_bytes;  /* workspace the plan needs on the device (FP32 or double partials) */
    double flops;             /* 2 * batch * M * N * K of the un-folded problem */
    double min_bytes;         /* element size * (numel A + numel B + numel Y) */
    int64_t tail_col;         /* GENERAL: > 0 when output columns [tail_col, N) run as a
                                 second launch (last-round balancing), else 0 */
    int32_t tail_tile;        /* tile table entry + 1 of that second launch (0 if none) */
    int32_t constant_b_packed; /* 1 if the plan holds a constant B also in the prepacked layout */
} mm_plan_info;

/* Create a plan for Y = MatMul(A, B) with A of shape a_shape[0..a_rank) and
 * B of shape b_shape[0..b_rank), all of type `dtype`.  Validates ranks
 * (1..MM_MAX_RANK), dimensions (>= 0), the inner dimension, batch
 * broadcasting and the type; resolves the output shape, collapsed batch
 * strides and the algorithm.  A plan that needs a workspace allocates it on
 * the current device (MM_ERR_ALLOC if that fails; skipped on a host without
 * a GPU); no other GPU call is made.  On error *out is set to NULL and a
 * status is returned (details: mm_last_error()). */
mm_status mm_plan_create(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank,
                         int dtype, mm_plan_t *out);

/* As mm_plan_create, with overrides (NULL = defaults). */
mm_status mm_plan_create_ex(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank,
                            int dtype, const mm_plan_options *opt, mm_plan_t *out);

/* Release a plan and its device workspace.  NULL is ignored.  The caller
 * must make sure no enqueued execution of the plan is still running. */
void mm_plan_destroy(mm_plan_t plan);

/* Enqueue Y = MatMul(A, B) on `stream` (a hipStream_t; NULL = the null
 * stream of the current device).  A, B, Y are device pointers to tensors of
 * the planned shapes and type.  Returns after enqueueing; results are ready
 * when the stream reaches this point.  Empty output: nothing is launched and
 * the pointers may be NULL.  K == 0: A and B are not read (may be NULL) and Y
 * is filled with zeros.  Otherwise NULL A, B or Y gives MM_ERR_NULL_ARG.
 * Pointers need no particular alignment (16-byte aligned buffers take the
 * vectorized kernels).  MM_ERR_HIP reports a failed launch or allocation. */
mm_status mm_execute(mm_plan_t plan, const void *A, const void *B, void *Y, void *stream);

/* mm_execute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels, but a split plan's partial sums go to a fixed 16 MiB device
 * array that the library holds on every device it runs on for the life of
 * the process, instead of the plan's workspace; the call itself allocates
 * nothing.  A plan whose workspace exceeds 16 MiB gives MM_ERR_TOO_LARGE
 * (nothing is launched); plans without a workspace run exactly as with
 * mm_execute.  All calls on one device share that array: calls that overlap
 * on a device (other streams, other threads) race and must be serialised by
 * the caller.  Other arguments and errors as for mm_execute. */
mm_status mm_execute_noalloc(mm_plan_t plan, const void *A, const void *B, void *Y, void *stream);

/* Constant B (page "MatMul Kernel Design": the reusable plan can own a
 * constant B, giving callers a lifetime independent of the source buffer;
 * that storage must hold exactly the planned matrix, and the B-less execute
 * is rejected when the plan owns no B).
 *
 * mm_plan_set_constant_b copies `numel` elements of the planned type from
 * the device buffer B (the dense B tensor of the planned shape) into device
 * memory the plan owns, on the current device, ordered on `stream` (a
 * hipStream_t; NULL = null stream), and returns once the copy has completed:
 * the caller may then reuse or free B.  Calling it again replaces the
 * contents.  Errors: MM_ERR_NULL_ARG (NULL plan, or NULL B with numel > 0),
 * MM_ERR_BAD_OPTION (a Gemm or MatMulInteger plan: constant B serves
 * mm_execute only), MM_ERR_SIZE (numel differs from the planned B's element
 * count),
 * MM_ERR_ALLOC, MM_ERR_HIP (copy failed, or the plan already holds B on
 * another device).  The storage is freed by mm_plan_destroy.
 *
 * For a FLOAT16 / BFLOAT16 plan on the GENERAL algorithm with N a multiple
 * of 8, mm_plan_set_constant_b also lays B out once in the tiled kernel's
 * stage order (page "Gemm and MatMul Performance Roadmap", section "Target
 * computation algorithm": a constant B prepacked once when its shape and
 * layout are stable; section "Remaining pull-request sequence", PR06.4): for
 * every tile column and K stage, that stage's B panel exactly as the kernel
 * stages it in LDS, zero-padded past K and N (mm_plan_info
 * constant_b_packed = 1).  This takes about as much device memory again as
 * B and is rebuilt by every call.
 *
 * mm_execute_constant_b is mm_execute with B taken from that storage (the
 * prepacked copy where the tiled kernel runs, the plain copy elsewhere; the
 * results are the same bits).  It gives MM_ERR_NO_CONSTANT_B when the plan
 * owns no B, and MM_ERR_HIP when called on a device other than the one
 * holding it.  A plan with a constant B may still be executed with an
 * explicit B through mm_execute. */
mm_status mm_plan_set_constant_b(mm_plan_t plan, const void *B, int64_t numel, void *stream);

/* 1 if the plan owns a constant B, 0 if not (or for a NULL plan). */
int mm_plan_has_constant_b(mm_plan_t plan);

mm_status mm_execute_constant_b(mm_plan_t plan, const void *A, void *Y, void *stream);

/* ONNX Gemm on the same engine (page "Gemm and MatMul Performance Roadmap",
 * section "Scope and type matrix": Gemm takes rank-2 inputs, alpha, beta,
 * an optional broadcast bias and transA / transB; section "Remaining
 * pull-request sequence", PR02: no, scalar, row, column and full C layouts
 * are consumed directly, with no expanded M x N bias):
 *
 *   Y[m][n] = alpha * sum_k A'[m][k] * B'[k][n] + beta * C(m, n)
 *
 * A' = A ([M, K]) or, with trans_a, A stored [K, M] read transposed; B' = B
 * ([K, N]) or, with trans_b, B stored [N, K] read transposed.  C is absent
 * (c_rank = -1: Y = alpha * A'B') or has rank 0..2 and broadcasts
 * unidirectionally to [M, N]: [] / [1] / [1, 1] scalar, [N] / [1, N] one
 * value per column, [M, 1] one value per row, [M, N] full.  A, B, C and Y
 * share the element type (FLOAT, FLOAT16 or BFLOAT16; DOUBLE gives
 * MM_ERR_DTYPE); 16-bit types accumulate in FP32 and alpha * sum + beta * c
 * is formed in FP32 before the single narrowing.  Y is dense [M, N]. */
typedef struct mm_gemm_desc {
    int64_t a_rows, a_cols; /* stored A shape */
    int64_t b_rows, b_cols; /* stored B shape */
    int32_t trans_a, trans_b;
    int32_t c_rank;         /* -1 (no C), 0, 1 or 2 */
    int32_t reserved;       /* must be 0 */
    int64_t c_shape[2];     /* the first c_rank entries are used */
    float alpha, beta;
} mm_gemm_desc;

/* Create a Gemm plan (shapes, transposes, C's layout and the algorithm are
 * resolved once; errors as for mm_plan_create, plus MM_ERR_BROADCAST for a
 * C that does not broadcast to [M, N] and MM_ERR_BAD_OPTION for an invalid
 * descriptor or an option the Gemm path does not run: forced SKINNY_M /
 * SKINNY_N, or a tile outside the Gemm subset of the tile table).  `opt` may be NULL.  The plan answers the introspection
 * calls above (output shape [M, N]). */
mm_status mm_gemm_plan_create(const mm_gemm_desc *desc, int dtype, const mm_plan_options *opt, mm_plan_t *out);

/* Enqueue Y = Gemm(A, B, C) on `stream`.  C must be non-NULL exactly when
 * the plan has one (else MM_ERR_NULL_ARG); K == 0 gives Y = beta * C (or
 * zeros) without reading A or B.  Other rules as for mm_execute.  A Gemm
 * plan is refused by mm_execute and a MatMul plan by mm_gemm_execute
 * (MM_ERR_BAD_OPTION). */
mm_status mm_gemm_execute(mm_plan_t plan, const void *A, const void *B, const void *C, void *Y, void *stream);

/* MatMulInteger (page "Gemm and MatMul Performance Roadmap", section
 * "Remaining pull-request sequence", Roadmap PR09.1: mixed INT8 / UINT8 operands,
 * optional scalar or per-row / per-column zero points, the MatMul batch
 * broadcasting and rank-one rules, and INT32 accumulation defined as
 * arithmetic modulo 2^32):
 *
 *   Y[i, m, n] = sum_k (A[iA(i), m, k] - za) * (B[iB(i), k, n] - zb)
 *
 * a_type / b_type: MM_UINT8 or MM_INT8.  Zero points (same type as their
 * operand): MM_ZP_NONE (0), MM_ZP_SCALAR (one value) or MM_ZP_VECTOR (A: one
 * value per row, [M]; B: one value per column, [N]; shared by every batch).
 * Y is INT32 of the MatMul output shape.  A plan whose tiles cannot fill
 * the GPU over a long K (few rows) splits K: INT32 partials in a workspace
 * the plan allocates at creation (mm_plan_workspace_bytes), summed modulo
 * 2^32 by a second kernel; such a plan's executions must not overlap, as
 * for a MatMul split plan.  Other MatMulInteger plans own no workspace and
 * may run on several streams at once.  Errors as for mm_plan_create, plus
 * MM_ERR_DTYPE for other types and MM_ERR_BAD_OPTION for an unknown
 * zero-point kind or an option other than DIRECT, GENERAL with an INT8 tile,
 * or SPLIT_K on the 128 x 128 INT8 tile (entry 2). */
enum { MM_ZP_NONE = 0, MM_ZP_SCALAR = 1, MM_ZP_VECTOR = 2 };

mm_status mm_int_plan_create(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank, int a_type,
                             int b_type, int a_zp_kind, int b_zp_kind, const mm_plan_options *opt, mm_plan_t *out);

/* Enqueue the MatMulInteger product on `stream`.  a_zero_point /
 * b_zero_point must be non-NULL exactly for the kinds other than
 * MM_ZP_NONE (MM_ERR_NULL_ARG otherwise).  Other rules as for mm_execute;
 * MM_ERR_BAD_OPTION for a plan that is not a MatMulInteger plan (and
 * mm_execute refuses MatMulInteger plans). */
mm_status mm_int_execute(mm_plan_t plan, const void *A, const void *B, const void *a_zero_point,
                         const void *b_zero_point, void *Y, void *stream);

/* Output shape: writes up to MM_MAX_RANK entries to `shape` and the rank to
 * *rank (0 when both inputs are rank one). */
mm_status mm_plan_output_shape(mm_plan_t plan, int64_t *shape, int *rank);

/* Number of output elements (the Y buffer must hold this many), or -1 for a
 * NULL plan. */
int64_t mm_plan_output_numel(mm_plan_t plan);

/* Selected algorithm (an mm_algo value), or -1 for a NULL plan. */
int mm_plan_algo(mm_plan_t plan);

/* Device workspace bytes the plan owns (0 unless SPLIT_K or a split SKINNY_M). */
size_t mm_plan_workspace_bytes(mm_plan_t plan);

/* Fill *info with everything the plan resolved. */
mm_status mm_plan_get_info(mm_plan_t plan, mm_plan_info *info);

/* Tile table of the tiled kernels for `dtype`: number of entries
 * (MM_UINT8, MM_INT8 and MM_INT32 all name the MatMulInteger table). */
int mm_tile_count(int dtype);

/* Entry `index` (0-based) of the tile table: block rows, block columns and
 * K elements per LDS stage.  MM_ERR_BAD_OPTION for an invalid index. */
mm_status mm_tile_config(int dtype, int index, int *block_m, int *block_n, int *block_k);

/* Static description of a status code. */
const char *mm_status_string(mm_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char *mm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MM_H */
