/*
 * oracle.c -- plain CPU reference for ONNX MatMul.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper
 * with the GPU library, and the GPU library never calls it.
 *
 * What it computes (page "MatMul Kernel Design", section "Shape and plan
 * model"; page "Gemm and MatMul Performance Roadmap", sections "Scope and type
 * matrix" and "Phase 4: complete MatMul"):
 *
 *   - a rank-one A of shape [K] is used as [1, K], and the M axis is removed
 *     from the output; a rank-one B of shape [K] is used as [K, 1], and the N
 *     axis is removed from the output;
 *   - the leading (batch) dimensions of the two inputs are broadcast NumPy
 *     style: right-aligned, missing dimensions count as 1, a dimension of 1
 *     stretches to the other input's size, otherwise the sizes must agree;
 *   - for every output batch index the product of the selected A matrix and
 *     the selected B matrix is formed.
 *
 * Arithmetic: every stored element is decoded exactly to double (FP32, FP16
 * and BF16 all embed exactly in binary64); each output is the sum over k in
 * ascending order of a[m,k]*b[k,n] accumulated in double.  Nothing is fused,
 * and no output's summation order changes: the full product walks k in the
 * outer loop over a handful of rows at a time (one double accumulator per
 * output, each still receiving its terms in ascending k), which gives the
 * same bits as the per-element loop that oracle_matmul_at keeps (a test pins
 * the two against each other) while reading each row of B once per group of
 * rows instead of once per output.  Build with -O2 -ffp-contract=off and no
 * fast-math, so every product and every sum is rounded on its own.
 *
 * The narrowing helpers (double -> FP16 / BF16, round to nearest, ties to
 * even, single rounding) exist so the comparator can narrow the exact result
 * to the output type; page "MatMul Kernel Design", section "Types and
 * algorithm selection" fixes FP32 accumulation with final narrowing for the
 * 16-bit types.  The rounding mode itself is a reading (nearest-even), since
 * the pages do not name it.
 *
 * MatMulInteger (exact integer sums reduced modulo 2^32) sits at the end of
 * the file.
 *
 * Parity pins: see tests/test_oracle.py (shape rules against numpy.matmul,
 * closed forms, identity and permutation products, small-integer exactness,
 * broadcast equals explicit repetition, narrowing against numpy float16 and a
 * hand-derived BF16 table).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* Type codes follow ONNX TensorProto: FLOAT=1, FLOAT16=10, DOUBLE=11, BFLOAT16=16. */
#define OR_FLOAT 1
#define OR_FLOAT16 10
#define OR_DOUBLE 11
#define OR_BFLOAT16 16

/* Status codes of this file (independent of the GPU library's). */
#define OR_OK 0
#define OR_ERR_RANK 1      /* an input has rank 0 */
#define OR_ERR_NEGATIVE 2  /* a dimension is negative */
#define OR_ERR_K 3         /* inner dimensions differ */
#define OR_ERR_BROADCAST 4 /* batch dimensions cannot be broadcast */
#define OR_ERR_DTYPE 5     /* unknown type code */
#define OR_ERR_ALLOC 6     /* host allocation failed */

/* ------------------------------------------------------------------------ */
/* Bit-level decoding of the stored element types.                          */
/* ------------------------------------------------------------------------ */

/* Decode an IEEE-style binary format with `ebits` exponent bits and `mbits`
 * fraction bits.  Exact for FP16 (5, 10) and BF16 (8, 7). */
static double decode_ieee(uint32_t bits, int ebits, int mbits)
{
    uint32_t sign = (bits >> (ebits + mbits)) & 1u;
    uint32_t expo = (bits >> mbits) & ((1u << ebits) - 1u);
    uint32_t frac = bits & ((1u << mbits) - 1u);
    int bias = (1 << (ebits - 1)) - 1;
    double v;
    if (expo == (1u << ebits) - 1u) {
        v = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        /* zero or subnormal: frac * 2^(1 - bias - mbits) */
        v = ldexp((double)frac, 1 - bias - mbits);
    } else {
        v = ldexp((double)((1u << mbits) | frac), (int)expo - bias - mbits);
    }
    return sign ? -v : v;
}

double oracle_decode_f16(uint16_t bits) { return decode_ieee(bits, 5, 10); }
double oracle_decode_bf16(uint16_t bits) { return decode_ieee(bits, 8, 7); }

static double *g_table_f16 = 0;
static double *g_table_bf16 = 0;

/* Full decode tables for the 16-bit types, built from decode_ieee. */
static int build_tables(void)
{
    if (g_table_f16 && g_table_bf16) return OR_OK;
    double *t16 = (double *)malloc(65536 * sizeof(double));
    double *tb16 = (double *)malloc(65536 * sizeof(double));
    if (!t16 || !tb16) {
        free(t16);
        free(tb16);
        return OR_ERR_ALLOC;
    }
    for (uint32_t i = 0; i < 65536u; ++i) {
        t16[i] = decode_ieee(i, 5, 10);
        tb16[i] = decode_ieee(i, 8, 7);
    }
    g_table_f16 = t16;
    g_table_bf16 = tb16;
    return OR_OK;
}

/* Element `idx` of a tensor stored with type `dtype`, as an exact double. */
static double load_elem(const void *base, int dtype, int64_t idx)
{
    switch (dtype) {
    case OR_FLOAT: {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    case OR_DOUBLE: {
        double d;
        memcpy(&d, (const char *)base + idx * 8, 8);
        return d;
    }
    case OR_FLOAT16:
        return g_table_f16[((const uint16_t *)base)[idx]];
    case OR_BFLOAT16:
        return g_table_bf16[((const uint16_t *)base)[idx]];
    }
    return NAN;
}

static int dtype_ok(int dtype)
{
    return dtype == OR_FLOAT || dtype == OR_FLOAT16 || dtype == OR_DOUBLE || dtype == OR_BFLOAT16;
}

/* ------------------------------------------------------------------------ */
/* Narrowing: double -> 16-bit format, round to nearest, ties to even.      */
/* ------------------------------------------------------------------------ */

static uint32_t narrow_ieee(double x, int ebits, int mbits)
{
    uint32_t sign = signbit(x) ? 1u : 0u;
    uint32_t sign_field = sign << (ebits + mbits);
    uint32_t exp_all = (1u << ebits) - 1u;
    int bias = (1 << (ebits - 1)) - 1;
    int emin = 1 - bias; /* exponent of the smallest normal */
    int emax = bias;     /* exponent of the largest finite */
    if (isnan(x)) /* quiet NaN, sign kept */
        return sign_field | (exp_all << mbits) | (1u << (mbits - 1));
    double a = fabs(x);
    if (a == 0.0) return sign_field;
    if (isinf(a)) return sign_field | (exp_all << mbits);

    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1): unbiased exponent e2 - 1 */
    int e = e2 - 1;
    if (e < emin) e = emin; /* subnormal range: fixed quantum */
    /* Scale so that one unit in the last place of the target is 1.0. */
    double scaled = ldexp(a, mbits - e);
    double fl = floor(scaled);
    double rem = scaled - fl;
    double r = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    uint32_t mant = (uint32_t)r; /* in [0, 2^(mbits+1)] */
    if (mant == (1u << (mbits + 1))) { /* rounding carried into the next binade */
        mant = 1u << mbits;
        e += 1;
    }
    if (e > emax) return sign_field | (exp_all << mbits); /* overflow to infinity */
    uint32_t biased = (mant >= (1u << mbits)) ? (uint32_t)(e + bias) : 0u;
    return sign_field | (biased << mbits) | (mant & ((1u << mbits) - 1u));
}

uint16_t oracle_narrow_f16(double x) { return (uint16_t)narrow_ieee(x, 5, 10); }
uint16_t oracle_narrow_bf16(double x) { return (uint16_t)narrow_ieee(x, 8, 7); }

/* Narrow `n` doubles to `dtype`'s storage (FLOAT: C cast; FLOAT16/BFLOAT16:
 * the nearest-even helpers above; DOUBLE: copy). */
int oracle_narrow_array(int dtype, const double *in, int64_t n, void *out)
{
    if (!dtype_ok(dtype)) return OR_ERR_DTYPE;
    for (int64_t i = 0; i < n; ++i) {
        switch (dtype) {
        case OR_FLOAT: ((float *)out)[i] = (float)in[i]; break;
        case OR_DOUBLE: ((double *)out)[i] = in[i]; break;
        case OR_FLOAT16: ((uint16_t *)out)[i] = oracle_narrow_f16(in[i]); break;
        case OR_BFLOAT16: ((uint16_t *)out)[i] = oracle_narrow_bf16(in[i]); break;
        }
    }
    return OR_OK;
}

int oracle_decode_array(int dtype, const void *in, int64_t n, double *out)
{
    if (!dtype_ok(dtype)) return OR_ERR_DTYPE;
    if (build_tables() != OR_OK) return OR_ERR_ALLOC;
    for (int64_t i = 0; i < n; ++i) out[i] = load_elem(in, dtype, i);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Shapes.                                                                    */
/* ------------------------------------------------------------------------ */

/* Everything the element loop needs, derived from the two input shapes. */
typedef struct {
    int64_t M, N, K;
    int brank;          /* number of broadcast batch dimensions */
    int64_t *bshape;    /* broadcast batch shape (brank entries) */
    int64_t *ashape_b;  /* A's batch dims right-aligned and padded with 1 */
    int64_t *bshape_b;  /* B's batch dims right-aligned and padded with 1 */
    int64_t nbatch;     /* product of bshape */
    int a_vec, b_vec;   /* input was rank one */
} shapes_t;

static void shapes_free(shapes_t *s)
{
    free(s->bshape);
    free(s->ashape_b);
    free(s->bshape_b);
    memset(s, 0, sizeof(*s));
}

static int resolve(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank, shapes_t *s)
{
    memset(s, 0, sizeof(*s));
    if (a_rank < 1 || b_rank < 1) return OR_ERR_RANK;
    for (int i = 0; i < a_rank; ++i)
        if (a_shape[i] < 0) return OR_ERR_NEGATIVE;
    for (int i = 0; i < b_rank; ++i)
        if (b_shape[i] < 0) return OR_ERR_NEGATIVE;

    s->a_vec = (a_rank == 1);
    s->b_vec = (b_rank == 1);
    /* Promotion: [K] -> [1, K] for A, [K] -> [K, 1] for B. */
    int64_t Ka, Kb;
    int a_batch_rank, b_batch_rank;
    if (s->a_vec) {
        s->M = 1;
        Ka = a_shape[0];
        a_batch_rank = 0;
    } else {
        s->M = a_shape[a_rank - 2];
        Ka = a_shape[a_rank - 1];
        a_batch_rank = a_rank - 2;
    }
    if (s->b_vec) {
        s->N = 1;
        Kb = b_shape[0];
        b_batch_rank = 0;
    } else {
        s->N = b_shape[b_rank - 1];
        Kb = b_shape[b_rank - 2];
        b_batch_rank = b_rank - 2;
    }
    if (Ka != Kb) return OR_ERR_K;
    s->K = Ka;

    int r = a_batch_rank > b_batch_rank ? a_batch_rank : b_batch_rank;
    s->brank = r;
    s->bshape = (int64_t *)malloc((size_t)(r + 1) * sizeof(int64_t));
    s->ashape_b = (int64_t *)malloc((size_t)(r + 1) * sizeof(int64_t));
    s->bshape_b = (int64_t *)malloc((size_t)(r + 1) * sizeof(int64_t));
    if (!s->bshape || !s->ashape_b || !s->bshape_b) {
        shapes_free(s);
        return OR_ERR_ALLOC;
    }
    s->nbatch = 1;
    for (int d = 0; d < r; ++d) {
        /* position d of the right-aligned batch shape */
        int ai = d - (r - a_batch_rank);
        int bi = d - (r - b_batch_rank);
        int64_t da = ai >= 0 ? a_shape[ai] : 1;
        int64_t db = bi >= 0 ? b_shape[bi] : 1;
        int64_t out;
        if (da == db) out = da;
        else if (da == 1) out = db;
        else if (db == 1) out = da;
        else {
            shapes_free(s);
            return OR_ERR_BROADCAST;
        }
        s->ashape_b[d] = da;
        s->bshape_b[d] = db;
        s->bshape[d] = out;
        s->nbatch *= out;
    }
    return OR_OK;
}

/* Output shape of MatMul(A, B).  `out_shape` must hold max(a_rank, b_rank)
 * entries; `*out_rank` may be 0 (both inputs rank one: a single element). */
int oracle_output_shape(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank,
                        int64_t *out_shape, int *out_rank)
{
    shapes_t s;
    int st = resolve(a_shape, a_rank, b_shape, b_rank, &s);
    if (st != OR_OK) return st;
    int r = 0;
    for (int d = 0; d < s.brank; ++d) out_shape[r++] = s.bshape[d];
    if (!s.a_vec) out_shape[r++] = s.M;
    if (!s.b_vec) out_shape[r++] = s.N;
    *out_rank = r;
    shapes_free(&s);
    return OR_OK;
}

/* Offsets (in elements) of the A and B matrices that output batch `bi` uses.
 * bi is unravelled row-major over the broadcast batch shape; an input whose
 * dimension is 1 takes index 0 along it. */
static void batch_offsets(const shapes_t *s, int64_t bi, int64_t *offa, int64_t *offb)
{
    int64_t ia = 0, ib = 0;       /* linear batch index inside each input */
    int64_t mula = 1, mulb = 1;   /* row-major multipliers, innermost first */
    int64_t rest = bi;
    for (int d = s->brank - 1; d >= 0; --d) {
        int64_t i = rest % s->bshape[d];
        rest /= s->bshape[d];
        int64_t ja = (s->ashape_b[d] == 1) ? 0 : i;
        int64_t jb = (s->bshape_b[d] == 1) ? 0 : i;
        ia += ja * mula;
        ib += jb * mulb;
        mula *= s->ashape_b[d];
        mulb *= s->bshape_b[d];
    }
    *offa = ia * s->M * s->K;
    *offb = ib * s->K * s->N;
}

/* One output element: sum over k ascending of a[m,k]*b[k,n], in double. */
static double dot_one(const shapes_t *s, int dtype, const void *A, const void *B, int64_t offa,
                      int64_t offb, int64_t m, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < s->K; ++k) {
        double a = load_elem(A, dtype, offa + m * s->K + k);
        double b = load_elem(B, dtype, offb + k * s->N + n);
        acc += a * b;
    }
    return acc;
}

/* Rows of one batch matrix that the full product carries at once. */
#define OR_ROW_GROUP 16

/* Full MatMul.  Y receives nbatch*M*N doubles in row-major order of the
 * output shape (squeezed axes have size 1, so the order is the same).
 * Work items are (batch, group of up to OR_ROW_GROUP rows); for each k in
 * ascending order, row k of B is decoded once and a[m,k]*b[k,n] is added to
 * the double accumulator of every output (m, n) of the group -- the same
 * operations, in the same order per output, as dot_one. */
int oracle_matmul(int dtype, const void *A, const int64_t *a_shape, int a_rank, const void *B,
                  const int64_t *b_shape, int b_rank, double *Y)
{
    if (!dtype_ok(dtype)) return OR_ERR_DTYPE;
    if (build_tables() != OR_OK) return OR_ERR_ALLOC;
    shapes_t s;
    int st = resolve(a_shape, a_rank, b_shape, b_rank, &s);
    if (st != OR_OK) return st;
    const int64_t groups = (s.M + OR_ROW_GROUP - 1) / OR_ROW_GROUP;
    const int64_t items = s.nbatch * groups;
    int failed = 0;
#pragma omp parallel
    {
        double *brow = (double *)malloc((size_t)(s.N > 0 ? s.N : 1) * sizeof(double));
        double *acc = (double *)malloc((size_t)(s.N > 0 ? s.N : 1) * OR_ROW_GROUP * sizeof(double));
        if (!brow || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            if (!brow || !acc) continue;
            const int64_t bi = it / groups, m0 = (it % groups) * OR_ROW_GROUP;
            const int64_t rows = (s.M - m0) < OR_ROW_GROUP ? (s.M - m0) : OR_ROW_GROUP;
            int64_t offa, offb;
            batch_offsets(&s, bi, &offa, &offb);
            for (int64_t i = 0; i < rows * s.N; ++i) acc[i] = 0.0;
            for (int64_t k = 0; k < s.K; ++k) {
                for (int64_t n = 0; n < s.N; ++n) brow[n] = load_elem(B, dtype, offb + k * s.N + n);
                for (int64_t r = 0; r < rows; ++r) {
                    const double a = load_elem(A, dtype, offa + (m0 + r) * s.K + k);
                    double *ar = acc + r * s.N;
                    for (int64_t n = 0; n < s.N; ++n) ar[n] += a * brow[n];
                }
            }
            memcpy(Y + (bi * s.M + m0) * s.N, acc, (size_t)(rows * s.N) * sizeof(double));
        }
        free(brow);
        free(acc);
    }
    shapes_free(&s);
    return failed ? OR_ERR_ALLOC : OR_OK;
}

/* Selected output elements, by flat row-major index into the output.  For
 * checks at sizes where the full product is too slow on a CPU. */
int oracle_matmul_at(int dtype, const void *A, const int64_t *a_shape, int a_rank, const void *B,
                     const int64_t *b_shape, int b_rank, const int64_t *flat_idx, int64_t count,
                     double *out)
{
    if (!dtype_ok(dtype)) return OR_ERR_DTYPE;
    if (build_tables() != OR_OK) return OR_ERR_ALLOC;
    shapes_t s;
    int st = resolve(a_shape, a_rank, b_shape, b_rank, &s);
    if (st != OR_OK) return st;
    if (count > 0 && s.nbatch * s.M * s.N == 0) { /* no element to select */
        shapes_free(&s);
        return OR_ERR_BROADCAST;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = flat_idx[i];
        int64_t n = f % s.N;
        int64_t m = (f / s.N) % s.M;
        int64_t bi = f / (s.N * s.M);
        int64_t offa, offb;
        batch_offsets(&s, bi, &offa, &offb);
        out[i] = dot_one(&s, dtype, A, B, offa, offb, m, n);
    }
    shapes_free(&s);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Gemm (page "Gemm and MatMul Performance Roadmap", section "Scope and type */
/* matrix": rank-2 inputs, alpha, beta, optional broadcast bias, transA and  */
/* transB):                                                                  */
/*   Y[m][n] = alpha * sum_k A'[m][k] * B'[k][n] + beta * C(m, n)            */
/* with A' = A, or A transposed (A stored [K][M]); B' = B, or B transposed    */
/* (B stored [N][K]); C broadcast unidirectionally to [M][N] NumPy style:     */
/* right-aligned, a dimension of 1 stretches, otherwise it must equal the    */
/* output's.  Without C the bias term is absent (beta unused).  The sum runs */
/* over ascending k in double, then alpha * sum + beta * c is formed in      */
/* double.                                                                   */
/* ------------------------------------------------------------------------ */

#define OR_ERR_SHAPE 7 /* Gemm operand ranks / sizes do not fit */

static int gemm_impl(int dtype, const void *A, int64_t a_rows, int64_t a_cols, int trans_a, const void *B,
                     int64_t b_rows, int64_t b_cols, int trans_b, const void *C, const int64_t *c_shape, int c_rank,
                     double alpha, double beta, const int64_t *flat_idx, int64_t n_idx, double *Y)
{
    if (!dtype_ok(dtype)) return OR_ERR_DTYPE;
    if (build_tables() != OR_OK) return OR_ERR_ALLOC;
    if (a_rows < 0 || a_cols < 0 || b_rows < 0 || b_cols < 0) return OR_ERR_NEGATIVE;
    int64_t M = trans_a ? a_cols : a_rows;
    int64_t K = trans_a ? a_rows : a_cols;
    int64_t Kb = trans_b ? b_cols : b_rows;
    int64_t N = trans_b ? b_rows : b_cols;
    if (K != Kb) return OR_ERR_K;
    /* C's dimensions, right-aligned against (M, N) and padded with 1. */
    int64_t cr = 1, cc = 1;
    if (C) {
        if (c_rank < 0 || c_rank > 2) return OR_ERR_SHAPE;
        if (c_rank == 1) cc = c_shape[0];
        if (c_rank == 2) {
            cr = c_shape[0];
            cc = c_shape[1];
        }
        if (cr < 0 || cc < 0) return OR_ERR_NEGATIVE;
        if ((cr != 1 && cr != M) || (cc != 1 && cc != N)) return OR_ERR_BROADCAST;
    }
    const int64_t count = flat_idx ? n_idx : M * N;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t f = flat_idx ? flat_idx[i] : i;
        const int64_t m = f / N, n = f % N;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = load_elem(A, dtype, trans_a ? k * M + m : m * K + k);
            double b = load_elem(B, dtype, trans_b ? n * K + k : k * N + n);
            acc += a * b;
        }
        double y = alpha * acc;
        if (C) {
            int64_t ci = (cr == 1 ? 0 : m) * cc + (cc == 1 ? 0 : n);
            y += beta * load_elem(C, dtype, ci);
        }
        Y[i] = y;
    }
    return OR_OK;
}

int oracle_gemm(int dtype, const void *A, int64_t a_rows, int64_t a_cols, int trans_a, const void *B,
                int64_t b_rows, int64_t b_cols, int trans_b, const void *C, const int64_t *c_shape, int c_rank,
                double alpha, double beta, double *Y)
{
    return gemm_impl(dtype, A, a_rows, a_cols, trans_a, B, b_rows, b_cols, trans_b, C, c_shape, c_rank, alpha,
                     beta, 0, 0, Y);
}

/* Selected outputs, by flat row-major index into [M, N]. */
int oracle_gemm_at(int dtype, const void *A, int64_t a_rows, int64_t a_cols, int trans_a, const void *B,
                   int64_t b_rows, int64_t b_cols, int trans_b, const void *C, const int64_t *c_shape, int c_rank,
                   double alpha, double beta, const int64_t *flat_idx, int64_t count, double *out)
{
    return gemm_impl(dtype, A, a_rows, a_cols, trans_a, B, b_rows, b_cols, trans_b, C, c_shape, c_rank, alpha,
                     beta, flat_idx, count, out);
}

/* ------------------------------------------------------------------------ */
/* MatMulInteger (page "Gemm and MatMul Performance Roadmap", section        */
/* "Remaining pull-request sequence", Roadmap PR09.1: INT8 or UINT8 A and B, */
/* optional zero points -- one value, or one per row of A / per column of   */
/* B --, the MatMul broadcasting and rank-one rules, INT32 accumulation     */
/* modulo 2^32):                                                             */
/*   Y[i][m][n] = sum_k (A[iA(i)][m][k] - za(m)) * (B[iB(i)][k][n] - zb(n))  */
/* Each product is formed exactly in int64 and summed exactly in int64      */
/* (|term| <= 255^2, so no overflow below K = 2^47); the sum is then reduced */
/* modulo 2^32 to the INT32 two's-complement value.  Reading: a vector zero  */
/* point has M (A) or N (B) entries and is shared by every batch.           */
/* ------------------------------------------------------------------------ */

#define OR_ZP_NONE 0
#define OR_ZP_SCALAR 1
#define OR_ZP_VECTOR 2

static int64_t load_byte(const void *base, int is_signed, int64_t idx)
{
    return is_signed ? (int64_t)((const int8_t *)base)[idx] : (int64_t)((const uint8_t *)base)[idx];
}

static int64_t zero_point(const void *zp, int kind, int is_signed, int64_t i)
{
    if (kind == OR_ZP_NONE) return 0;
    return load_byte(zp, is_signed, kind == OR_ZP_SCALAR ? 0 : i);
}

/* Exact sum reduced modulo 2^32, as the INT32 two's-complement value. */
static int32_t wrap32(int64_t v)
{
    uint32_t u = (uint32_t)((uint64_t)v & 0xffffffffu);
    return u >= 0x80000000u ? (int32_t)((int64_t)u - 4294967296LL) : (int32_t)u;
}

static int integer_impl(const void *A, const int64_t *a_shape, int a_rank, int a_signed, const void *B,
                        const int64_t *b_shape, int b_rank, int b_signed, const void *za, int za_kind,
                        const void *zb, int zb_kind, const int64_t *flat_idx, int64_t n_idx, int32_t *Y)
{
    if (za_kind < OR_ZP_NONE || za_kind > OR_ZP_VECTOR || zb_kind < OR_ZP_NONE || zb_kind > OR_ZP_VECTOR)
        return OR_ERR_SHAPE;
    if ((za_kind != OR_ZP_NONE && !za) || (zb_kind != OR_ZP_NONE && !zb)) return OR_ERR_SHAPE;
    shapes_t s;
    int st = resolve(a_shape, a_rank, b_shape, b_rank, &s);
    if (st != OR_OK) return st;
    const int64_t total = s.nbatch * s.M * s.N;
    const int64_t count = flat_idx ? n_idx : total;
    if (flat_idx && count > 0 && total == 0) {
        shapes_free(&s);
        return OR_ERR_BROADCAST;
    }
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        const int64_t f = flat_idx ? flat_idx[i] : i;
        const int64_t n = f % s.N;
        const int64_t m = (f / s.N) % s.M;
        const int64_t bi = f / (s.N * s.M);
        int64_t offa, offb;
        batch_offsets(&s, bi, &offa, &offb);
        const int64_t a0 = zero_point(za, za_kind, a_signed, m);
        const int64_t b0 = zero_point(zb, zb_kind, b_signed, n);
        int64_t acc = 0;
        for (int64_t k = 0; k < s.K; ++k)
            acc += (load_byte(A, a_signed, offa + m * s.K + k) - a0) * (load_byte(B, b_signed, offb + k * s.N + n) - b0);
        Y[i] = wrap32(acc);
    }
    shapes_free(&s);
    return OR_OK;
}

/* Full MatMulInteger: Y receives nbatch*M*N INT32 values in row-major order. */
int oracle_matmul_integer(const void *A, const int64_t *a_shape, int a_rank, int a_signed, const void *B,
                          const int64_t *b_shape, int b_rank, int b_signed, const void *za, int za_kind,
                          const void *zb, int zb_kind, int32_t *Y)
{
    return integer_impl(A, a_shape, a_rank, a_signed, B, b_shape, b_rank, b_signed, za, za_kind, zb, zb_kind, 0, 0,
                        Y);
}

/* Selected MatMulInteger outputs, by flat row-major index into the output. */
int oracle_matmul_integer_at(const void *A, const int64_t *a_shape, int a_rank, int a_signed, const void *B,
                             const int64_t *b_shape, int b_rank, int b_signed, const void *za, int za_kind,
                             const void *zb, int zb_kind, const int64_t *flat_idx, int64_t count, int32_t *out)
{
    return integer_impl(A, a_shape, a_rank, a_signed, B, b_shape, b_rank, b_signed, za, za_kind, zb, zb_kind,
                        flat_idx, count, out);
}

/* Number of OpenMP threads the loops above use (for reporting). */
int oracle_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
