// execute.cpp -- mm_execute / mm_plan_destroy: turn a plan into kernel
// launches on the caller's stream.
#include <string.h>

#include "internal.h"
#include "plan.h"

using namespace mm;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static mm_status hip_fail(hipError_t e, const char *what) {
    return fail(MM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

namespace mm {

// Split-K workspace: allocated once, on the current device, by plan creation
// (at_create) or -- when creation found no GPU -- by the first execution.
mm_status alloc_workspace(mm_plan_s *p, bool at_create) {
    if (p->workspace_bytes <= 0) return MM_OK;
    if (at_create) {
        int count = 0;
        if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
            (void)hipGetLastError();  // no GPU here: leave no error behind for later launches
            return MM_OK;
        }
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(e, "hipGetDevice");
    }
    std::lock_guard<std::mutex> lock(p->ws_mutex);
    if (p->ws) {
        if (p->ws_device != dev)
            return fail(MM_ERR_HIP, "plan workspace lives on device %d; executing on device %d needs its own plan",
                        p->ws_device, dev);
        return MM_OK;
    }
    void *ptr = nullptr;
    e = hipMalloc(&ptr, (size_t)p->workspace_bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MM_ERR_ALLOC, "hipMalloc of %lld workspace bytes: %s", (long long)p->workspace_bytes,
                    hipGetErrorString(e));
    }
    p->ws = ptr;
    p->ws_device = dev;
    return MM_OK;
}

}  // namespace mm

static mm_status ensure_workspace(mm_plan_s *p) { return alloc_workspace(p, false); }

// Launches of a MatMul or Gemm plan (C: the Gemm bias, NULL if none).  The
// split partial sums go to `ws` when it is not NULL (at least the plan's
// workspace_bytes, on the current device), else to the plan's workspace.
mm_status mm::execute_plan(mm_plan_s *p, const void *A, const void *B, const void *C, void *Y, void *stream,
                           void *ws, bool packed_b) {
    if (p->algo == MM_ALGO_EMPTY) return MM_OK;
    if (!Y) return fail(MM_ERR_NULL_ARG, "Y is NULL for a non-empty output");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (p->algo == MM_ALGO_ZERO_FILL) {
        e = launch_fill_zero(p->dtype, Y, p->out_numel, s);
        return e == hipSuccess ? MM_OK : hip_fail(e, "zero-fill launch");
    }
    if (p->K > 0 && (!A || !B)) return fail(MM_ERR_NULL_ARG, "A or B is NULL");
    if (p->is_gemm && p->c_mode != kBiasNone && !C) return fail(MM_ERR_NULL_ARG, "the plan has a C but C is NULL");

    KArgs a;
    memset(&a, 0, sizeof(a));
    a.A = A;
    a.B = B;
    a.Y = Y;
    a.W = nullptr;
    a.M = p->kernel_m;
    a.N = p->N;
    a.K = p->K;
    a.lda = p->ta ? p->M : p->K;
    a.ldb = p->tb ? p->K : p->N;
    a.ldy = p->N;
    if (p->is_gemm) {
        a.ta = p->ta;
        a.tb = p->tb;
        a.gemm_epi = 1;
        a.c_mode = p->c_mode;
        a.alpha = p->alpha;
        a.beta = p->beta;
        a.C = C;
        a.ldc = p->ldc;
    }
    a.batch = p->batch;
    a.kchunk = p->kchunk;
    a.split = p->split;
    a.bd = p->bd;

    const int64_t es = elem_size(p->dtype);
    Align al;
    al.a = aligned16(A) && (a.lda * es) % 16 == 0;
    al.b = aligned16(B) && (a.ldb * es) % 16 == 0;
    al.y = aligned16(Y) && (p->N * es) % 16 == 0;
    // Split-K partials are FP32 rows (double for DOUBLE) in a workspace of
    // our own (aligned); only the 16- and 32-bit kernels read y_vec.
    a.y_vec = p->algo == MM_ALGO_SPLIT_K ? (p->N * 4) % 16 == 0 : al.y;

    const bool f64 = p->dtype == MM_DOUBLE;
    switch (p->algo) {
    case MM_ALGO_DIRECT:
        e = f64 ? launch_direct_f64(a, s) : launch_direct(p->dtype, a, s);
        break;
    case MM_ALGO_SKINNY_M:
        if (p->split > 1) {
            // K cut into chunks: FP32 partials, then the split-K reduction.
            if (!ws) {
                mm_status st = ensure_workspace(p);
                if (st != MM_OK) return st;
            }
            a.W = (float *)(ws ? ws : p->ws);
            e = launch_skinny_m(p->dtype, al, a, s);
            if (e == hipSuccess) e = launch_splitk_reduce(p->dtype, a, s);
        } else {
            e = launch_skinny_m(p->dtype, al, a, s);
        }
        break;
    case MM_ALGO_SKINNY_N:
        e = launch_skinny_n(p->dtype, al, a, s);
        break;
    case MM_ALGO_GENERAL:
        if (f64) {
            e = launch_general_f64(p->tile, al, false, a, s);
        } else if (p->tail_col > 0) {
            // Columns [0, tail_col) in whole rounds of `tile`, then the rest
            // with `tail_tile`; both read B and write Y (and a Gemm's C) with
            // their full pitches.  Column c of B' is column c of B, or row c
            // of a transposed B; a per-column or full C moves by c columns.
            // A prepacked constant B holds each launch's columns separately.
            const int64_t nmat = packed_b ? p->b_numel / (p->K * p->N) : 0;
            KArgs m = a;
            m.N = p->tail_col;
            if (packed_b) {
                m.Bp = p->cbp;
                m.bp_mat_bytes = p->cbp_main;
                m.bp_mat_elems = p->K * p->N;
                m.b_packed = 1;
            }
            e = launch_general(p->dtype, p->tile, al, false, m, s);
            if (e == hipSuccess) {
                KArgs r = a;
                if (packed_b) {
                    r.Bp = (const char *)p->cbp + nmat * p->cbp_main;
                    r.bp_mat_bytes = p->cbp_tail;
                    r.bp_mat_elems = p->K * p->N;
                    r.b_packed = 1;
                }
                r.N = p->N - p->tail_col;
                r.B = (const char *)B + p->tail_col * (p->tb ? a.ldb : 1) * es;
                r.Y = (char *)Y + p->tail_col * es;
                if (p->is_gemm && (p->c_mode == kBiasRow || p->c_mode == kBiasFull))
                    r.C = (const char *)C + p->tail_col * es;
                Align ar = al;
                ar.b = al.b && aligned16(r.B);
                r.y_vec = al.y && aligned16(r.Y) && (r.N * es) % 16 == 0;
                e = launch_general(p->dtype, p->tail_tile, ar, false, r, s);
            }
        } else {
            KArgs m = a;
            if (packed_b) {
                m.Bp = p->cbp;
                m.bp_mat_bytes = p->cbp_main;
                m.bp_mat_elems = p->K * p->N;
                m.b_packed = 1;
            }
            e = launch_general(p->dtype, p->tile, al, false, m, s);
        }
        break;
    case MM_ALGO_SPLIT_K: {
        if (!ws) {
            mm_status st = ensure_workspace(p);
            if (st != MM_OK) return st;
        }
        a.W = (float *)(ws ? ws : p->ws);
        if (f64) {
            e = launch_general_f64(p->tile, al, true, a, s);
            if (e == hipSuccess) e = launch_splitk_reduce_f64(a, s);
        } else {
            e = launch_general(p->dtype, p->tile, al, true, a, s);
            if (e == hipSuccess) e = launch_splitk_reduce(p->dtype, a, s);
        }
        break;
    }
    default:
        return fail(MM_ERR_BAD_OPTION, "plan has no executable algorithm (%d)", p->algo);
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return MM_OK;
}

// Page "Gemm and MatMul Performance Roadmap", section "Target computation
// algorithm" (a constant B prepacked once, when its shape and layout are
// stable) and section "Remaining pull-request sequence", PR06.4 (its panels
// no longer re-derived on every run): a 16-bit plan on the tiled kernel also
// keeps its constant B as the LDS image of every stage's B panel, so each
// stage's B is one contiguous block and its loads need no per-lane address
// or range arithmetic.  The row-major copy stays for the kernels that read
// B as stored (unaligned A, other algorithms).
static mm_status pack_constant_b(mm_plan_s *p, hipStream_t s) {
    if (p->algo != MM_ALGO_GENERAL || (p->dtype != MM_FLOAT16 && p->dtype != MM_BFLOAT16)) return MM_OK;
    if (p->K <= 0 || p->N <= 0 || p->N % 8 != 0 || p->tile < 0 || (p->tail_col > 0 && p->tail_tile < 0)) return MM_OK;
    const TileCfg *t = tile_entry(p->dtype, p->tile);
    const TileCfg *tt = p->tail_col > 0 ? tile_entry(p->dtype, p->tail_tile) : nullptr;
    if (t->bkb != 128 || (tt && tt->bkb != 128)) return MM_OK;
    const int64_t nmat = p->b_numel / (p->K * p->N);
    const int64_t nmain = p->tail_col > 0 ? p->tail_col : p->N;
    const int64_t main_b = packed_b_bytes(nmain, p->K, t->bn);
    const int64_t tail_b = tt ? packed_b_bytes(p->N - p->tail_col, p->K, tt->bn) : 0;
    const size_t bytes = (size_t)(nmat * (main_b + tail_b));
    if (p->cbp && p->cbp_bytes != bytes) {
        (void)hipFree(p->cbp);
        p->cbp = nullptr;
    }
    if (!p->cbp) {
        hipError_t e = hipMalloc(&p->cbp, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            p->cbp = nullptr;
            return fail(MM_ERR_ALLOC, "hipMalloc of %zu prepacked constant-B bytes: %s", bytes, hipGetErrorString(e));
        }
        p->cbp_bytes = bytes;
    }
    hipError_t e = launch_pack_b(t->bn, p->cb, nmat, p->K * p->N, p->K, p->N, 0, nmain, p->cbp, s);
    if (e == hipSuccess && tt)
        e = launch_pack_b(tt->bn, p->cb, nmat, p->K * p->N, p->K, p->N, p->tail_col, p->N - p->tail_col,
                          (char *)p->cbp + nmat * main_b, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "constant-B prepack");
    p->cbp_main = main_b;
    p->cbp_tail = tail_b;
    p->cbp_ok = true;
    return MM_OK;
}

extern "C" {

mm_status mm_execute(mm_plan_t p, const void *A, const void *B, void *Y, void *stream) {
    clear_error();
    if (!p) return fail(MM_ERR_NULL_ARG, "plan is NULL");
    if (p->is_gemm) return fail(MM_ERR_BAD_OPTION, "a Gemm plan runs through mm_gemm_execute");
    if (p->is_int) return fail(MM_ERR_BAD_OPTION, "a MatMulInteger plan runs through mm_int_execute");
    return execute_plan(p, A, B, nullptr, Y, stream, nullptr);
}

mm_status mm_int_execute(mm_plan_t p, const void *A, const void *B, const void *za, const void *zb, void *Y,
                         void *stream) {
    clear_error();
    if (!p) return fail(MM_ERR_NULL_ARG, "plan is NULL");
    if (!p->is_int) return fail(MM_ERR_BAD_OPTION, "not a MatMulInteger plan");
    if (p->algo == MM_ALGO_EMPTY) return MM_OK;
    if (!Y) return fail(MM_ERR_NULL_ARG, "Y is NULL for a non-empty output");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (p->algo == MM_ALGO_ZERO_FILL) {
        e = launch_fill_zero(MM_INT32, Y, p->out_numel, s);
        return e == hipSuccess ? MM_OK : hip_fail(e, "zero-fill launch");
    }
    if (!A || !B) return fail(MM_ERR_NULL_ARG, "A or B is NULL");
    if ((p->zpa_kind != MM_ZP_NONE && !za) || (p->zpb_kind != MM_ZP_NONE && !zb))
        return fail(MM_ERR_NULL_ARG, "a zero point the plan expects is NULL");
    KArgs a;
    memset(&a, 0, sizeof(a));
    a.A = A;
    a.B = B;
    a.Y = Y;
    a.M = p->kernel_m;
    a.N = p->N;
    a.K = p->K;
    a.lda = p->K;
    a.ldb = p->N;
    a.ldy = p->N;
    a.batch = p->batch;
    a.kchunk = p->K;
    a.split = 1;
    a.bd = p->bd;
    a.a_signed = p->a_type == MM_INT8;
    a.b_signed = p->b_type == MM_INT8;
    a.flip_a = a.a_signed ? 0u : 0x80808080u;
    a.flip_b = a.b_signed ? 0u : 0x80808080u;
    a.zpa_mode = p->zpa_kind;
    a.zpb_mode = p->zpb_kind;
    a.zpa = za;
    a.zpb = zb;
    a.zp_rows = p->M > 0 ? p->M : 1;
    a.y_vec = aligned16(Y) && (p->N * 4) % 16 == 0;
    bool tiled = p->algo == MM_ALGO_GENERAL || p->algo == MM_ALGO_SPLIT_K;
    if (tiled) {
        // The tiled kernel streams 16-byte chunks of A rows and B rows, with
        // 32-bit offsets within one tile of A rows and one stage of B rows.
        const TileCfg *t = tile_entry(MM_INT8, p->tile);
        tiled = aligned16(A) && aligned16(B) && p->K % 16 == 0 && p->N % 16 == 0 &&
                (int64_t)t->bm * p->K < 0x7fff0000LL && (int64_t)t->bkb * p->N < 0x7fff0000LL;
    }
    if (!tiled) {
        e = launch_int_direct(a, s);
        return e == hipSuccess ? MM_OK : hip_fail(e, "kernel launch");
    }
    a.sum_a = p->need_ra;
    a.sum_b = p->need_cb;
    if (p->tail_col > 0) {
        // Columns [0, tail_col) in whole rounds of `tile`, then the rest with
        // `tail_tile` (B, Y and a per-column B zero point moved by tail_col
        // columns; tail_col is a multiple of 256, so alignment holds).
        KArgs m = a;
        m.N = p->tail_col;
        e = launch_general_int(p->tile, false, m, s);
        if (e == hipSuccess) {
            KArgs r = a;
            r.N = p->N - p->tail_col;
            r.B = (const uint8_t *)B + p->tail_col;
            r.Y = (int32_t *)Y + p->tail_col;
            if (p->zpb_kind == MM_ZP_VECTOR) r.zpb = (const uint8_t *)zb + p->tail_col;
            r.y_vec = aligned16(r.Y) && (r.N * 4) % 16 == 0;
            e = launch_general_int(p->tail_tile, false, r, s);
        }
        return e == hipSuccess ? MM_OK : hip_fail(e, "kernel launch");
    }
    if (p->algo == MM_ALGO_SPLIT_K) {
        // K in partitions: INT32 partials in the plan's workspace (rows of N),
        // then their sum modulo 2^32.
        mm_status st = ensure_workspace(p);
        if (st != MM_OK) return st;
        a.W = (float *)p->ws;
        a.split = p->split;
        a.kchunk = p->kchunk;
        a.y_vec = (p->N * 4) % 16 == 0;
        e = launch_general_int(p->tile, true, a, s);
        if (e == hipSuccess) {
            KArgs r = a;
            r.y_vec = aligned16(Y);
            e = launch_splitk_reduce_i32(r, s);
        }
        return e == hipSuccess ? MM_OK : hip_fail(e, "kernel launch");
    }
    e = launch_general_int(p->tile, false, a, s);
    return e == hipSuccess ? MM_OK : hip_fail(e, "kernel launch");
}

mm_status mm_gemm_execute(mm_plan_t p, const void *A, const void *B, const void *C, void *Y, void *stream) {
    clear_error();
    if (!p) return fail(MM_ERR_NULL_ARG, "plan is NULL");
    if (!p->is_gemm) return fail(MM_ERR_BAD_OPTION, "not a Gemm plan");
    return execute_plan(p, A, B, C, Y, stream, nullptr);
}

mm_status mm_plan_set_constant_b(mm_plan_t p, const void *B, int64_t numel, void *stream) {
    clear_error();
    if (!p) return fail(MM_ERR_NULL_ARG, "plan is NULL");
    if (p->is_gemm || p->is_int)
        return fail(MM_ERR_BAD_OPTION, "constant B is for MatMul plans (it runs through mm_execute)");
    if (numel != p->b_numel)
        return fail(MM_ERR_SIZE, "constant B has %lld elements; the planned B has %lld", (long long)numel,
                    (long long)p->b_numel);
    if (!B && numel > 0) return fail(MM_ERR_NULL_ARG, "B is NULL");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(p->cb_mutex);
    if (p->cb && p->cb_device != dev)
        return fail(MM_ERR_HIP, "plan holds its constant B on device %d; setting it on device %d needs its own plan",
                    p->cb_device, dev);
    const size_t bytes = (size_t)numel * (size_t)elem_size(p->dtype);
    p->cbp_ok = false;
    if (bytes > 0) {
        if (!p->cb) {
            void *ptr = nullptr;
            e = hipMalloc(&ptr, bytes);
            if (e != hipSuccess)
                return fail(MM_ERR_ALLOC, "hipMalloc of %zu constant-B bytes: %s", bytes, hipGetErrorString(e));
            p->cb = ptr;
            p->cb_device = dev;
        }
        hipStream_t s = (hipStream_t)stream;
        e = hipMemcpyAsync(p->cb, B, bytes, hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "constant-B copy");
        mm_status st = pack_constant_b(p, s);
        if (st != MM_OK) return st;
    }
    p->cb_set = true;
    return MM_OK;
}

int mm_plan_has_constant_b(mm_plan_t p) {
    if (!p) return 0;
    std::lock_guard<std::mutex> lock(p->cb_mutex);
    return p->cb_set ? 1 : 0;
}

mm_status mm_execute_constant_b(mm_plan_t p, const void *A, void *Y, void *stream) {
    clear_error();
    if (!p) return fail(MM_ERR_NULL_ARG, "plan is NULL");
    const void *B = nullptr;
    bool packed = false;
    {
        std::lock_guard<std::mutex> lock(p->cb_mutex);
        if (!p->cb_set) return fail(MM_ERR_NO_CONSTANT_B, "the plan owns no constant B (mm_plan_set_constant_b)");
        if (p->cb) {
            int dev = -1;
            hipError_t e = hipGetDevice(&dev);
            if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
            if (dev != p->cb_device)
                return fail(MM_ERR_HIP, "plan holds its constant B on device %d; executing on device %d",
                            p->cb_device, dev);
        }
        B = p->cb;
        packed = p->cbp_ok;
    }
    if (p->is_gemm || p->is_int) return fail(MM_ERR_BAD_OPTION, "constant B serves MatMul plans");
    return execute_plan(p, A, B, nullptr, Y, stream, nullptr, packed);
}

void mm_plan_destroy(mm_plan_t p) {
    if (!p) return;
    if (p->cb || p->cbp) {
        int cur = -1;
        bool have_cur = hipGetDevice(&cur) == hipSuccess;
        if (hipSetDevice(p->cb_device) == hipSuccess) {
            if (p->cb) (void)hipFree(p->cb);
            if (p->cbp) (void)hipFree(p->cbp);
        }
        if (have_cur) (void)hipSetDevice(cur);
        p->cb = nullptr;
        p->cbp = nullptr;
    }
    if (p->ws) {
        int cur = -1;
        bool have_cur = hipGetDevice(&cur) == hipSuccess;
        if (hipSetDevice(p->ws_device) == hipSuccess) (void)hipFree(p->ws);
        if (have_cur) (void)hipSetDevice(cur);
        p->ws = nullptr;
    }
    delete p;
}

}  // extern "C"
