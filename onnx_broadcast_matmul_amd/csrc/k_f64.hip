// k_f64.hip -- DOUBLE (FP64) MatMul on the gfx950 FP64 matrix cores.
//
// Page "MatMul Kernel Design", section "Types and algorithm selection": the
// MatMul adapter accepts DOUBLE next to FLOAT, FLOAT16 and BFLOAT16, and a
// DOUBLE product accumulates in double (there is nothing to narrow).  The
// plan, the broadcast batch decode, the selector's decision points and the
// split-K reduction order are those of the other types; only the arithmetic
// changes:
//
// * k_gemm_f64 (general and split-K phase 1): one workgroup of 4 waves per
//   BM x BN output tile; each wave owns a (BM/2) x (BN/2) sub-tile made of
//   16 x 16 blocks, each accumulated by v_mfma_f64_16x16x4f64 (A operand:
//   lane l carries A[l % 16][k0 + l / 16]; B operand: lane l carries
//   B[k0 + l / 16][l % 16]; the accumulator's element r of lane l is row
//   l / 16 + 4 r, column l % 16 of the block -- rows interleaved across the
//   lane groups, unlike the FP32 16 x 16 blocks).  A and B K-slices of 16
//   doubles are staged through registers into two LDS buffers, so the next
//   slice's global loads overlap the current slice's MFMAs.  A rows in LDS
//   are padded to 17 doubles, which puts the 16 rows one fragment read
//   touches on distinct banks; B rows are read 16 consecutive doubles at a
//   time and need no padding.
// * k_direct_f64: tiny products, one thread per output, ascending k.
// * k_splitk_reduce_f64: Y = sum of the partitions' partials in ascending
//   partition order (one thread per output), so results are reproducible.
#include "device.h"
#include "tiles.h"

namespace mm {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kF64BK = 16;  // K elements (doubles) per LDS stage: 128 bytes of a row

template <int BM, int BN, bool VEC, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_f64(KArgs a) {
    constexpr int BK = kF64BK;
    constexpr int WM = BM / 2, WN = BN / 2;    // wave sub-tile
    constexpr int FM = WM / 16, FN = WN / 16;  // 16 x 16 blocks per wave
    constexpr int AP = BK + 1;                 // padded A row pitch (doubles)
    constexpr int A_CH = BM * BK / 2 / 256;    // 16-byte chunks of A per thread and stage
    constexpr int B_CH = BK * BN / 2 / 256;    // 16-byte chunks of B per thread and stage
    constexpr int BCPR = BN / 2;               // chunks per B row
    static_assert(FM >= 1 && FN >= 1 && A_CH >= 1 && B_CH >= 1, "tile");
    static_assert(BM * BK / 2 == A_CH * 256 && BK * BN / 2 == B_CH * 256, "whole chunks per thread");

    __shared__ double As[2][BM * AP];
    __shared__ __attribute__((aligned(16))) double Bs[2][BK * BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t per_batch = tiles_m * tiles_n;
    const int64_t nsplit = SPLIT ? a.split : 1;
    const int64_t total = a.batch * per_batch * nsplit;
    int64_t id = xcd_remap(blockIdx.x, total);
    const int64_t sidx = SPLIT ? id % nsplit : 0;
    id /= nsplit;
    const int64_t b = id / per_batch;
    const int64_t t = id % per_batch;
    // Grouped order inside a batch: 8 tile rows sweep the tile columns
    // together so their shared B panels stay in cache.
    constexpr int64_t GM = 8;
    const int64_t group = t / (GM * tiles_n);
    const int64_t first_m = group * GM;
    const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int64_t tm = first_m + (t % (GM * tiles_n)) % gsize;
    const int64_t tn = (t % (GM * tiles_n)) / gsize;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    int64_t oa, ob;
    batch_offsets(a.bd, b, oa, ob);
    const double *__restrict__ Ab = (const double *)a.A + oa;
    const double *__restrict__ Bb = (const double *)a.B + ob;

    const int64_t kbeg = SPLIT ? sidx * a.kchunk : 0;
    const int64_t kend = SPLIT ? ((kbeg + a.kchunk) < K ? (kbeg + a.kchunk) : K) : K;
    const int nk = (int)((kend - kbeg + BK - 1) / BK);

    double ra[A_CH][2], rb[B_CH][2];
    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int cid = tid + 256 * i;
            const int row = cid / (BK / 2), c = cid % (BK / 2);
            const int64_t gm = m0 + row, gk = k0 + 2 * c;
            if constexpr (VEC) {
                // K is even and rows are 16-byte aligned: a chunk lies wholly inside or outside.
                if (gm < M && gk < kend) {
                    const double2 v = *(const double2 *)(Ab + gm * K + gk);
                    ra[i][0] = v.x;
                    ra[i][1] = v.y;
                } else {
                    ra[i][0] = ra[i][1] = 0.0;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 2; ++e) ra[i][e] = (gm < M && gk + e < kend) ? Ab[gm * K + gk + e] : 0.0;
            }
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int cid = tid + 256 * i;
            const int kr = cid / BCPR, c = cid % BCPR;
            const int64_t gk = k0 + kr, gn = n0 + 2 * c;
            if constexpr (VEC) {
                // N is even and rows are 16-byte aligned.
                if (gk < kend && gn < N) {
                    const double2 v = *(const double2 *)(Bb + gk * N + gn);
                    rb[i][0] = v.x;
                    rb[i][1] = v.y;
                } else {
                    rb[i][0] = rb[i][1] = 0.0;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 2; ++e) rb[i][e] = (gk < kend && gn + e < N) ? Bb[gk * N + gn + e] : 0.0;
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int cid = tid + 256 * i;
            const int row = cid / (BK / 2), c = cid % (BK / 2);
            As[buf][row * AP + 2 * c] = ra[i][0];
            As[buf][row * AP + 2 * c + 1] = ra[i][1];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int cid = tid + 256 * i;
            const int kr = cid / BCPR, c = cid % BCPR;
            *(double2 *)&Bs[buf][kr * BN + 2 * c] = make_double2(rb[i][0], rb[i][1]);
        }
    };

    f64x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

    if (nk > 0) {
        load_stage(kbeg);
        store_stage(0);
    }
    __syncthreads();

    const int fr = lane & 15, fk = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_stage(kbeg + (int64_t)(kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 4; ++ks) {
            double af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = As[cur][(wr * WM + i * 16 + fr) * AP + ks * 4 + fk];
#pragma unroll
            for (int j = 0; j < FN; ++j) bf[j] = Bs[cur][(ks * 4 + fk) * BN + wc * WN + j * 16 + fr];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (more) store_stage(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: element r of block (i, j) is row lane / 16 + 4 r, column
    // lane % 16; the 16 lanes of a quarter-wave write 128 contiguous bytes.
    double *out = SPLIT ? (double *)a.W + (sidx * a.batch + b) * M * N : (double *)a.Y + b * M * N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wr * WM + i * 16 + fk + 4 * r;
                const int64_t col = n0 + wc * WN + j * 16 + fr;
                if (row < M && col < N) out[row * N + col] = acc[i][j][r];
            }
}

__global__ __launch_bounds__(256) void k_direct_f64(KArgs a) {
    const double *__restrict__ A = (const double *)a.A;
    const double *__restrict__ B = (const double *)a.B;
    double *__restrict__ Y = (double *)a.Y;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t total = a.batch * M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int64_t n = idx % N;
        const int64_t m = (idx / N) % M;
        const int64_t b = idx / (M * N);
        int64_t oa, ob;
        batch_offsets(a.bd, b, oa, ob);
        const double *ap = A + oa + m * K;
        const double *bp = B + ob + n;
        double acc = 0.0;
        // Ascending k; the loads of 16 k are issued together (same order).
        int64_t k = 0;
        for (; k + 16 <= K; k += 16) {
            double av[16], bv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                av[u] = ap[k + u];
                bv[u] = bp[(k + u) * N];
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) acc = fma(av[u], bv[u], acc);
        }
        for (; k < K; ++k) acc = fma(ap[k], bp[k * N], acc);
        Y[idx] = acc;
    }
}

// Y[i] = sum_{s=0}^{split-1} W[s][i], s ascending.
__global__ __launch_bounds__(256) void k_splitk_reduce_f64(KArgs a) {
    const int64_t total = a.batch * a.M * a.N;
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= total) return;
    const double *__restrict__ W = (const double *)a.W;
    double acc = 0.0;
    for (int s = 0; s < a.split; ++s) acc += W[(int64_t)s * total + o];
    ((double *)a.Y)[o] = acc;
}

template <int BM, int BN>
static hipError_t launch_f64_tile(bool vec, bool split, const KArgs &a, hipStream_t s) {
    const int64_t tiles = a.batch * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * (split ? a.split : 1);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g((unsigned)tiles), blk(256);
    if (vec) {
        if (split) hipLaunchKernelGGL((k_gemm_f64<BM, BN, true, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f64<BM, BN, true, false>), g, blk, 0, s, a);
    } else {
        if (split) hipLaunchKernelGGL((k_gemm_f64<BM, BN, false, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f64<BM, BN, false, false>), g, blk, 0, s, a);
    }
    return hipGetLastError();
}

static_assert(kNumTiles64 == 3 && kTiles64[0].bm == 128 && kTiles64[0].bn == 128 && kTiles64[1].bm == 64 &&
                  kTiles64[1].bn == 64 && kTiles64[2].bm == 32 && kTiles64[2].bn == 128 &&
                  kTiles64[0].bkb == kF64BK * 8 && kTiles64[1].bkb == kF64BK * 8 && kTiles64[2].bkb == kF64BK * 8,
              "launch switch must cover the FP64 tile table");

hipError_t launch_general_f64(int tile, const Align &al, bool split, const KArgs &a, hipStream_t s) {
    const bool vec = al.a && al.b;
    switch (tile) {
    case 0: return launch_f64_tile<128, 128>(vec, split, a, s);
    case 1: return launch_f64_tile<64, 64>(vec, split, a, s);
    case 2: return launch_f64_tile<32, 128>(vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_direct_f64(const KArgs &a, hipStream_t s) {
    int64_t g = (a.batch * a.M * a.N + 255) / 256;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(k_direct_f64, dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce_f64(const KArgs &a, hipStream_t s) {
    const int64_t g = (a.batch * a.M * a.N + 255) / 256;
    if (g > 0x7fffffff) return hipErrorInvalidValue;
    if (g > 0) hipLaunchKernelGGL(k_splitk_reduce_f64, dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mm
