// k_int.hip -- MatMulInteger (page "Gemm and MatMul Performance Roadmap",
// section "Remaining pull-request sequence", Roadmap PR09.1; the byte-sum
// correction of PR09.2 / PR09.3): INT8 or UINT8 A and B, optional scalar or
// per-row (A) / per-column (B) zero points, the MatMul batch broadcasting and
// rank-one rules, and
//
//   Y[m][n] = sum_k (A[m][k] - za) * (B[k][n] - zb)   (INT32, modulo 2^32).
//
// The pages fold a signed operand's offset into its zero point and recover
// the raw products with per-row / per-column byte sums; here the gfx950
// signed INT8 matrix cores take UINT8 operands with their sign bit flipped
// (x - 128), and with RA[m] = sum_k A'[m][k], CB[n] = sum_k B'[k][n] over the
// fed values A', B' and za' = za - offset_A, zb' = zb - offset_B:
//
//   Y = sum A'B' - zb' RA[m] - za' (CB[n] - K zb')   (all modulo 2^32).
//
// (The tiled kernel's zero-filled K tail becomes -128 under the flip; with
// both operands flipped the epilogue removes the 16384 each padded k adds.)
//
// The sums come from two small passes before the tiled kernel (only those
// the zero points need); k_int_direct computes the definition directly for
// tiny, unaligned or 2 GiB-spanning products.  Integer arithmetic modulo
// 2^32 is exact and associative, so every order gives the same bits.
#include "k_gemm_impl.h"

namespace mm {

// RA[r] = sum_k A'[r][k] for every stored row r of A (rows of K bytes); one
// wave per row.
__global__ __launch_bounds__(256) void k_int_rowsum(const uint8_t *__restrict__ A, int64_t rows, int64_t K,
                                                    uint32_t flip, int32_t *__restrict__ ra) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // whole waves leave together
    const uint8_t *row = A + r * K;
    uint32_t s = 0;
    for (int64_t k = lane; k < K; k += 64) s += (uint32_t)(int32_t)(int8_t)(row[k] ^ (uint8_t)flip);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += (uint32_t)__shfl_xor((int)s, off);
    if (lane == 0) ra[r] = (int32_t)s;
}

// CB[j][n] += sum over one 256-element K slice of B'[j][k][n]; CB starts at
// zero.  Grid: (column blocks, K slices, B matrices).
__global__ __launch_bounds__(256) void k_int_colsum(const uint8_t *__restrict__ B, int64_t K, int64_t N,
                                                    uint32_t flip, int32_t *__restrict__ cb) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int64_t j = blockIdx.z;
    const int64_t k0 = (int64_t)blockIdx.y * 256, k1 = k0 + 256 < K ? k0 + 256 : K;
    const uint8_t *col = B + j * K * N + n;
    uint32_t s = 0;
    for (int64_t k = k0; k < k1; ++k) s += (uint32_t)(int32_t)(int8_t)(col[k * N] ^ (uint8_t)flip);
    atomicAdd((unsigned int *)&cb[j * N + n], s);
}

__global__ __launch_bounds__(256) void k_int_fill_zero(int32_t *__restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// One thread per output: the definition, in 32-bit modular arithmetic.
__global__ __launch_bounds__(256) void k_int_direct(KArgs a) {
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t total = a.batch * M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int64_t n = idx % N;
        const int64_t m = (idx / N) % M;
        const int64_t b = idx / (M * N);
        int64_t oa, ob;
        batch_offsets(a.bd, b, oa, ob);
        const uint8_t *ap = (const uint8_t *)a.A + oa + m * K;
        const uint8_t *bp = (const uint8_t *)a.B + ob + n;
        // zero points as raw values (int_zp subtracts the UINT8 offset, added back here)
        const uint32_t za = int_zp(a.zpa, a.zpa_mode, a.a_signed, m % a.zp_rows) + (a.a_signed ? 0u : 128u);
        const uint32_t zb = int_zp(a.zpb, a.zpb_mode, a.b_signed, n) + (a.b_signed ? 0u : 128u);
        uint32_t acc = 0;
        for (int64_t k = 0; k < K; ++k) {
            const int32_t av = a.a_signed ? (int32_t)(int8_t)ap[k] : (int32_t)ap[k];
            const int32_t bv = a.b_signed ? (int32_t)(int8_t)bp[k * N] : (int32_t)bp[k * N];
            acc += ((uint32_t)av - za) * ((uint32_t)bv - zb);
        }
        ((int32_t *)a.Y)[idx] = (int32_t)acc;
    }
}

hipError_t launch_int_direct(const KArgs &a, hipStream_t s) {
    int64_t g = (a.batch * a.M * a.N + 255) / 256;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(k_int_direct, dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_int_sums(const KArgs &a, int64_t a_rows, int64_t b_mats, int32_t *ra, int32_t *cb, hipStream_t s) {
    if (ra && a_rows > 0) {
        const int64_t g = (a_rows + 3) / 4;
        if (g > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_int_rowsum, dim3((unsigned)g), dim3(256), 0, s, (const uint8_t *)a.A, a_rows, a.K,
                           a.flip_a, ra);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (cb && b_mats > 0 && a.N > 0) {
        const int64_t n = b_mats * a.N;
        hipLaunchKernelGGL(k_int_fill_zero, dim3((unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536)),
                           dim3(256), 0, s, cb, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t gx = (a.N + 255) / 256, gy = (a.K + 255) / 256;
        if (gx > 0x7fffffff || gy > 65535 || b_mats > 65535) return hipErrorInvalidValue;
        if (gy > 0)
            hipLaunchKernelGGL(k_int_colsum, dim3((unsigned)gx, (unsigned)gy, (unsigned)b_mats), dim3(256), 0, s,
                               (const uint8_t *)a.B, a.K, a.N, a.flip_b, cb);
        return hipGetLastError();
    }
    return hipSuccess;
}

static_assert(kNumTiles8 == 2, "launch switch must cover the INT8 tile table");

hipError_t launch_general_int(int tile, const KArgs &a, hipStream_t s) {
    switch (tile) {
    case 0:
        return launch_tile<MM_INT8, kTiles8[0].bm, kTiles8[0].bn, kTiles8[0].wgm, kTiles8[0].wgn, kTiles8[0].bkb,
                           kTiles8[0].stages, kTiles8[0].producers, kTiles8[0].kgroups>(true, false, a, s);
    case 1:
        return launch_tile<MM_INT8, kTiles8[1].bm, kTiles8[1].bn, kTiles8[1].wgm, kTiles8[1].wgn, kTiles8[1].bkb,
                           kTiles8[1].stages, kTiles8[1].producers, kTiles8[1].kgroups>(true, false, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
