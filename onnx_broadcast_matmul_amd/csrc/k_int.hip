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
// The tiled kernel (k_gemm_impl.h) forms RA and CB itself from the operand
// fragments it feeds the matrix cores, over its padded reduction length;
// k_int_direct computes the definition directly for tiny, unaligned or
// 2 GiB-spanning products.  Integer arithmetic modulo 2^32 is exact and
// associative, so every order gives the same bits.
#include "k_gemm_impl.h"

namespace mm {

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
        auto term = [&](uint8_t x, uint8_t y) {
            const int32_t av = a.a_signed ? (int32_t)(int8_t)x : (int32_t)x;
            const int32_t bv = a.b_signed ? (int32_t)(int8_t)y : (int32_t)y;
            return ((uint32_t)av - za) * ((uint32_t)bv - zb);
        };
        // The loads of 16 k are issued together so their latencies overlap.
        uint32_t acc = 0;
        int64_t k = 0;
        for (; k + 16 <= K; k += 16) {
            uint8_t xv[16], yv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                xv[u] = ap[k + u];
                yv[u] = bp[(k + u) * N];
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) acc += term(xv[u], yv[u]);
        }
        for (; k < K; ++k) acc += term(ap[k], bp[k * N]);
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

static_assert(kNumTiles8 == 5, "launch switch must cover the INT8 tile table");

hipError_t launch_general_int(int tile, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
    case 0:
        return launch_tile<MM_INT8, kTiles8[0].bm, kTiles8[0].bn, kTiles8[0].wgm, kTiles8[0].wgn, kTiles8[0].bkb,
                           kTiles8[0].stages, kTiles8[0].producers, kTiles8[0].kgroups>(true, split, a, s);
    case 1:
        return launch_tile<MM_INT8, kTiles8[1].bm, kTiles8[1].bn, kTiles8[1].wgm, kTiles8[1].wgn, kTiles8[1].bkb,
                           kTiles8[1].stages, kTiles8[1].producers, kTiles8[1].kgroups>(true, split, a, s);
    case 2:
        return launch_tile<MM_INT8, kTiles8[2].bm, kTiles8[2].bn, kTiles8[2].wgm, kTiles8[2].wgn, kTiles8[2].bkb,
                           kTiles8[2].stages, kTiles8[2].producers, kTiles8[2].kgroups>(true, split, a, s);
    case 3:
        return launch_tile<MM_INT8, kTiles8[3].bm, kTiles8[3].bn, kTiles8[3].wgm, kTiles8[3].wgn, kTiles8[3].bkb,
                           kTiles8[3].stages, kTiles8[3].producers, kTiles8[3].kgroups>(true, split, a, s);
    case 4:
        return launch_tile<MM_INT8, kTiles8[4].bm, kTiles8[4].bn, kTiles8[4].wgm, kTiles8[4].wgn, kTiles8[4].bkb,
                           kTiles8[4].stages, kTiles8[4].producers, kTiles8[4].kgroups>(true, split, a, s);
    }
    return hipErrorInvalidValue;
}

// MatMulInteger split-K phase 2: Y = the sum of the partitions' INT32
// partials modulo 2^32 (integer adds: any order gives the same value).  A
// thread owns four consecutive outputs.
template <bool VEC>
__global__ __launch_bounds__(256) void k_splitk_reduce_i32(KArgs a) {
    const int64_t total = a.batch * a.M * a.N;
    const int64_t o0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (o0 >= total) return;
    const uint32_t *__restrict__ W = (const uint32_t *)a.W;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
    if constexpr (VEC) {
        // total is a multiple of 4: every group is whole and 16-byte aligned.
        for (int s = 0; s < a.split; ++s) {
            const uint4 v = *(const uint4 *)(W + (int64_t)s * total + o0);
            acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
        }
        *(uint4 *)((uint32_t *)a.Y + o0) = make_uint4(acc[0], acc[1], acc[2], acc[3]);
    } else {
        for (int s = 0; s < a.split; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (o0 + e < total) acc[e] += W[(int64_t)s * total + o0 + e];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (o0 + e < total) ((uint32_t *)a.Y)[o0 + e] = acc[e];
    }
}

hipError_t launch_splitk_reduce_i32(const KArgs &a, hipStream_t s) {
    const int64_t total = a.batch * a.M * a.N;
    const int64_t g = ((total + 3) / 4 + 255) / 256;
    if (g > 0x7fffffff) return hipErrorInvalidValue;
    if (g <= 0) return hipSuccess;
    // Vector stores need Y 16-byte aligned as well.
    if (total % 4 == 0 && a.y_vec) hipLaunchKernelGGL(k_splitk_reduce_i32<true>, dim3((unsigned)g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_splitk_reduce_i32<false>, dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mm
