// k_simple.hip -- the direct kernel (tiny products), the zero fill (K == 0)
// and the ordered split-K reduction.
//
// Direct: page "Gemm and MatMul Performance Roadmap", section "Target
// computation algorithm" (tiny matrices: an un-packed kernel, since staging
// costs more than the arithmetic).  One thread computes one output element
// with an FP32 accumulator over ascending k (for Gemm: of the transposed
// operands when asked, then the alpha / beta / C epilogue).
//
// Split-K reduction: same page, section "Parallel execution" (K partitioned
// into partial products that are summed afterwards).  Partials are summed in
// an order fixed by the split count alone, so the result is bitwise
// reproducible.
#include "device.h"

namespace mm {

template <int DT>
__global__ __launch_bounds__(256) void k_direct(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    const S *__restrict__ A = (const S *)a.A;
    const S *__restrict__ B = (const S *)a.B;
    S *__restrict__ Y = (S *)a.Y;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t total = a.batch * M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        const int64_t n = idx % N;
        const int64_t m = (idx / N) % M;
        const int64_t b = idx / (M * N);
        int64_t oa, ob;
        batch_offsets(a.bd, b, oa, ob);
        // A'[m][k] and B'[k][n], each stored as given or transposed (Gemm).
        const S *ap = A + oa + (a.ta ? m : m * a.lda);
        const S *bp = B + ob + (a.tb ? n * a.ldb : n);
        const int64_t sak = a.ta ? a.lda : 1, sbk = a.tb ? 1 : a.ldb;
        // Ascending k, one accumulator; the loads of 16 k are issued together
        // so their latencies overlap (the summation order is unchanged).
        float acc = 0.0f;
        int64_t k = 0;
        for (; k + 16 <= K; k += 16) {
            float av[16], bv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                av[u] = E::to_f32(ap[(k + u) * sak]);
                bv[u] = E::to_f32(bp[(k + u) * sbk]);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) acc = fmaf(av[u], bv[u], acc);
        }
        for (; k < K; ++k) acc = fmaf(E::to_f32(ap[k * sak]), E::to_f32(bp[k * sbk]), acc);
        if (a.gemm_epi) acc = gemm_epilogue<E>(a, acc, m, n);
        Y[idx] = E::from_f32(acc);
    }
}

template <typename S>
__global__ __launch_bounds__(256) void k_fill_zero(S *__restrict__ Y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) Y[i] = (S)0;
}

// Y[i] = narrow(sum_{s=0}^{split-1} W[s][i]) for every output element i.
//
// A workgroup owns OG groups of four consecutive outputs and SG partition
// lanes (SG = the split count rounded up to a power of two, at most 32; OG *
// SG = 256).  Partition lane g sums the partitions g, g + SG, g + 2 SG, ...
// in ascending order; the SG lane sums are then combined by a fixed pairwise
// tree in LDS.  The order depends only on the split count, so results are
// bitwise reproducible.  Lanes that share a partition read consecutive
// outputs, so each load instruction covers whole 128-byte lines (at SG = 32)
// or more of each partition it touches, and a lane's loads (up to eight per
// pass) are all in flight together.
template <int DT, int SG, bool VEC>
__global__ __launch_bounds__(256) void k_splitk_reduce(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int OG = 256 / SG;
    const int t = threadIdx.x, og = t % OG, sg = t / OG;
    const int64_t total = a.batch * a.M * a.N;
    const int64_t o0 = ((int64_t)blockIdx.x * OG + og) * 4;
    const float *__restrict__ W = a.W;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (o0 < total) {
        if constexpr (VEC) {
            // total is a multiple of 4: every group is whole and 16-byte aligned.
#pragma unroll 8
            for (int s = sg; s < a.split; s += SG) {
                const float4 v = *(const float4 *)(W + (int64_t)s * total + o0);
                acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
            }
        } else {
            for (int s = sg; s < a.split; s += SG)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (o0 + e < total) acc[e] += W[(int64_t)s * total + o0 + e];
        }
    }
    __shared__ float red[SG][OG][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) red[sg][og][e] = acc[e];
    __syncthreads();
#pragma unroll
    for (int w = SG / 2; w >= 1; w >>= 1) {
        if (sg < w) {
#pragma unroll
            for (int e = 0; e < 4; ++e) red[sg][og][e] += red[sg + w][og][e];
        }
        __syncthreads();
    }
    if (sg == 0 && o0 < total) {
        S *__restrict__ Y = (S *)a.Y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (o0 + e < total) {
                float v = red[0][og][e];
                if (a.gemm_epi) v = gemm_epilogue<E>(a, v, (o0 + e) / a.N, (o0 + e) % a.N);
                Y[o0 + e] = E::from_f32(v);
            }
    }
}

static unsigned grid_for(int64_t n, int64_t cap) {
    int64_t g = (n + 255) / 256;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (unsigned)g;
}

hipError_t launch_direct(int dtype, const KArgs &a, hipStream_t s) {
    const unsigned g = grid_for(a.batch * a.M * a.N, 65536);
    switch (dtype) {
    case MM_FLOAT: hipLaunchKernelGGL(k_direct<MM_FLOAT>, dim3(g), dim3(256), 0, s, a); break;
    case MM_FLOAT16: hipLaunchKernelGGL(k_direct<MM_FLOAT16>, dim3(g), dim3(256), 0, s, a); break;
    case MM_BFLOAT16: hipLaunchKernelGGL(k_direct<MM_BFLOAT16>, dim3(g), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(int dtype, void *Y, int64_t n, hipStream_t s) {
    const unsigned g = grid_for(n, 65536);
    if (dtype == MM_DOUBLE) hipLaunchKernelGGL(k_fill_zero<double>, dim3(g), dim3(256), 0, s, (double *)Y, n);
    else if (dtype == MM_INT32) hipLaunchKernelGGL(k_fill_zero<int32_t>, dim3(g), dim3(256), 0, s, (int32_t *)Y, n);
    else if (dtype == MM_FLOAT) hipLaunchKernelGGL(k_fill_zero<float>, dim3(g), dim3(256), 0, s, (float *)Y, n);
    else hipLaunchKernelGGL(k_fill_zero<uint16_t>, dim3(g), dim3(256), 0, s, (uint16_t *)Y, n);
    return hipGetLastError();
}

template <int DT, int SG>
static hipError_t launch_reduce_sg(const KArgs &a, hipStream_t s) {
    const int64_t total = a.batch * a.M * a.N;
    const int64_t groups = (total + 3) / 4;
    const int64_t g = (groups + 256 / SG - 1) / (256 / SG);
    if (g > 0x7fffffff) return hipErrorInvalidValue;
    if (total % 4 == 0) hipLaunchKernelGGL((k_splitk_reduce<DT, SG, true>), dim3((unsigned)g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_splitk_reduce<DT, SG, false>), dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_reduce_dt(const KArgs &a, hipStream_t s) {
    // Partition lanes: the split count rounded up to a power of two, at most 32.
    if (a.split <= 1) return launch_reduce_sg<DT, 1>(a, s);
    if (a.split <= 2) return launch_reduce_sg<DT, 2>(a, s);
    if (a.split <= 4) return launch_reduce_sg<DT, 4>(a, s);
    if (a.split <= 8) return launch_reduce_sg<DT, 8>(a, s);
    if (a.split <= 16) return launch_reduce_sg<DT, 16>(a, s);
    return launch_reduce_sg<DT, 32>(a, s);
}

hipError_t launch_splitk_reduce(int dtype, const KArgs &a, hipStream_t s) {
    switch (dtype) {
    case MM_FLOAT: return launch_reduce_dt<MM_FLOAT>(a, s);
    case MM_FLOAT16: return launch_reduce_dt<MM_FLOAT16>(a, s);
    case MM_BFLOAT16: return launch_reduce_dt<MM_BFLOAT16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mm
