// k_simple.hip -- the direct kernel (tiny products), the zero fill (K == 0)
// and the ordered split-K reduction.
//
// Direct: page "Gemm and MatMul Performance Roadmap", section "Target
// computation algorithm" (tiny matrices: an un-packed kernel, since staging
// costs more than the arithmetic).  One thread computes one output element
// with an FP32 accumulator over ascending k.
//
// Split-K reduction: same page, section "Parallel execution" (K partitioned
// into partial products that are summed afterwards).  Partials are summed in
// ascending partition order, so the result is bitwise reproducible.
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
        const S *ap = A + oa + m * K;
        const S *bp = B + ob + n;
        float acc = 0.0f;
        for (int64_t k = 0; k < K; ++k) acc = fmaf(E::to_f32(ap[k]), E::to_f32(bp[k * N]), acc);
        Y[idx] = E::from_f32(acc);
    }
}

template <typename S>
__global__ __launch_bounds__(256) void k_fill_zero(S *__restrict__ Y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) Y[i] = (S)0;
}

// Y[i] = narrow(sum_{s=0}^{split-1} W[s][i]) for every output element i.
template <int DT>
__global__ __launch_bounds__(256) void k_splitk_reduce(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    const int64_t total = a.batch * a.M * a.N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const float *__restrict__ W = a.W;
    S *__restrict__ Y = (S *)a.Y;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        float acc = W[i];
        for (int s = 1; s < a.split; ++s) acc += W[(int64_t)s * total + i];
        Y[i] = E::from_f32(acc);
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
    if (dtype == MM_FLOAT) hipLaunchKernelGGL(k_fill_zero<float>, dim3(g), dim3(256), 0, s, (float *)Y, n);
    else hipLaunchKernelGGL(k_fill_zero<uint16_t>, dim3(g), dim3(256), 0, s, (uint16_t *)Y, n);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(int dtype, const KArgs &a, hipStream_t s) {
    const unsigned g = grid_for(a.batch * a.M * a.N, 65536);
    switch (dtype) {
    case MM_FLOAT: hipLaunchKernelGGL(k_splitk_reduce<MM_FLOAT>, dim3(g), dim3(256), 0, s, a); break;
    case MM_FLOAT16: hipLaunchKernelGGL(k_splitk_reduce<MM_FLOAT16>, dim3(g), dim3(256), 0, s, a); break;
    case MM_BFLOAT16: hipLaunchKernelGGL(k_splitk_reduce<MM_BFLOAT16>, dim3(g), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mm
