// k_skinny.hip -- bandwidth-bound kernels for a small M (GEMV) or a small N.
//
// Skinny-M: page "Gemm and MatMul Performance Roadmap", section "Target
// computation algorithm" (M == 1 or very small M: stream B once, vectorize
// across N) and section "Remaining pull-request sequence", roadmap PR06.3
// (each B row streamed once per k and reused across the few output rows).
// Each lane owns VE adjacent output columns and keeps MT x VE FP32
// accumulators; the waves of a workgroup split K into contiguous slabs, so
// every B element is read exactly once from HBM with 16-byte coalesced loads.
// The per-wave partial sums meet in LDS and are added in wave order.
//
// Skinny-N: same page, same table (N == 1 or very small N: vectorize the K
// reduction, no B packing) and roadmap PR06.2 (several partial accumulators
// over a unit-stride K body).  Lanes run along K with 16-byte loads of A, so
// each A row is read exactly once; the few columns of B are kept in LDS
// (transposed, K contiguous) and each lane accumulates R x NT partial sums,
// reduced across the wavefront with a fixed butterfly at the end of the row.
#include "device.h"

namespace mm {

// ------------------------------------------------------------------ skinny-M

constexpr int kSkMWaves = 8;

template <int DT, int MT, bool VEC>
__global__ __launch_bounds__(64 * kSkMWaves) void k_skinny_m(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int VE = VEC ? E::kVE : 1;  // columns per lane
    constexpr int COLS = 64 * VE;         // columns per workgroup
    constexpr int KU = VEC ? E::kVE : 1;  // K rows per unrolled step

    __shared__ float red[kSkMWaves][COLS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t ncb = (N + COLS - 1) / COLS;
    const int64_t nmg = (M + MT - 1) / MT;
    int64_t id = blockIdx.x;
    const int64_t cb = id % ncb;
    id /= ncb;
    const int64_t mg = id % nmg;
    const int64_t b = id / nmg;

    int64_t oa, ob;
    batch_offsets(a.bd, b, oa, ob);
    const S *__restrict__ Ab = (const S *)a.A + oa;
    const S *__restrict__ Bb = (const S *)a.B + ob;
    const int64_t m0 = mg * MT;
    const int64_t n = cb * COLS + (int64_t)lane * VE;

    // Wave slab of K, a multiple of KU.
    const int64_t kper = ((K + kSkMWaves - 1) / kSkMWaves + KU - 1) / KU * KU;
    const int64_t klo = wave * kper;
    const int64_t khi = (klo + kper) < K ? (klo + kper) : K;

    float acc[MT][VE];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < VE; ++v) acc[m][v] = 0.0f;

    const bool col_ok = n < N;
    for (int64_t k = klo; k < khi; k += KU) {
        float bv[KU][VE];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            if constexpr (VEC) {
                uint4 raw = (col_ok && k + u < khi) ? *(const uint4 *)(Bb + (k + u) * N + n) : make_uint4(0, 0, 0, 0);
                S tmp[VE];
                __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
                for (int v = 0; v < VE; ++v) bv[u][v] = E::to_f32(tmp[v]);
            } else {
                bv[u][0] = (col_ok && k + u < khi) ? E::to_f32(Bb[(k + u) * N + n]) : 0.0f;
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool row_ok = m0 + m < M;
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const float av = (row_ok && k + u < khi) ? E::to_f32(Ab[(m0 + m) * K + k + u]) : 0.0f;
#pragma unroll
                for (int v = 0; v < VE; ++v) acc[m][v] = fmaf(av, bv[u][v], acc[m][v]);
            }
        }
    }

    // Cross-wave reduction in wave order, one output row at a time.
    S *__restrict__ Y = (S *)a.Y + b * M * N;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int v = 0; v < VE; ++v) red[wave][lane * VE + v] = acc[m][v];
        __syncthreads();
        for (int c = tid; c < COLS; c += 64 * kSkMWaves) {
            float s = red[0][c];
#pragma unroll
            for (int w = 1; w < kSkMWaves; ++w) s += red[w][c];
            const int64_t col = cb * COLS + c;
            if (m0 + m < M && col < N) Y[(m0 + m) * N + col] = E::from_f32(s);
        }
        __syncthreads();
    }
}

template <int DT, int MT>
static hipError_t launch_skm(bool vec, const KArgs &a, hipStream_t s) {
    const int cols = 64 * (vec ? Elem<DT>::kVE : 1);
    const int64_t blocks = a.batch * ((a.M + MT - 1) / MT) * ((a.N + cols - 1) / cols);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (vec) hipLaunchKernelGGL((k_skinny_m<DT, MT, true>), dim3((unsigned)blocks), dim3(64 * kSkMWaves), 0, s, a);
    else hipLaunchKernelGGL((k_skinny_m<DT, MT, false>), dim3((unsigned)blocks), dim3(64 * kSkMWaves), 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_skm_dt(bool vec, const KArgs &a, hipStream_t s) {
    // Smallest row group that covers M (B is then read once); M >= 16 uses
    // groups of 16 rows.
    if (a.M <= 1) return launch_skm<DT, 1>(vec, a, s);
    if (a.M <= 2) return launch_skm<DT, 2>(vec, a, s);
    if (a.M <= 4) return launch_skm<DT, 4>(vec, a, s);
    if (a.M <= 8) return launch_skm<DT, 8>(vec, a, s);
    return launch_skm<DT, 16>(vec, a, s);
}

hipError_t launch_skinny_m(int dtype, const Align &al, const KArgs &a, hipStream_t s) {
    const bool vec = al.b && al.y;
    switch (dtype) {
    case MM_FLOAT: return launch_skm_dt<MM_FLOAT>(vec, a, s);
    case MM_FLOAT16: return launch_skm_dt<MM_FLOAT16>(vec, a, s);
    case MM_BFLOAT16: return launch_skm_dt<MM_BFLOAT16>(vec, a, s);
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ skinny-N

constexpr int kSkNRows = 4;           // rows per wave
constexpr int kSkNBlockRows = 16;     // rows per workgroup (4 waves)
constexpr int kSkNLdsBytes = 65536;   // B slab budget

__device__ __forceinline__ float wave_sum(float v) {
    // Fixed butterfly over the 64 lanes: every lane ends with the same sum.
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int DT, int NT, bool VEC>
__global__ __launch_bounds__(256) void k_skinny_n(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int ES = (int)sizeof(S);
    constexpr int VE = VEC ? E::kVE : 1;           // K elements per lane and step
    constexpr int KSTEP = 64 * VE;                  // K elements per wave step
    constexpr int KS = (kSkNLdsBytes / (NT * ES)) / KSTEP * KSTEP;  // slab length
    static_assert(KS >= KSTEP, "slab");

    __shared__ __attribute__((aligned(16))) S bt[NT][KS];  // B slab, transposed: bt[n][k]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t nrb = (M + kSkNBlockRows - 1) / kSkNBlockRows;
    const int64_t nng = (N + NT - 1) / NT;
    const int64_t nitems = a.batch * nng * nrb;
    const int64_t nslabs = (K + KS - 1) / KS;

    int64_t loaded_key = -1;  // (batch, n-group) of the resident slab, single-slab case
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int64_t rb = item % nrb;
        const int64_t ng = (item / nrb) % nng;
        const int64_t b = item / (nrb * nng);
        int64_t oa, ob;
        batch_offsets(a.bd, b, oa, ob);
        const S *__restrict__ Ab = (const S *)a.A + oa;
        const S *__restrict__ Bb = (const S *)a.B + ob;
        const int64_t n0 = ng * NT;
        const int64_t r0 = rb * kSkNBlockRows + wave * kSkNRows;

        float acc[kSkNRows][NT];
#pragma unroll
        for (int r = 0; r < kSkNRows; ++r)
#pragma unroll
            for (int q = 0; q < NT; ++q) acc[r][q] = 0.0f;

        for (int64_t sl = 0; sl < nslabs; ++sl) {
            const int64_t k0 = sl * KS;
            const int64_t klen = (K - k0) < KS ? (K - k0) : KS;
            const int64_t key = b * nng + ng;
            if (nslabs > 1 || key != loaded_key) {
                __syncthreads();
                for (int64_t e = tid; e < (int64_t)NT * KS; e += 256) {
                    const int64_t kk = e / NT, q = e % NT;
                    S v = (S)0;
                    if (kk < klen && n0 + q < N) v = Bb[(k0 + kk) * N + n0 + q];
                    bt[q][kk] = v;
                }
                __syncthreads();
                loaded_key = key;
            }
            for (int64_t kk = (int64_t)lane * VE; kk < klen; kk += KSTEP) {
                float bf[NT][VE];
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    if constexpr (VEC) {
                        S tmp[VE];
                        __builtin_memcpy(tmp, &bt[q][kk], 16);
#pragma unroll
                        for (int v = 0; v < VE; ++v) bf[q][v] = E::to_f32(tmp[v]);
                    } else {
                        bf[q][0] = E::to_f32(bt[q][kk]);
                    }
                }
#pragma unroll
                for (int r = 0; r < kSkNRows; ++r) {
                    const int64_t row = r0 + r;
                    float av[VE];
                    if constexpr (VEC) {
                        // K is a multiple of VE and kk < klen, so the chunk is in range.
                        uint4 raw = row < M ? *(const uint4 *)(Ab + row * K + k0 + kk) : make_uint4(0, 0, 0, 0);
                        S tmp[VE];
                        __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
                        for (int v = 0; v < VE; ++v) av[v] = E::to_f32(tmp[v]);
                    } else {
                        av[0] = row < M ? E::to_f32(Ab[row * K + k0 + kk]) : 0.0f;
                    }
#pragma unroll
                    for (int q = 0; q < NT; ++q)
#pragma unroll
                        for (int v = 0; v < VE; ++v) acc[r][q] = fmaf(av[v], bf[q][v], acc[r][q]);
                }
            }
        }

        S *__restrict__ Y = (S *)a.Y + b * M * N;
#pragma unroll
        for (int r = 0; r < kSkNRows; ++r) {
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const float s = wave_sum(acc[r][q]);
                const int64_t row = r0 + r;
                if (lane == q && row < M && n0 + q < N) Y[row * N + n0 + q] = E::from_f32(s);
            }
        }
    }
}

template <int DT, int NT>
static hipError_t launch_skn(bool vec, const KArgs &a, hipStream_t s) {
    const int64_t items = a.batch * ((a.N + NT - 1) / NT) * ((a.M + kSkNBlockRows - 1) / kSkNBlockRows);
    if (items <= 0) return hipSuccess;
    // Persistent workgroups: two per CU keep their B slab resident across rows.
    const int64_t g = items < 2 * kNumCUs ? items : 2 * kNumCUs;
    if (vec) hipLaunchKernelGGL((k_skinny_n<DT, NT, true>), dim3((unsigned)g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_skinny_n<DT, NT, false>), dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_skn_dt(bool vec, const KArgs &a, hipStream_t s) {
    if (a.N <= 1) return launch_skn<DT, 1>(vec, a, s);
    if (a.N <= 2) return launch_skn<DT, 2>(vec, a, s);
    if (a.N <= 4) return launch_skn<DT, 4>(vec, a, s);
    if (a.N <= 8) return launch_skn<DT, 8>(vec, a, s);
    return launch_skn<DT, 16>(vec, a, s);
}

hipError_t launch_skinny_n(int dtype, const Align &al, const KArgs &a, hipStream_t s) {
    const bool vec = al.a;
    switch (dtype) {
    case MM_FLOAT: return launch_skn_dt<MM_FLOAT>(vec, a, s);
    case MM_FLOAT16: return launch_skn_dt<MM_FLOAT16>(vec, a, s);
    case MM_BFLOAT16: return launch_skn_dt<MM_BFLOAT16>(vec, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
