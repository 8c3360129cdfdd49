// k_skinny.hip -- bandwidth-bound kernels for a small M (GEMV) or a small N.
//
// Skinny-M: page "Gemm and MatMul Performance Roadmap", section "Target
// computation algorithm" (M == 1 or very small M: stream B once, vectorize
// across N) and section "Remaining pull-request sequence", roadmap PR06.3
// (each B row streamed once per k and reused across the few output rows).
// Each lane owns VE adjacent output columns and keeps MT x VE FP32
// accumulators; the waves of a workgroup split K into contiguous slabs, so
// every B element is read exactly once from HBM with 16-byte coalesced
// loads, and the next eight B rows are in flight while the current eight are
// multiplied.  The per-wave partial sums meet in LDS and are added in wave
// order.  When the columns give too few workgroups to keep every CU
// streaming, K is also cut into `split` chunks of whole workgroups; each
// chunk writes FP32 partial sums, which the split-K reduction adds in chunk
// order (the same fixed order on every run).
//
// Skinny-N: same page, same table (N == 1 or very small N: vectorize the K
// reduction, no B packing) and roadmap PR06.2 (several partial accumulators
// over a unit-stride K body).  Eight consecutive lanes share one row of A and
// read a full 128-byte line of it per step (16 bytes each), so each A row is
// streamed once, coalesced.  The waves of a workgroup split K; the few
// columns of B sit in LDS transposed (K contiguous) and are shared by the two
// rows each lane carries.  16-bit inputs use the packed dot instructions
// (two products into an FP32 sum).  Each lane's NT partial sums are reduced
// over its 8-lane group with a fixed butterfly, then over the K-split waves in
// wave order through LDS.
//
// Skinny-N with eight columns and K <= 4096 (16-bit types) has a kernel of
// its own on the matrix cores: v_mfma_f32_16x16x32 multiplies 16 rows of A
// by 32 elements of K against the 8 columns padded to 16, so the reduction
// costs a few MFMAs instead of the packed dot products and cross-lane sums,
// whose VALU time was about half the memory time.  A is loaded straight into
// the MFMA operand layout with every load of a wave in flight at once; each
// wave's slice of B is read through LDS with transposing reads.
#include <type_traits>

#include "device.h"

namespace mm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bfloat2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ skinny-M

constexpr int kSkMWaves = 8;

// B rows per pipeline step: deep for one or two output rows, shallower as the
// MT x VE accumulators take the registers, but never below the elements of
// one 16-byte A load (av), so that A rows keep 16-byte loads: with fewer,
// every row of a step costs one scalar A load per output row, and those
// loads, not B, set the pace.
constexpr int skm_unroll(int mt, int av) {
    const int u = mt <= 2 ? 16 : (mt <= 4 ? 8 : (mt <= 8 ? 4 : 2));
    return u > av ? u : av;
}

template <int DT, int MT, bool VEC, bool AVEC>
__global__ __launch_bounds__(64 * kSkMWaves) void k_skinny_m(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int VE = VEC ? E::kVE : 1;  // columns per lane
    constexpr int COLS = 64 * VE;         // columns per workgroup
    constexpr int AV = 16 / (int)sizeof(S);  // A elements per 16-byte load
    constexpr int U = skm_unroll(MT, AVEC ? AV : 1);
    // 16-byte A loads when rows allow them and each step covers whole chunks.
    constexpr bool AV_OK = AVEC && U % AV == 0;

    __shared__ float red[kSkMWaves][COLS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t ncb = (N + COLS - 1) / COLS;
    const int64_t nmg = (M + MT - 1) / MT;
    const int64_t ns = a.split;
    int64_t id = blockIdx.x;
    const int64_t cb = id % ncb;
    id /= ncb;
    const int64_t mg = id % nmg;
    id /= nmg;
    const int64_t sidx = id % ns;
    const int64_t b = id / ns;

    int64_t oa, ob;
    batch_offsets(a.bd, b, oa, ob);
    const S *__restrict__ Ab = (const S *)a.A + oa;
    const S *__restrict__ Bb = (const S *)a.B + ob;
    const int64_t m0 = mg * MT;
    const int64_t n = cb * COLS + (int64_t)lane * VE;
    const bool col_ok = n < N;

    // K chunk of this workgroup (a multiple of 64 rows), then the wave slab
    // within it: a multiple of U rows (and of the A vector width).
    const int64_t kb = sidx * a.kchunk;
    const int64_t ke = (kb + a.kchunk) < K ? (kb + a.kchunk) : K;
    const int64_t kper = ((ke - kb + kSkMWaves - 1) / kSkMWaves + U - 1) / U * U;
    const int64_t klo = kb + wave * kper;
    const int64_t khi = (klo + kper) < ke ? (klo + kper) : ke;

    float acc[MT][VE];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < VE; ++v) acc[m][v] = 0.0f;

    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // 16-bit types with 16-byte A and B rows: packed dot products.  The two
    // B rows k + 2p and k + 2p + 1 are paired per column with byte selects
    // (one select per column and pair of rows), and each output row takes
    // a_{k+2p} b_{k+2p} + a_{k+2p+1} b_{k+2p+1} in one v_dot2_f32 (FP32
    // accumulation), pairs in ascending k.  That halves the per-row vector
    // work of the FP32 multiply-adds and drops the FP32 conversions.
    constexpr bool DOT2 = (DT == MM_FLOAT16 || DT == MM_BFLOAT16) && VEC && AV_OK;
    static_assert(!DOT2 || (U % 2 == 0 && VE == 8), "row pairs of eight-column chunks");
    if constexpr (DOT2) {
        for (int64_t k = klo; k < khi; k += U) {
            uint32_t braw[U][4];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = col_ok && k + u < khi;
                u32x4 raw = {0, 0, 0, 0};
                if (ok) raw = __builtin_nontemporal_load((const u32x4 *)(Bb + (k + u) * N + n));
#pragma unroll
                for (int w = 0; w < 4; ++w) braw[u][w] = raw[w];
            }
            // bp[p][v]: (B[k+2p][n+v], B[k+2p+1][n+v]) as a packed pair.
            uint32_t bp[U / 2][VE];
#pragma unroll
            for (int q = 0; q < U / 2; ++q)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t x = braw[2 * q][w], y = braw[2 * q + 1][w];
                    bp[q][2 * w] = (x & 0xffffu) | (y << 16);
                    bp[q][2 * w + 1] = (x >> 16) | (y & 0xffff0000u);
                }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const bool row_ok = m0 + m < M;
                uint32_t ap[U / 2];  // (A[m][k+2p], A[m][k+2p+1])
#pragma unroll
                for (int q = 0; q < U / AV; ++q) {
                    uint4 raw = make_uint4(0, 0, 0, 0);
                    if (row_ok && k + q * AV < khi) raw = *(const uint4 *)(Ab + (m0 + m) * K + k + q * AV);
                    ap[4 * q] = raw.x; ap[4 * q + 1] = raw.y; ap[4 * q + 2] = raw.z; ap[4 * q + 3] = raw.w;
                }
#pragma unroll
                for (int q = 0; q < U / 2; ++q)
#pragma unroll
                    for (int v = 0; v < VE; ++v) {
                        if constexpr (DT == MM_FLOAT16)
                            acc[m][v] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, ap[q]),
                                                               __builtin_bit_cast(half2_t, bp[q][v]), acc[m][v], false);
                        else
                            acc[m][v] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bfloat2_t, ap[q]),
                                                                        __builtin_bit_cast(bfloat2_t, bp[q][v]),
                                                                        acc[m][v], false);
                    }
            }
        }
    }
    for (int64_t k = klo; k < (DOT2 ? klo : khi); k += U) {
        // B rows k .. k+U-1: streamed once, so loaded non-temporally.
        float bv[U][VE];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = col_ok && k + u < khi;
            if constexpr (VEC) {
                u32x4 raw = {0, 0, 0, 0};
                if (ok) raw = __builtin_nontemporal_load((const u32x4 *)(Bb + (k + u) * N + n));
                S tmp[VE];
                __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
                for (int v = 0; v < VE; ++v) bv[u][v] = E::to_f32(tmp[v]);
            } else {
                bv[u][0] = ok ? E::to_f32(Bb[(k + u) * N + n]) : 0.0f;
            }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool row_ok = m0 + m < M;
            float av[U];
            if constexpr (AV_OK) {
                // K is a multiple of AV and k of U: whole aligned 16-byte chunks (wave-uniform).
#pragma unroll
                for (int q = 0; q < U / AV; ++q) {
                    uint4 raw = make_uint4(0, 0, 0, 0);
                    if (row_ok && k + q * AV < khi) raw = *(const uint4 *)(Ab + (m0 + m) * K + k + q * AV);
                    S tmp[AV];
                    __builtin_memcpy(tmp, &raw, 16);
#pragma unroll
                    for (int e = 0; e < AV; ++e) av[q * AV + e] = E::to_f32(tmp[e]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    av[u] = (row_ok && k + u < khi) ? E::to_f32(Ab[(m0 + m) * K + k + u]) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < VE; ++v) acc[m][v] = fmaf(av[u], bv[u][v], acc[m][v]);
        }
    }

    // Cross-wave reduction in wave order, one output row at a time; with a
    // K split the sums go to the chunk's FP32 partial rows.
    S *__restrict__ Y = (S *)a.Y + b * M * N;
    float *__restrict__ P = ns > 1 ? a.W + (sidx * a.batch + b) * M * N : nullptr;
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
            if (m0 + m < M && col < N) {
                if (ns > 1) P[(m0 + m) * N + col] = s;
                else Y[(m0 + m) * N + col] = E::from_f32(s);
            }
        }
        __syncthreads();
    }
}

template <int DT, int MT>
static hipError_t launch_skm(bool vec, bool avec, const KArgs &a, hipStream_t s) {
    const int cols = 64 * (vec ? Elem<DT>::kVE : 1);
    const int64_t blocks = a.batch * ((a.M + MT - 1) / MT) * ((a.N + cols - 1) / cols) * a.split;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), blk(64 * kSkMWaves);
    if (vec) {
        if (avec) hipLaunchKernelGGL((k_skinny_m<DT, MT, true, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_skinny_m<DT, MT, true, false>), g, blk, 0, s, a);
    } else {
        if (avec) hipLaunchKernelGGL((k_skinny_m<DT, MT, false, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_skinny_m<DT, MT, false, false>), g, blk, 0, s, a);
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_skm_dt(bool vec, bool avec, const KArgs &a, hipStream_t s) {
    // Smallest row group that covers M (B is then read once); M >= 16 uses
    // groups of 16 rows.
    if (a.M <= 1) return launch_skm<DT, 1>(vec, avec, a, s);
    if (a.M <= 2) return launch_skm<DT, 2>(vec, avec, a, s);
    if (a.M <= 4) return launch_skm<DT, 4>(vec, avec, a, s);
    if (a.M <= 8) return launch_skm<DT, 8>(vec, avec, a, s);
    return launch_skm<DT, 16>(vec, avec, a, s);
}

hipError_t launch_skinny_m(int dtype, const Align &al, const KArgs &a, hipStream_t s) {
    const bool vec = al.b && al.y;  // B and Y rows in 16-byte chunks
    const bool avec = al.a;         // A rows in 16-byte chunks
    switch (dtype) {
    case MM_FLOAT: return launch_skm_dt<MM_FLOAT>(vec, avec, a, s);
    case MM_FLOAT16: return launch_skm_dt<MM_FLOAT16>(vec, avec, a, s);
    case MM_BFLOAT16: return launch_skm_dt<MM_BFLOAT16>(vec, avec, a, s);
    }
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ skinny-N

constexpr int kSkNWaves = 8;                            // 512 threads
constexpr int kSkNKParts = 8;                           // waves splitting K
constexpr int kSkNRowGroups = kSkNWaves / kSkNKParts;   // waves splitting rows
constexpr int kSkNRowsPerLane = 2;
constexpr int kSkNBlockRows = kSkNRowGroups * 8 * kSkNRowsPerLane;  // 16 rows per workgroup
constexpr int kSkNLdsBytes = 65536;                     // B slab budget

// Sum over the 8 lanes of each 8-lane group (fixed butterfly).
__device__ __forceinline__ float group8_sum(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    return v;
}

template <int DT, int NT, bool VEC, bool BVEC>
__global__ __launch_bounds__(64 * kSkNWaves) void k_skinny_n(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int ES = (int)sizeof(S);
    constexpr int VE = VEC ? 16 / ES : 1;  // K elements per lane and step
    constexpr int KSTEP = 8 * VE;          // K elements per 8-lane group and step
    constexpr int KALIGN = kSkNKParts * KSTEP;
    constexpr int KS = (kSkNLdsBytes / (NT * ES)) / KALIGN * KALIGN;  // slab length
    constexpr int R = kSkNRowsPerLane;
    static_assert(KS >= KALIGN, "slab");

    __shared__ __attribute__((aligned(16))) S bt[NT][KS];              // B slab, transposed: bt[n][k]
    __shared__ float red[kSkNKParts][kSkNBlockRows][NT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kp = wave % kSkNKParts, rg = wave / kSkNKParts;
    const int sub = lane & 7;    // position inside the 8-lane group
    const int grp = lane >> 3;   // 8-lane group = row slot

    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t nrb = (M + kSkNBlockRows - 1) / kSkNBlockRows;
    const int64_t nng = (N + NT - 1) / NT;
    int64_t id = blockIdx.x;
    const int64_t rb = id % nrb;
    id /= nrb;
    const int64_t ng = id % nng;
    const int64_t b = id / nng;

    int64_t oa, ob;
    batch_offsets(a.bd, b, oa, ob);
    const S *__restrict__ Ab = (const S *)a.A + oa;
    const S *__restrict__ Bb = (const S *)a.B + ob;
    const int64_t n0 = ng * NT;

    // Rows of this lane: slot r covers row rb*kSkNBlockRows + (r*kSkNRowGroups + rg)*8 + grp.
    int64_t row[R];
    bool row_ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = rb * kSkNBlockRows + (int64_t)(r * kSkNRowGroups + rg) * 8 + grp;
        row_ok[r] = row[r] < M;
    }

    float acc[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < NT; ++q) acc[r][q] = 0.0f;

    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // The wave's part of a slab of length klen: a multiple of KSTEP long.
    auto part_bounds = [&](int64_t klen, int64_t &plo, int64_t &phi) {
        const int64_t part = ((klen + kSkNKParts - 1) / kSkNKParts + KSTEP - 1) / KSTEP * KSTEP;
        plo = kp * part;
        phi = (plo + part) < klen ? (plo + part) : klen;
    };
    // A chunk (16 bytes) of row slot r at slab-relative k; A is streamed once: non-temporal.
    auto load_a = [&](int r, int64_t k0, int64_t kk) -> uint4 {
        u32x4 raw = {0, 0, 0, 0};
        if (row_ok[r]) raw = __builtin_nontemporal_load((const u32x4 *)(Ab + row[r] * K + k0 + kk));
        return make_uint4(raw[0], raw[1], raw[2], raw[3]);
    };
    // Multiply-accumulate one K chunk of both row slots against the B slab.
    auto mac = [&](int64_t kk, const uint4 *av) {
        uint4 bv[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) bv[q] = *(const uint4 *)&bt[q][kk];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (DT == MM_FLOAT) {
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    float s = acc[r][q];
                    s = fmaf(__uint_as_float(av[r].x), __uint_as_float(bv[q].x), s);
                    s = fmaf(__uint_as_float(av[r].y), __uint_as_float(bv[q].y), s);
                    s = fmaf(__uint_as_float(av[r].z), __uint_as_float(bv[q].z), s);
                    s = fmaf(__uint_as_float(av[r].w), __uint_as_float(bv[q].w), s);
                    acc[r][q] = s;
                }
            } else {
                const uint32_t aw[4] = {av[r].x, av[r].y, av[r].z, av[r].w};
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    const uint32_t bw[4] = {bv[q].x, bv[q].y, bv[q].z, bv[q].w};
                    float s = acc[r][q];
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        if constexpr (DT == MM_FLOAT16)
                            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, aw[w]),
                                                       __builtin_bit_cast(half2_t, bw[w]), s, false);
                        else
                            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bfloat2_t, aw[w]),
                                                                __builtin_bit_cast(bfloat2_t, bw[w]), s, false);
                    }
                    acc[r][q] = s;
                }
            }
        }
    };

    for (int64_t k0 = 0; k0 < K; k0 += KS) {
        const int64_t klen = (K - k0) < KS ? (K - k0) : KS;
        __syncthreads();
        if constexpr (BVEC) {
            // B rows are exactly NT elements in whole 16-byte chunks: a thread
            // loads BR consecutive rows and writes NT transposed 16-byte chunks.
            constexpr int BR = 16 / ES;
            constexpr int CPRW = NT * ES / 16;  // 16-byte chunks per B row
            for (int64_t kb = tid; kb * BR < klen; kb += 64 * kSkNWaves) {
                S vals[BR][NT];
#pragma unroll
                for (int r = 0; r < BR; ++r) {
                    const int64_t kk = kb * BR + r;
#pragma unroll
                    for (int c = 0; c < CPRW; ++c) {
                        uint4 v = make_uint4(0, 0, 0, 0);
                        if (kk < klen) v = *(const uint4 *)(Bb + (k0 + kk) * NT + c * (16 / ES));
                        __builtin_memcpy(&vals[r][c * (16 / ES)], &v, 16);
                    }
                }
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    S col[BR];
#pragma unroll
                    for (int r = 0; r < BR; ++r) col[r] = vals[r][q];
                    __builtin_memcpy(&bt[q][kb * BR], col, 16);
                }
            }
        } else {
            for (int64_t e = tid; e < (int64_t)NT * klen; e += 64 * kSkNWaves) {
                const int64_t kk = e / NT, q = e % NT;
                bt[q][kk] = (n0 + q < N) ? Bb[(k0 + kk) * N + n0 + q] : (S)0;
            }
        }
        __syncthreads();
        int64_t plo, phi;
        part_bounds(klen, plo, phi);
        if constexpr (VEC) {
            // K is a multiple of VE, so each lane's chunk lies wholly inside [0, klen).
#pragma unroll 2
            for (int64_t kk = plo + sub * VE; kk < phi; kk += KSTEP) {
                uint4 av[R];
#pragma unroll
                for (int r = 0; r < R; ++r) av[r] = load_a(r, k0, kk);
                mac(kk, av);
            }
        } else {
            for (int64_t kk = plo + sub; kk < phi; kk += KSTEP) {
                float bv[NT];
#pragma unroll
                for (int q = 0; q < NT; ++q) bv[q] = E::to_f32(bt[q][kk]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float av = row_ok[r] ? E::to_f32(Ab[row[r] * K + k0 + kk]) : 0.0f;
#pragma unroll
                    for (int q = 0; q < NT; ++q) acc[r][q] = fmaf(av, bv[q], acc[r][q]);
                }
            }
        }
    }

    // Reduce over the 8-lane group, then over the K parts in wave order.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const float s = group8_sum(acc[r][q]);
            if (sub == 0) red[kp][(r * kSkNRowGroups + rg) * 8 + grp][q] = s;
        }
    __syncthreads();
    S *__restrict__ Y = (S *)a.Y + b * M * N;
    for (int e = tid; e < kSkNBlockRows * NT; e += 64 * kSkNWaves) {
        const int rl = e / NT, q = e % NT;
        float s = red[0][rl][q];
#pragma unroll
        for (int p = 1; p < kSkNKParts; ++p) s += red[p][rl][q];
        const int64_t rr = rb * kSkNBlockRows + rl;
        if (rr < M && n0 + q < N) Y[rr * N + n0 + q] = E::from_f32(s);
    }
}

// ------------------------------------------------- skinny-N, eight columns

constexpr int kSkN8MaxK = 4096;  // eight waves x 512 elements of K

// Eight columns on the matrix cores.  A workgroup of 8 waves owns 16 rows
// of A; wave w owns elements 512 w .. 512 w + 511 of K (K <= 4096).  Each
// v_mfma_f32_16x16x32 multiplies the 16 rows by 32 elements of K against
// the 8 columns of B padded to 16 with zeros.  A is loaded straight into
// the operand layout (lane l: row l % 16, elements 8 (l / 16) .. + 7 of the
// K step), all 16 K steps of the wave in flight at once.  The wave's 8 KB
// slice of B sits in LDS in its own row-major layout, and the B operand
// comes from two gfx950 transposing reads per K step (lanes of columns 8 ..
// 15 point at a zero pad).  The eight waves' partial sums meet in LDS and
// are added in wave order.
constexpr int kSkN8Rows = 16;  // rows per workgroup

template <int DT>
__global__ __launch_bounds__(512) void k_skinny_n8(KArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int RB = 1;  // 16-row blocks per wave (two, with 32 rows per workgroup, measured 13 % slower)
    using E = Elem<DT>;
    using S = typename E::S;
    static_assert(sizeof(S) == 2, "16-bit element types");
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    constexpr int BW = 512 * 16;  // B bytes per wave: 512 rows of 8 columns
    __shared__ __attribute__((aligned(16))) char lds[8 * BW + 16];
    char *zero = lds + 8 * BW;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = a.M, K = a.K;
    const int64_t nrb = (M + kSkN8Rows - 1) / kSkN8Rows;
    const int64_t b = blockIdx.x / nrb;
    const int64_t row0 = (blockIdx.x % nrb) * kSkN8Rows;
    int64_t oa, ob;
    batch_offsets(a.bd, b, oa, ob);
    const S *__restrict__ A = (const S *)a.A + oa;
    const uint4 *__restrict__ Bg = (const uint4 *)((const S *)a.B + ob);  // row k of B = chunk k
    const int kw = wave * 512;

    // Loads are unconditional from clamped addresses; values outside the
    // operands become zeros.  B first (it is needed first), then every K
    // step of A.  K is a multiple of 8, so a lane's 8 elements of K lie
    // wholly inside or outside.
    uint4 bg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t k = kw + 64 * i + lane;
        const uint4 v = Bg[k < K ? k : 0];
        bg[i] = k < K ? v : make_uint4(0, 0, 0, 0);
    }
    // K elements of step s for lane group g: 32 s + 8 g .. + 7.  (Giving each
    // lane 64 contiguous bytes over four steps instead was measured 40 %
    // slower: each load instruction then touches 16 B pieces spread over the
    // rows rather than 64 contiguous bytes of each.)
    auto kstep = [](int s, int g) { return 32 * s + 8 * g; };
    uint32_t av[RB][16][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int64_t arow = row0 + rb * 16 + (lane & 15);
        const bool rok = arow < M;
        const S *ap = A + (rok ? arow : M - 1) * K;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int64_t k = kw + kstep(s, lane >> 4);
            const u32x4 t = __builtin_nontemporal_load((const u32x4 *)(ap + (k < K ? k : 0)));
            const bool ok = rok && k < K;
#pragma unroll
            for (int e = 0; e < 4; ++e) av[rb][s][e] = ok ? t[e] : 0u;
        }
    }
    char *bw = lds + wave * BW;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(uint4 *)(bw + (64 * i + lane) * 16) = bg[i];
    if (tid == 0) *(uint4 *)zero = make_uint4(0, 0, 0, 0);
    __syncthreads();

    // B operand of K step s: in each 16-lane group g, lanes 4r + j address
    // 4 columns of block row r = B row 32 s + 8 g + 4 h + r (j = 0, 1) or the
    // zero pad (j = 2, 3); lane i of the group receives column i of the
    // four rows.
    const int g = lane >> 4, gr = (lane >> 2) & 3, gj = lane & 3;
    f32x4v acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        uint2 h2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kr = kstep(s, g) + 4 * h + gr;
            const char *addr = gj < 2 ? bw + kr * 16 + gj * 8 : zero;
            if constexpr (DT == MM_BFLOAT16)
                h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                      (__attribute__((address_space(3))) bf16x4 *)(addr)));
            else
                h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                                      (__attribute__((address_space(3))) fp16x4 *)(addr)));
        }
        const uint4 bv = make_uint4(h2[0].x, h2[0].y, h2[1].x, h2[1].y);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const uint4 avv = make_uint4(av[rb][s][0], av[rb][s][1], av[rb][s][2], av[rb][s][3]);
            if constexpr (DT == MM_FLOAT16)
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, avv),
                                                                 __builtin_bit_cast(f16x8, bv), acc[rb], 0, 0, 0);
            else
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, avv),
                                                                  __builtin_bit_cast(bf16x8, bv), acc[rb], 0, 0, 0);
        }
    }

    // Element r of acc is row 4 (lane / 16) + r, column lane % 16.
    __syncthreads();
    float *red = (float *)lds;  // [wave][rb][r][lane]
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * RB + rb) * 4 + r) * 64 + lane] = acc[rb][r];
    __syncthreads();
    if (tid < kSkN8Rows * 8) {
        const int orow = tid >> 3, ocol = tid & 7;
        const int rb = orow >> 4, rr = orow & 15;
        const int ln = (rr >> 2) * 16 + ocol, r = rr & 3;
        float sum = red[(rb * 4 + r) * 64 + ln];
#pragma unroll
        for (int w = 1; w < 8; ++w) sum += red[((w * RB + rb) * 4 + r) * 64 + ln];
        const int64_t row = row0 + orow;
        if (row < M) ((S *)a.Y)[(b * M + row) * 8 + ocol] = E::from_f32(sum);
    }
#endif
}

template <int DT, int NT>
static hipError_t launch_skn(bool vec, bool bvec, const KArgs &a, hipStream_t s) {
    const int64_t items = a.batch * ((a.N + NT - 1) / NT) * ((a.M + kSkNBlockRows - 1) / kSkNBlockRows);
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g((unsigned)items), blk(64 * kSkNWaves);
    constexpr bool kWhole = NT * sizeof(typename Elem<DT>::S) % 16 == 0;
    if constexpr (kWhole) {
        if (bvec && a.N == NT) {
            if (vec) hipLaunchKernelGGL((k_skinny_n<DT, NT, true, true>), g, blk, 0, s, a);
            else hipLaunchKernelGGL((k_skinny_n<DT, NT, false, true>), g, blk, 0, s, a);
            return hipGetLastError();
        }
    }
    if (vec) hipLaunchKernelGGL((k_skinny_n<DT, NT, true, false>), g, blk, 0, s, a);
    else hipLaunchKernelGGL((k_skinny_n<DT, NT, false, false>), g, blk, 0, s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_skn_dt(bool vec, bool bvec, const KArgs &a, hipStream_t s) {
    if constexpr (DT != MM_FLOAT) {
        if (vec && bvec && a.N == 8 && a.K <= kSkN8MaxK) {
            const int64_t blocks = a.batch * ((a.M + kSkN8Rows - 1) / kSkN8Rows);
            if (blocks <= 0) return hipSuccess;
            if (blocks > 0x7fffffff) return hipErrorInvalidValue;
            hipLaunchKernelGGL(k_skinny_n8<DT>, dim3((unsigned)blocks), dim3(512), 0, s, a);
            return hipGetLastError();
        }
    }
    if (a.N <= 1) return launch_skn<DT, 1>(vec, bvec, a, s);
    if (a.N <= 2) return launch_skn<DT, 2>(vec, bvec, a, s);
    if (a.N <= 4) return launch_skn<DT, 4>(vec, bvec, a, s);
    if (a.N <= 8) return launch_skn<DT, 8>(vec, bvec, a, s);
    return launch_skn<DT, 16>(vec, bvec, a, s);
}

hipError_t launch_skinny_n(int dtype, const Align &al, const KArgs &a, hipStream_t s) {
    const bool vec = al.a;   // A rows in 16-byte chunks
    const bool bvec = al.b;  // B rows in 16-byte chunks
    switch (dtype) {
    case MM_FLOAT: return launch_skn_dt<MM_FLOAT>(vec, bvec, a, s);
    case MM_FLOAT16: return launch_skn_dt<MM_FLOAT16>(vec, bvec, a, s);
    case MM_BFLOAT16: return launch_skn_dt<MM_BFLOAT16>(vec, bvec, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
