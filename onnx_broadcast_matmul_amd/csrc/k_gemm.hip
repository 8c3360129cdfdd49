// k_gemm.hip -- batch-broadcast tiled GEMM on the gfx950 matrix cores.
//
// Page "Gemm and MatMul Performance Roadmap", section "Target computation
// algorithm": the general path moves operand panels through the memory
// hierarchy so each staged B panel serves a whole block of rows, each staged
// A panel serves a whole block of columns, and the output tile stays in
// registers for the full reduction.  On gfx950 that becomes: one workgroup
// per BM x BN output tile, A and B K-slices staged in LDS (two stages, so the
// next slice's global loads overlap the current slice's MFMAs), FP32
// accumulators in the register file for the whole K loop, and the narrowing
// epilogue applied once at the end (page "MatMul Kernel Design", section
// "Types and algorithm selection": FP32 accumulation, final narrowing).
//
// Batches (page "MatMul Kernel Design", section "Shape and plan model") are
// a grid dimension: each workgroup decodes its batch index into per-operand
// offsets, where a zero stride re-reads the same matrix instead of a copy.
//
// Split-K (page "Gemm and MatMul Performance Roadmap", section "Parallel
// execution"): the same kernel, restricted to one K partition, writes FP32
// partials to the workspace; k_simple.hip sums them in partition order.
//
// LDS layout: every staged row (an A row or a B column) is 128 bytes of K
// (8 chunks of 16 bytes); chunk c of row r sits at c ^ ((r ^ (r >> 3)) & 7),
// so the 16-byte MFMA operand reads of 8 consecutive rows and the transposed
// B writes of 8 consecutive columns hit distinct bank groups.
//
// MFMA operands: a lane reads one 16-byte chunk of its row and of its column.
// 16-bit types: v_mfma_f32_32x32x16_{bf16,f16}, lanes 0-31 carry K chunk 2s,
// lanes 32-63 chunk 2s+1.  FP32: four v_mfma_f32_32x32x2_f32, element e of
// the lane's chunk pairing k = 4(2s) + e with k = 4(2s+1) + e.
#include "device.h"
#include "tiles.h"

namespace mm {

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

template <int BYTES>
struct RawVec;
template <>
struct RawVec<16> {
    using T = uint4;
};
template <>
struct RawVec<8> {
    using T = uint2;
};
template <>
struct RawVec<4> {
    using T = uint32_t;
};

template <int DT, int BM, int BN, bool VEC, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm(KArgs a) {
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int ES = (int)sizeof(S);
    constexpr int VE = E::kVE;        // elements per 16-byte chunk
    constexpr int BK = 128 / ES;      // K elements per stage
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int A_CHUNKS = BM * 8 / 256;  // 16-byte A chunks per thread and stage
    constexpr int CW = BN / 32;             // B columns per thread and stage
    constexpr int ROWS = BM + BN;
    static_assert(FM >= 1 && FN >= 1 && A_CHUNKS >= 1 && CW >= 1 && CW <= VE, "tile");

    __shared__ uint4 lds[2 * ROWS * 8];

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
    const S *__restrict__ Ab = (const S *)a.A + oa;
    const S *__restrict__ Bb = (const S *)a.B + ob;

    const int64_t kbeg = SPLIT ? sidx * a.kchunk : 0;
    const int64_t kend = SPLIT ? ((kbeg + a.kchunk) < K ? (kbeg + a.kchunk) : K) : K;
    const int nk = (int)((kend - kbeg + BK - 1) / BK);

    // ---- staging registers
    uint4 ra[A_CHUNKS];
    S rb[VE][CW];

    // B thread mapping: column group cg (CW columns), K chunk kc (VE rows).
    const int cg = tid & 31, kc = tid >> 5;

    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int cid = tid + 256 * i;
            const int row = cid >> 3, c = cid & 7;
            const int64_t gm = m0 + row;
            const int64_t gk = k0 + c * VE;
            if constexpr (VEC) {
                if (gm < M && gk < kend) ra[i] = *(const uint4 *)(Ab + gm * K + gk);
                else ra[i] = make_uint4(0, 0, 0, 0);
            } else {
                S tmp[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e) tmp[e] = (gm < M && gk + e < kend) ? Ab[gm * K + gk + e] : (S)0;
                __builtin_memcpy(&ra[i], tmp, 16);
            }
        }
        const int64_t gn = n0 + cg * CW;
#pragma unroll
        for (int r = 0; r < VE; ++r) {
            const int64_t gk = k0 + kc * VE + r;
            if constexpr (VEC) {
                using V = typename RawVec<CW * ES>::T;
                V v;
                if (gk < kend && gn < N) v = *(const V *)(Bb + gk * N + gn);
                else __builtin_memset(&v, 0, sizeof(v));
                __builtin_memcpy(&rb[r][0], &v, sizeof(v));
            } else {
#pragma unroll
                for (int j = 0; j < CW; ++j) rb[r][j] = (gk < kend && gn + j < N) ? Bb[gk * N + gn + j] : (S)0;
            }
        }
    };

    auto store_stage = [&](int buf) {
        uint4 *base = lds + buf * ROWS * 8;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int cid = tid + 256 * i;
            const int row = cid >> 3, c = cid & 7;
            base[row * 8 + swz(row, c)] = ra[i];
        }
        // Transpose: column (cg*CW + j) receives the VE K values of chunk kc.
#pragma unroll
        for (int j = 0; j < CW; ++j) {
            S col[VE];
#pragma unroll
            for (int r = 0; r < VE; ++r) col[r] = rb[r][j];
            uint4 v;
            __builtin_memcpy(&v, col, 16);
            const int row = BM + cg * CW + j;
            base[row * 8 + swz(row - BM, kc)] = v;
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
        load_stage(kbeg);
        store_stage(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_stage(kbeg + (int64_t)(kt + 1) * BK);

        const uint4 *As = lds + cur * ROWS * 8;
        const uint4 *Bs = As + BM * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 2 * ks + (lane >> 5);
            uint4 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wr * WM + i * 32 + (lane & 31);
                af[i] = As[row * 8 + swz(row, c)];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = wc * WN + j * 32 + (lane & 31);
                bfr[j] = Bs[col * 8 + swz(col, c)];
            }
            if constexpr (DT == MM_BFLOAT16) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
            } else if constexpr (DT == MM_FLOAT16) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, af[i]), __builtin_bit_cast(f16x8, bfr[j]), acc[i][j], 0, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const float av = __uint_as_float(e == 0 ? af[i].x : e == 1 ? af[i].y : e == 2 ? af[i].z : af[i].w);
                            const float bv = __uint_as_float(e == 0 ? bfr[j].x : e == 1 ? bfr[j].y : e == 2 ? bfr[j].z : bfr[j].w);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[i][j], 0, 0, 0);
                        }
            }
        }
        if (more) store_stage(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: 32x32 block (i, j), element r of lane: row 8(r/4) + 4(lane/32) + r%4, column lane%32.
    const int64_t ybase = b * M * N;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wr * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int64_t col = n0 + wc * WN + j * 32 + (lane & 31);
                if (row < M && col < N) {
                    if constexpr (SPLIT) {
                        a.W[(sidx * a.batch + b) * M * N + row * N + col] = acc[i][j][r];
                    } else {
                        ((S *)a.Y)[ybase + row * N + col] = E::from_f32(acc[i][j][r]);
                    }
                }
            }
}

template <int DT, int BM, int BN>
static hipError_t launch_tile(bool vec, bool split, const KArgs &a, hipStream_t s) {
    const int64_t tiles = a.batch * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * (split ? a.split : 1);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g((unsigned)tiles), blk(256);
    if (vec) {
        if (split) hipLaunchKernelGGL((k_gemm<DT, BM, BN, true, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm<DT, BM, BN, true, false>), g, blk, 0, s, a);
    } else {
        if (split) hipLaunchKernelGGL((k_gemm<DT, BM, BN, false, true>), g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm<DT, BM, BN, false, false>), g, blk, 0, s, a);
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_16(int tile, bool vec, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
    case 0: return launch_tile<DT, 256, 256>(vec, split, a, s);
    case 1: return launch_tile<DT, 256, 128>(vec, split, a, s);
    case 2: return launch_tile<DT, 128, 128>(vec, split, a, s);
    case 3: return launch_tile<DT, 128, 64>(vec, split, a, s);
    case 4: return launch_tile<DT, 64, 64>(vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

static hipError_t launch_32(int tile, bool vec, bool split, const KArgs &a, hipStream_t s) {
    switch (tile) {
    case 0: return launch_tile<MM_FLOAT, 128, 128>(vec, split, a, s);
    case 1: return launch_tile<MM_FLOAT, 128, 64>(vec, split, a, s);
    case 2: return launch_tile<MM_FLOAT, 64, 64>(vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

static_assert(kNumTiles16 == 5 && kNumTiles32 == 3, "launch switch must cover the tile table");

hipError_t launch_general(int dtype, int tile, const Align &al, bool split, const KArgs &a, hipStream_t s) {
    const bool vec = al.a && al.b;
    switch (dtype) {
    case MM_FLOAT: return launch_32(tile, vec, split, a, s);
    case MM_FLOAT16: return launch_16<MM_FLOAT16>(tile, vec, split, a, s);
    case MM_BFLOAT16: return launch_16<MM_BFLOAT16>(tile, vec, split, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
