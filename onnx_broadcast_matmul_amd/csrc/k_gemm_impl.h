// k_gemm_impl.h -- batch-broadcast tiled GEMM on the gfx950 matrix cores
// (kernel templates; k_gemm.hip and k_gemm_t.hip instantiate them).
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
#pragma once

#include <type_traits>

#include "device.h"
#include "tiles.h"

namespace mm {

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }

// Chunk position swizzle of a staged M/N-contiguous row (one k) of cpr
// 16-byte chunks, for elements of ES bytes: chunk c of k-row k sits at
// position c ^ kn_swizzle<ES>(k, cpr).  16-bit: a transposing read covers
// k = 4 consecutive rows and n = 4 chunks per half-wave; FP32: the two
// half-waves read rows k and k + 4; 8-bit: a transposing read by 32 lanes
// covers 8 consecutive k-rows and two neighbouring chunks (c, c ^ 1), and
// even shifts put the 16 pieces on 16 distinct chunk positions of the
// 256-byte bank window (for 8-chunk rows the window holds two rows, so rows
// of one parity take the four even shifts).
template <int ES>
__host__ __device__ __forceinline__ int kn_swizzle(int k, int cpr) {
    if constexpr (ES == 4) return cpr >= 16 ? 8 * ((k >> 2) & 1) : 0;  // 8 chunks: no room to move
    else if constexpr (ES == 1) return cpr >= 16 ? 2 * (k & 7) : 2 * ((k >> 1) & 3);
    else return cpr >= 16 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}

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
__global__ __launch_bounds__(256) void k_gemm_generic(KArgs a) {
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
                if (gm < M && gk < kend) ra[i] = *(const uint4 *)(Ab + gm * a.lda + gk);
                else ra[i] = make_uint4(0, 0, 0, 0);
            } else {
                // A'[m][k] is A[m][k], or A[k][m] for a transposed A.
                S tmp[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    tmp[e] = (gm < M && gk + e < kend) ? Ab[a.ta ? (gk + e) * a.lda + gm : gm * a.lda + gk + e] : (S)0;
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
                if (gk < kend && gn < N) v = *(const V *)(Bb + gk * a.ldb + gn);
                else __builtin_memset(&v, 0, sizeof(v));
                __builtin_memcpy(&rb[r][0], &v, sizeof(v));
            } else {
#pragma unroll
                for (int j = 0; j < CW; ++j)
                    rb[r][j] = (gk < kend && gn + j < N) ? Bb[a.tb ? (gn + j) * a.ldb + gk : gk * a.ldb + gn + j] : (S)0;
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
    const int64_t ybase = b * M * a.ldy;
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
                        float v = acc[i][j][r];
                        if (a.gemm_epi) v = gemm_epilogue<E>(a, v, row, col);
                        ((S *)a.Y)[ybase + row * a.ldy + col] = E::from_f32(v);
                    }
                }
            }
}


// ---------------------------------------------------------------------------
// Vectorized variant for 16-byte aligned rows: operands move from global
// memory straight into LDS (gfx950 buffer loads with the LDS destination),
// several stages deep, with no register staging.
//
// * A stage holds BKB bytes of K for the BM rows of A (row-major, K
//   contiguous) and the same K slice of B for the BN columns in B's own
//   row-major [k][n] layout.
// * Each direct load moves 16 bytes per lane into LDS at base + 16 * lane.
//   The LDS swizzle is realised by choosing which global chunk each lane
//   fetches: A rows of 128 (64) bytes store logical chunk c at
//   c ^ ((row >> 1) & 7) (c ^ ((row >> 2) & 3)), so the 16 rows that one
//   quarter-wave of fragment reads touches fall on 16 distinct 16-byte bank
//   groups; B rows store chunk c at c ^ bswz(k), chosen so that one
//   transposing read (16-bit) or one column read (FP32) touches distinct
//   bank groups across its lanes.  Chunks outside the matrix (rows past M,
//   columns past N, K past the partition end) take an offset outside the
//   buffer range, for which the hardware returns zeros, so tails need no
//   branches.
// * MFMA A operands are 16-byte LDS reads of the swizzled rows.  B operands
//   for the 16-bit types come from ds_read_b64_tr_b16: in each group of 16
//   lanes, lanes 4r..4r+3 address row r of a 4 x 16 block of B and lane i
//   receives column i, i.e. four consecutive k of one column -- two such
//   reads give the eight k values of a 32x32x16 operand.  FP32 B operands
//   are plain 4-byte reads of one column per lane.
// * MatMulInteger (INT8): a 128-byte stage is 128 k.  B operands come from
//   ds_read_b64_tr_b8 (in each 16-lane group, lanes 2r and 2r + 1 address
//   the two halves of row r of an 8 x 16 byte block, lane i receives column
//   i; two reads give the 16 k of a 32x32x32 operand).  UINT8 fragments are
//   sign-flipped into INT8, the waves form the row / column byte sums the
//   zero points need, accumulation is INT32 (modulo 2^32), and the store
//   loop applies the zero-point terms per output chunk.
// * Only waves 0..PW-1 issue the direct loads.  Waves are dealt to the four
//   SIMDs round-robin, so each SIMD pairs a producer with a wave that only
//   computes: while a producer waits on a full memory queue, its partner
//   keeps the matrix core busy.
// * The loads are asm so the compiler does not serialise later LDS reads
//   behind them; completion is awaited with explicit vmcnt before the
//   per-stage barrier.
// ---------------------------------------------------------------------------

// IFL (MatMulInteger only): bit 0 = A is UINT8, bit 1 = B is UINT8; those
// operands' fragments are sign-flipped after every read.
// PACKB: B comes from the prepacked constant-B layout (KArgs::Bp): each
// stage's B panel is one contiguous block in LDS order, copied verbatim.
template <int DT, int BM, int BN, int WGM, int WGN, int BKB, int STAGES, int PW, int KG, bool SPLIT, bool TA, bool TB,
          bool GEMM, int IFL = 0, bool PACKB = false>
__global__ __launch_bounds__(64 * WGM * WGN * KG) void k_gemm_lds_dma(KArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int NWC = WGM * WGN;         // waves of one K group
    constexpr int NW = NWC * KG;
    constexpr int ES = (int)sizeof(S);
    constexpr int VE = 16 / ES;            // elements per 16-byte chunk
    constexpr int BK = BKB / ES;           // K elements per stage
    constexpr int CA = BKB / 16;           // chunks per A row
    constexpr int KS = BKB / 32;           // MFMA steps per stage (32 bytes of K each)
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    // Each operand is staged in the layout it has in memory: K-contiguous
    // rows (A, or a transposed B) of BKB bytes, or M/N-contiguous rows (B, or
    // a transposed A) of one k each.
    constexpr int RBA = BM * ES;           // bytes of one k-row of a transposed A tile
    constexpr int CPRA = RBA / 16;
    constexpr int RBB = BN * ES;           // bytes of one B row (one k) in the tile
    constexpr int CPR = RBB / 16;          // chunks per B row
    constexpr int A_BYTES = BM * BKB;
    constexpr int B_BYTES = BK * RBB;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int A_INSTR = A_BYTES / 1024 / PW;  // 1 KB direct loads per producer and stage
    constexpr int B_INSTR = B_BYTES / 1024 / PW;
    constexpr int LPW = A_INSTR + B_INSTR;
    constexpr int A_RPB = TA ? 1024 / RBA : 1024 / BKB;  // A rows per 1 KB load
    constexpr int B_RPB = TB ? 1024 / BKB : 1024 / RBB;  // B rows per 1 KB load
    static_assert(CA == 4 || CA == 8, "A rows are 64 or 128 bytes");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
    static_assert(PW >= 1 && PW <= NW, "producers");
    static_assert(A_INSTR >= 1 && A_INSTR * PW * 1024 == A_BYTES, "A loads");
    static_assert(B_INSTR >= 1 && B_INSTR * PW * 1024 == B_BYTES, "B loads");
    static_assert(TB || (CPR >= 8 && RBB <= 1024), "B rows");
    static_assert(!TA || (CPRA >= 8 && RBA <= 1024 && (CPRA & (CPRA - 1)) == 0), "transposed A rows");
    static_assert(STAGES >= 2 && STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
    static_assert((STAGES - 2) * LPW < 64, "vmcnt range");
    static_assert(TB || (CPR & (CPR - 1)) == 0, "B row chunks");
    static_assert(KG >= 1 && KS % KG == 0, "K groups split the MFMA steps of a stage");
    // 16-byte chunk position swizzles of A rows and B rows (see above).
    auto aswz = [](int row) { return CA == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3); };
    auto mswz = [](int k, int cpr) { return kn_swizzle<ES>(k, cpr); };  // k-row of cpr chunks
    static_assert(DT != MM_INT8 || KG == 1, "INT8: no K groups");
    static_assert(!PACKB || (ES == 2 && !SPLIT && !TA && !TB && !GEMM), "prepacked B: 16-bit MatMul tiles only");
    auto bswz = [&](int k) { return mswz(k, CPR); };

    __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char *)lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave / NWC;             // K group: MFMA steps kg, kg + KG, ...
    const int wr = (wave % NWC) / WGN, wc = wave % WGN;

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
    constexpr int64_t GM = 8;
    const int64_t group = t / (GM * tiles_n);
    const int64_t first_m = group * GM;
    const int64_t gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int64_t tm = first_m + (t % (GM * tiles_n)) % gsize;
    const int64_t tn = (t % (GM * tiles_n)) / gsize;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    int64_t oa, ob;
    batch_offsets(a.bd, b, oa, ob);
    // Tile origins (k = 0): row m0 of A (column m0 of a transposed A) and
    // column n0 of B (row n0 of a transposed B).
    const char *Atile = (const char *)((const S *)a.A + oa + (TA ? m0 : m0 * a.lda));
    // Prepacked B: this matrix's panels for tile column tn, one per K stage.
    const char *Btile =
        PACKB ? (const char *)a.Bp + (ob / a.bp_mat_elems) * a.bp_mat_bytes + tn * ((K + BK - 1) / BK) * B_BYTES
              : (const char *)((const S *)a.B + ob + (TB ? n0 * a.ldb : n0));

    const int64_t kbeg = SPLIT ? sidx * a.kchunk : 0;
    const int64_t kend = SPLIT ? ((kbeg + a.kchunk) < K ? (kbeg + a.kchunk) : K) : K;
    const int nk = (int)((kend - kbeg + BK - 1) / BK);

    // Producer lane coordinates, fixed over K.
    const bool producer = wave < PW;
    uint32_t a_off[A_INSTR];
    int a_k[A_INSTR];
    bool a_ok[A_INSTR];
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
        if constexpr (!TA) {
            const int row = (wave * A_INSTR + q) * A_RPB + lane / CA;
            const int p = lane % CA;
            const int c = p ^ aswz(row);
            a_off[q] = (uint32_t)((int64_t)row * a.lda * ES + c * 16);
            a_k[q] = c * VE;
            a_ok[q] = m0 + row < M;
        } else {
            const int row = (wave * A_INSTR + q) * A_RPB + lane / CPRA;  // k within the stage
            const int p = lane % CPRA;
            const int c = p ^ mswz(row, CPRA);
            a_off[q] = (uint32_t)((int64_t)row * a.lda * ES + c * 16);
            a_k[q] = row;
            a_ok[q] = m0 + c * VE < M;
        }
    }
    uint32_t b_off[B_INSTR];
    int b_k[B_INSTR];
    bool b_ok[B_INSTR];
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q) {
        if constexpr (PACKB) {
            b_off[q] = (uint32_t)((wave * B_INSTR + q) * 1024 + lane * 16);
            b_k[q] = 0;
            b_ok[q] = true;
        } else if constexpr (!TB) {
            const int row = (wave * B_INSTR + q) * B_RPB + lane / CPR;  // k within the stage
            const int p = lane % CPR;
            const int c = p ^ bswz(row);
            b_off[q] = (uint32_t)((int64_t)row * a.ldb * ES + c * 16);
            b_k[q] = row;
            b_ok[q] = n0 + c * VE < N;
        } else {
            const int row = (wave * B_INSTR + q) * B_RPB + lane / CA;  // n within the tile
            const int p = lane % CA;
            const int c = p ^ aswz(row);
            b_off[q] = (uint32_t)((int64_t)row * a.ldb * ES + c * 16);
            b_k[q] = c * VE;
            b_ok[q] = n0 + row < N;
        }
    }

    // Lanes whose rows / columns lie outside the output never load.
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q)
        if (!a_ok[q]) a_off[q] = kOutOfRange;
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q)
        if (!b_ok[q]) b_off[q] = kOutOfRange;

    auto issue_stage = [&](int st) {
        if (!producer) return;
        const uint32_t sbase = lds_base + (st % STAGES) * STAGE_BYTES;
        const int64_t k0 = kbeg + (int64_t)st * BK;
        const i32x4 ra = buffer_rsrc(Atile + (TA ? k0 * a.lda : k0) * ES);
        const i32x4 rb = buffer_rsrc(PACKB ? Btile + (int64_t)st * B_BYTES : Btile + (TB ? k0 : k0 * a.ldb) * ES);
        if (k0 + BK <= kend) {  // a whole stage: no K check per load
#pragma unroll
            for (int q = 0; q < A_INSTR; ++q) load_to_lds16(ra, sbase + (wave * A_INSTR + q) * 1024, a_off[q]);
#pragma unroll
            for (int q = 0; q < B_INSTR; ++q)
                load_to_lds16(rb, sbase + A_BYTES + (wave * B_INSTR + q) * 1024, b_off[q]);
        } else {
            // The last, partial stage: A (and an unpacked B) past kend read
            // zeros; a prepacked panel is already zero past K.
            const int rem = (int)(kend - k0);  // 0 < rem < BK
#pragma unroll
            for (int q = 0; q < A_INSTR; ++q)
                load_to_lds16(ra, sbase + (wave * A_INSTR + q) * 1024, a_k[q] < rem ? a_off[q] : kOutOfRange);
#pragma unroll
            for (int q = 0; q < B_INSTR; ++q)
                load_to_lds16(rb, sbase + A_BYTES + (wave * B_INSTR + q) * 1024,
                              PACKB || b_k[q] < rem ? b_off[q] : kOutOfRange);
        }
    };

    using AccT = typename std::conditional<DT == MM_INT8, i32x16, f32x16>::type;
    AccT acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    uint4 fa[2][FM], fb[2][FN];
    // MatMulInteger: running row sums of A' and column sums of B' over the
    // stages' K, including the zero padding of the last.  The WGN waves that
    // share a row block take turns by MFMA step (step ks goes to the wave
    // with wc == ks % WGN), as do the WGM waves that share a column block;
    // their partial sums meet in LDS.
    constexpr int SA = DT == MM_INT8 ? FM : 1, SB = DT == MM_INT8 ? FN : 1;
    int32_t rs_acc[SA], cs_acc[SB];
#pragma unroll
    for (int i = 0; i < SA; ++i) rs_acc[i] = 0;
#pragma unroll
    for (int j = 0; j < SB; ++j) cs_acc[j] = 0;
    const bool do_rs = DT == MM_INT8 && a.sum_a;
    const bool do_cs = DT == MM_INT8 && a.sum_b;
    __shared__ int32_t sums_lds[DT == MM_INT8 ? BM + BN : 1];
    if constexpr (DT == MM_INT8) {
        // Cleared before the main loop's first barrier, added to after it.
        for (int x = tid; x < BM + BN; x += 64 * NW) sums_lds[x] = 0;
    }
    // Gemm with a per-column or per-row C: the tile's BN (or BM) values of C,
    // staged in LDS as FP32 before the main loop (visible after its first
    // barrier), so the epilogue reads them from LDS instead of waiting on
    // global loads at the end of the tile.  Positions outside the output hold
    // zero.
    constexpr bool EPI = GEMM && !SPLIT;
    __shared__ __attribute__((aligned(16))) float ebias[EPI ? (BM > BN ? BM : BN) : 1];
    if constexpr (EPI) {
        if (a.gemm_epi && (a.c_mode == kBiasRow || a.c_mode == kBiasCol)) {
            const S *Cp = (const S *)a.C;
            const bool row = a.c_mode == kBiasRow;  // one C value per output column
            const int len = row ? BN : BM;
            const int64_t base = row ? n0 : m0, lim = row ? N : M;
            for (int x = tid; x < len; x += 64 * NW) ebias[x] = base + x < lim ? E::to_f32(Cp[base + x]) : 0.0f;
        }
    }
    // Fragment of K-contiguous rows: chunk c of row `row`.
    auto read_k = [&](const char *Xs, int row, int c) -> uint4 {
        return *(const uint4 *)(Xs + row * BKB + ((c ^ aswz(row)) * 16));
    };
    // Fragment of M/N-contiguous k-rows (rbytes per row, cpr chunks): the
    // lane's 8 (16-bit) or 4 (FP32) consecutive k of index base + lane % 32.
    auto read_mn = [&](const char *Xs, int rbytes, int cpr, int base, int ks, int c) -> uint4 {
        if constexpr (ES == 1) {
            // 8-bit transposing reads: in each 16-lane group, lanes 2r, 2r + 1
            // address the two 8-byte halves of row r of an 8 x 16 block and
            // lane i receives column i -- two reads give 16 consecutive k.
            const int G = lane >> 4, jl = lane & 15;
            const int n = base + (G & 1) * 16 + (jl & 1) * 8;
            uint2 h2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = ks * 32 + (G >> 1) * 16 + h * 8 + (jl >> 1);
                const int p = (n >> 4) ^ mswz(k, cpr);
                const char *addr = Xs + k * rbytes + p * 16 + ((n >> 3) & 1) * 8;
                typedef int i32x2v __attribute__((ext_vector_type(2)));
                h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                                      (__attribute__((address_space(3))) i32x2v *)(addr)));
            }
            return make_uint4(h2[0].x, h2[0].y, h2[1].x, h2[1].y);
        } else if constexpr (ES == 2) {
            const int G = lane >> 4, jl = lane & 15;
            const int n = base + (G & 1) * 16 + (jl & 3) * 4;
            uint2 h2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = ks * 16 + (G >> 1) * 8 + h * 4 + (jl >> 2);
                const int p = (n >> 3) ^ mswz(k, cpr);
                const char *addr = Xs + k * rbytes + p * 16 + ((n >> 2) & 1) * 8;
                if constexpr (DT == MM_BFLOAT16)
                    h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                          (__attribute__((address_space(3))) bf16x4 *)(addr)));
                else
                    h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                                          (__attribute__((address_space(3))) fp16x4 *)(addr)));
            }
            return make_uint4(h2[0].x, h2[0].y, h2[1].x, h2[1].y);
        } else {
            const int n = base + (lane & 31);
            uint32_t v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = c * 4 + e;
                const int p = (n >> 2) ^ mswz(k, cpr);
                v[e] = *(const uint32_t *)(Xs + k * rbytes + p * 16 + (n & 3) * 4);
            }
            return make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    auto read_frags = [&](int buf, int ks, int slot) {
        const char *As = lds + buf * STAGE_BYTES;
        const char *Bs = As + A_BYTES;
        const int c = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if constexpr (TA) fa[slot][i] = read_mn(As, RBA, CPRA, wr * WM + i * 32, ks, c);
            else fa[slot][i] = read_k(As, wr * WM + i * 32 + (lane & 31), c);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (TB) fb[slot][j] = read_k(Bs, wc * WN + j * 32 + (lane & 31), c);
            else fb[slot][j] = read_mn(Bs, RBB, CPR, wc * WN + j * 32, ks, c);
        }
        if constexpr (DT == MM_INT8) {  // UINT8 operands: x - 128 in INT8
            constexpr uint32_t X = 0x80808080u;
            if constexpr (IFL & 1) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    fa[slot][i].x ^= X; fa[slot][i].y ^= X; fa[slot][i].z ^= X; fa[slot][i].w ^= X;
                }
            }
            if constexpr (IFL & 2) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    fb[slot][j].x ^= X; fb[slot][j].y ^= X; fb[slot][j].z ^= X; fb[slot][j].w ^= X;
                }
            }
            // Byte sums of the 16 k this lane holds: dot products with ones.
            if (do_rs && ks % WGN == wc) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const uint4 &f = fa[slot][i];
                    int s = rs_acc[i];
                    s = __builtin_amdgcn_sdot4((int)f.x, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4((int)f.y, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4((int)f.z, 0x01010101, s, false);
                    rs_acc[i] = __builtin_amdgcn_sdot4((int)f.w, 0x01010101, s, false);
                }
            }
            if (do_cs && ks % WGM == wr) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const uint4 &f = fb[slot][j];
                    int s = cs_acc[j];
                    s = __builtin_amdgcn_sdot4((int)f.x, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4((int)f.y, 0x01010101, s, false);
                    s = __builtin_amdgcn_sdot4((int)f.z, 0x01010101, s, false);
                    cs_acc[j] = __builtin_amdgcn_sdot4((int)f.w, 0x01010101, s, false);
                }
            }
        }
    };
    // The B fragment is the first MFMA operand, so each 32x32 accumulator holds
    // the transposed output block: column n of the block in the MFMA's row
    // position, row m in its column position.
    auto mfmas = [&](int slot) {
        if constexpr (DT == MM_INT8) {
            typedef int i32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4v, fb[slot][j]),
                                                                     __builtin_bit_cast(i32x4v, fa[slot][i]),
                                                                     acc[i][j], 0, 0, 0);
        } else if constexpr (DT == MM_BFLOAT16) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[slot][j]),
                                                                       __builtin_bit_cast(bf16x8, fa[slot][i]),
                                                                       acc[i][j], 0, 0, 0);
        } else if constexpr (DT == MM_FLOAT16) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fb[slot][j]),
                                                                      __builtin_bit_cast(f16x8, fa[slot][i]),
                                                                      acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const uint4 &x = fa[slot][i];
                        const uint4 &y = fb[slot][j];
                        const float av = __uint_as_float(e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w);
                        const float bv = __uint_as_float(e == 0 ? y.x : e == 1 ? y.y : e == 2 ? y.z : y.w);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv, av, acc[i][j], 0, 0, 0);
                    }
        }
    };

    // Pipeline: STAGES - 1 stages in flight ahead of the one computed.
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_stage(s);

    for (int kt = 0; kt < nk; ++kt) {
        // This wave's loads of stage kt are complete once at most the loads of
        // the stages issued after it are still outstanding.
        const int later = (nk - 1 - kt) < (STAGES - 2) ? (nk - 1 - kt) : (STAGES - 2);
        if (later >= STAGES - 2) wait_vmcnt<(STAGES - 2) * LPW>();
        else if (STAGES > 3 && later == 1) wait_vmcnt<LPW>();
        else wait_vmcnt<0>();
        // After the barrier every wave's loads of stage kt have landed and every
        // wave has finished reading stage kt - 1, whose buffer is refilled next.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // INT8 issues the next stage's loads after its first MFMA step
        // (measured 1.6 % faster); the other types right after the barrier.
        constexpr bool LATE_ISSUE = DT == MM_INT8 && KG == 1;
        if (!LATE_ISSUE && kt + STAGES - 1 < nk) issue_stage(kt + STAGES - 1);
        const int buf = kt % STAGES;
        if constexpr (KG == 1) {
            // 16-bit types: the compiler, left alone, reuses one set of
            // fragment registers and waits on each step's LDS reads right
            // before its MFMAs.  Scheduling groups (mask 0x100: LDS reads,
            // 0x008: MFMAs) keep the next step's reads ahead, in pairs
            // between the step's first MFMAs, so that they land while the
            // rest of the step's MFMAs run.  (Measured: no gain for FP32 or
            // INT8, which keep the compiler's order.)
            constexpr bool SCHED = DT == MM_FLOAT16 || DT == MM_BFLOAT16;
            constexpr int RPA = TA ? 2 : 1;  // LDS reads per A fragment (transposing: two)
            constexpr int RPB = TB ? 1 : 2;  // per B fragment
            constexpr int RPS = FM * RPA + FN * RPB;
            constexpr int MPS = FM * FN;     // MFMAs per step
            read_frags(buf, 0, 0);
            if constexpr (SCHED) __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) read_frags(buf, ks + 1, (ks + 1) & 1);
                mfmas(ks & 1);
                if (LATE_ISSUE && ks == 0 && kt + STAGES - 1 < nk) issue_stage(kt + STAGES - 1);
                if constexpr (SCHED) {
                    if (ks + 1 < KS) {
#pragma unroll
                        for (int q = 0; q < RPS / 2; ++q) {
                            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        }
                        if constexpr (MPS > RPS / 2) __builtin_amdgcn_sched_group_barrier(0x008, MPS - RPS / 2, 0);
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x008, MPS, 0);
                    }
                }
            }
        } else {
            read_frags(buf, kg, 0);
#pragma unroll
            for (int j = 0; j < KS / KG; ++j) {
                if (j + 1 < KS / KG) read_frags(buf, kg + (j + 1) * KG, (j + 1) & 1);
                mfmas(j & 1);
            }
        }
    }

    // MatMulInteger sums: lanes l and l + 32 held the two 16-k halves of
    // each step; the waves' partial totals are added into the LDS table the
    // store loop reads (integer adds: the order does not matter).
    if constexpr (DT == MM_INT8) {
        if (do_rs) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int s = rs_acc[i] + __shfl_xor(rs_acc[i], 32);
                if (lane < 32) atomicAdd(&sums_lds[wr * WM + i * 32 + lane], s);
            }
        }
        if (do_cs) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int s = cs_acc[j] + __shfl_xor(cs_acc[j], 32);
                if (lane < 32) atomicAdd(&sums_lds[BM + wc * WN + j * 32 + lane], s);
            }
        }
    }

    // Epilogue through LDS.  Element r of a lane's accumulator block (i, j) is
    // output row (lane % 32) and column 8(r/4) + 4(lane/32) + r%4 of the
    // block, so the four elements r = 4q..4q+3 are four consecutive columns of
    // one row: one 8-byte (16-bit output) or 16-byte (FP32) LDS write.  The
    // tile is row-major with 16-byte chunk c of tile row r at c ^ (r % OCPR),
    // which spreads the 32 rows of one write over distinct chunks; the
    // workgroup then writes whole 16-byte chunks of output rows.  Tiles larger
    // than the stage buffers go in row passes.
    // Split-K partials: FP32, or INT32 for MatMulInteger (added modulo 2^32).
    using O = typename std::conditional<DT == MM_INT8, int32_t, typename std::conditional<SPLIT, float, S>::type>::type;
    constexpr int OS = (int)sizeof(O);
    constexpr int OV = 16 / OS;            // output elements per chunk
    constexpr int OCPR = BN * OS / 16;     // output chunks per tile row
    constexpr int NP = (BM * BN * OS + STAGES * STAGE_BYTES - 1) / (STAGES * STAGE_BYTES);
    constexpr int PR = BM / NP;            // tile rows per pass
    static_assert(BM % NP == 0, "epilogue passes");
    static_assert((OCPR & (OCPR - 1)) == 0 && OCPR >= 8, "tile row swizzle");
    char *tile = lds;
    // Output rows: the dense workspace (pitch N) or Y (pitch ldy).
    const int64_t ldo = SPLIT ? N : a.ldy;
    O *out = SPLIT ? (O *)(a.W + (sidx * a.batch + b) * M * N) : (O *)a.Y + b * M * a.ldy;
    if constexpr (KG > 1) {
        // Groups 1..KG-1 hand their accumulators to group 0 through LDS
        // (element-major, lane-contiguous), which adds them in group order.
        static_assert((KG - 1) * BM * BN * 4 <= STAGES * STAGE_BYTES, "K-group exchange fits in LDS");
        float *xch = (float *)lds;
        const int wq = wave % NWC;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        xch[((((kg - 1) * NWC + wq) * FM + i) * FN * 16 + j * 16 + r) * 64 + lane] = acc[i][j][r];
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kg == 0) {
#pragma unroll
            for (int g = 1; g < KG; ++g)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[i][j][r] += xch[((((g - 1) * NWC + wq) * FM + i) * FN * 16 + j * 16 + r) * 64 + lane];
        }
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    // Gemm: a scalar C is read once here; per-column and per-row C come from
    // the LDS copy staged before the main loop; a full C is read per element
    // below.  Only the Gemm instantiations carry the epilogue's code.
    float bias_one = 0.0f;
    int cmode = kBiasNone;
    if constexpr (EPI) {
        if (a.gemm_epi) {
            cmode = a.c_mode;
            if (cmode == kBiasScalar) bias_one = E::to_f32(((const S *)a.C)[0]);
        }
    }
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int rl = wr * WM + i * 32 + (lane & 31) - pass * PR;
            if (kg == 0 && (NP == 1 || (rl >= 0 && rl < PR))) {
                char *trow = tile + rl * (BN * OS);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int cl = wc * WN + j * 32 + 8 * q + 4 * (lane >> 5);
                        const int ch = (cl / OV) ^ (rl & (OCPR - 1));
                        char *dst = trow + ch * 16 + (cl % OV) * OS;
                        if constexpr (DT == MM_INT8) {
                            // Raw INT32 sums of the fed operands; the zero-point
                            // terms are applied per output chunk below.
                            const AccT &v = acc[i][j];
                            *(uint4 *)dst = make_uint4((uint32_t)v[4 * q], (uint32_t)v[4 * q + 1],
                                                       (uint32_t)v[4 * q + 2], (uint32_t)v[4 * q + 3]);
                            continue;
                        }
                        const AccT &v = acc[i][j];
                        float w[4] = {(float)v[4 * q], (float)v[4 * q + 1], (float)v[4 * q + 2], (float)v[4 * q + 3]};
                        if constexpr (EPI) {
                            if (a.gemm_epi) {
                                if (cmode == kBiasFull) {
                                    // One row of C, four consecutive columns (C rows
                                    // need not be 16-byte aligned: element loads).
                                    const int64_t gm = m0 + wr * WM + i * 32 + (lane & 31);
                                    const S *Cr = (const S *)a.C + (gm < M ? gm : 0) * a.ldc + n0 + cl;
#pragma unroll
                                    for (int e = 0; e < 4; ++e) {
                                        const float c = gm < M && n0 + cl + e < N ? E::to_f32(Cr[e]) : 0.0f;
                                        w[e] = a.alpha * w[e] + a.beta * c;
                                    }
                                } else if (cmode == kBiasRow) {
                                    const float4 c4 = *(const float4 *)&ebias[cl];
                                    const float c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                                    for (int e = 0; e < 4; ++e) w[e] = a.alpha * w[e] + a.beta * c[e];
                                } else {
                                    const float c = cmode == kBiasCol ? ebias[wr * WM + i * 32 + (lane & 31)] : bias_one;
#pragma unroll
                                    for (int e = 0; e < 4; ++e)
                                        w[e] = cmode == kBiasNone ? a.alpha * w[e] : a.alpha * w[e] + a.beta * c;
                                }
                            }
                        }
                        if constexpr (OS == 4) {
                            *(float4 *)dst = make_float4(w[0], w[1], w[2], w[3]);
                        } else {
                            *(uint2 *)dst = make_uint2(E::pack2(w[0], w[1]), E::pack2(w[2], w[3]));
                        }
                    }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int idx = tid; idx < PR * OCPR; idx += 64 * NW) {
            const int rl = idx / OCPR, c = idx % OCPR;
            const int64_t row = m0 + pass * PR + rl, col = n0 + (int64_t)c * OV;
            if (row < M && col < N) {
                uint4 v = *(const uint4 *)(tile + rl * (BN * OS) + (c ^ (rl & (OCPR - 1))) * 16);
                if constexpr (DT == MM_INT8) {
                    // Over the padded reduction length Kp (zero bytes after
                    // K, i.e. raw values 0) the kernel holds P = sum A'B',
                    // RA = sum A' and CB = sum B'; then
                    //   Y = P - zb' RA - za' (CB - Kp zb') - (Kp - K) za zb
                    // modulo 2^32, with za' = za - offset_A, zb' = zb -
                    // offset_B and raw zero points za, zb.  Rows and the
                    // zero-point period are below 2^31.
                    const uint32_t za = int_zp(a.zpa, a.zpa_mode, a.a_signed, (uint32_t)row % (uint32_t)a.zp_rows);
                    const uint32_t za_raw = za + (a.a_signed ? 0u : 128u);
                    // (K is this partition's length under split-K: each
                    // partition's terms are those of its own K range, and
                    // their sum is the whole product's.)
                    const uint32_t kp = (uint32_t)((int64_t)nk * BK), pad = kp - (uint32_t)(kend - kbeg);
                    const uint32_t rsum = a.sum_a ? (uint32_t)sums_lds[pass * PR + rl] : 0u;
                    uint32_t y[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t gn = col + e;
                        if (gn < N) {
                            const uint32_t zb = int_zp(a.zpb, a.zpb_mode, a.b_signed, gn);
                            const uint32_t csum = a.sum_b ? (uint32_t)sums_lds[BM + c * OV + e] : 0u;
                            y[e] -= zb * rsum + za * (csum - kp * zb) + pad * za_raw * (zb + (a.b_signed ? 0u : 128u));
                        }
                    }
                    v = make_uint4(y[0], y[1], y[2], y[3]);
                }
                O *dst = out + row * ldo + col;
                if (a.y_vec) {
                    // Rows are whole 16-byte chunks: the chunk lies inside the row.
                    const u32x4 w = {v.x, v.y, v.z, v.w};
                    __builtin_nontemporal_store(w, (u32x4 *)dst);
                } else {
                    O e[OV];
                    __builtin_memcpy(e, &v, 16);
#pragma unroll
                    for (int q = 0; q < OV; ++q)
                        if (col + q < N) dst[q] = e[q];
                }
            }
        }
    }
#endif
}

// Persistent variant for 16-bit MatMul with two LDS stages: one workgroup per
// CU walks the tiles blockIdx.x, blockIdx.x + gridDim.x, ... (in the same
// XCD-aware order as the one-tile-per-workgroup grid), and the stage
// pipeline runs on across tile boundaries: the first stage of the next tile
// is loaded while the last stage of the current one is multiplied.  The
// output leaves straight from the accumulators (8-byte stores, no LDS), so
// the stage buffers never wait for an epilogue and the stores of one tile
// drain while the next tile computes.  Per tile, the K order, the MFMA
// sequence and the narrowing are those of k_gemm_lds_dma, so both give the
// same bits.
template <int DT, int BM, int BN, int WGM, int WGN, int BKB, int PW>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm_persist(KArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int ES = (int)sizeof(S);
    static_assert(ES == 2, "16-bit element types");
    constexpr int STAGES = 2;
    constexpr int VE = 16 / ES;
    constexpr int BK = BKB / ES;
    constexpr int CA = BKB / 16;
    constexpr int KS = BKB / 32;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int RBB = BN * ES;
    constexpr int CPR = RBB / 16;
    constexpr int A_BYTES = BM * BKB;
    constexpr int B_BYTES = BK * RBB;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int A_INSTR = A_BYTES / 1024 / PW;
    constexpr int B_INSTR = B_BYTES / 1024 / PW;
    constexpr int A_RPB = 1024 / BKB;
    constexpr int B_RPB = 1024 / RBB;
    static_assert(CA == 8, "A rows are 128 bytes");
    static_assert(FM >= 1 && FN >= 1 && PW >= 1 && PW <= WGM * WGN, "wave tile, producers");
    static_assert(A_INSTR >= 1 && A_INSTR * PW * 1024 == A_BYTES, "A loads");
    static_assert(B_INSTR >= 1 && B_INSTR * PW * 1024 == B_BYTES, "B loads");
    static_assert(CPR >= 8 && RBB <= 1024 && (CPR & (CPR - 1)) == 0, "B rows");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
    static_assert(FM * FN * 4 < 64, "stores counted by vmcnt");
    auto aswz = [](int row) { return (row >> 1) & 7; };
    auto bswz = [](int k) { return kn_swizzle<ES>(k, CPR); };

    __shared__ __attribute__((aligned(1024))) char lds[STAGES * STAGE_BYTES];
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char *)lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / WGN, wc = wave % WGN;
    // Tile counts, origins and batch indices fit in 32 bits (checked at
    // launch); only element offsets are 64-bit.
    const int64_t M = a.M, N = a.N, K = a.K;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int per_batch = tiles_m * tiles_n;
    const int total = (int)a.batch * per_batch;
    const int G = (int)gridDim.x;
    const int bid = (int)blockIdx.x;
    const int ntiles = bid < total ? (total - 1 - bid) / G + 1 : 0;
    const int nk = (int)((K + BK - 1) / BK);
    if (ntiles == 0 || nk == 0) return;

    // Tile j of this workgroup: batch, origin and operand panels.
    struct Tile {
        int b, m0, n0;
        const char *At, *Bt;
    };
    auto tile_at = [&](int j) {
        const int id = (int)xcd_remap(bid + j * G, total);
        const int b = id / per_batch, t = id % per_batch;
        constexpr int GM = 8;
        const int group = t / (GM * tiles_n);
        const int first_m = group * GM;
        const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
        const int tm = first_m + (t % (GM * tiles_n)) % gsize;
        const int tn = (t % (GM * tiles_n)) / gsize;
        int64_t oa, ob;
        batch_offsets(a.bd, b, oa, ob);
        Tile T;
        T.b = b;
        T.m0 = tm * BM;
        T.n0 = tn * BN;
        T.At = (const char *)((const S *)a.A + oa + (int64_t)T.m0 * a.lda);
        T.Bt = (const char *)((const S *)a.B + ob + T.n0);
        return T;
    };

    // Stage st of tile T into LDS buffer buf (whole tiles and stages: M, N
    // and K are multiples of BM, BN and BK).  Lane offsets are formed here
    // rather than kept in registers across the loop.
    const bool producer = wave < PW;
    const uint32_t a_pitch = (uint32_t)(a.lda * ES), b_pitch = (uint32_t)(a.ldb * ES);
    auto issue = [&](const Tile &T, int st, int buf) {
        if (!producer) return;
        const uint32_t sbase = lds_base + buf * STAGE_BYTES;
        const int64_t k0 = (int64_t)st * BK;
        const i32x4 ra = buffer_rsrc(T.At + k0 * ES);
        const i32x4 rb = buffer_rsrc(T.Bt + k0 * a.ldb * ES);
#pragma unroll
        for (int q = 0; q < A_INSTR; ++q) {
            const int row = (wave * A_INSTR + q) * A_RPB + lane / CA;
            const int c = (lane % CA) ^ aswz(row);
            load_to_lds16(ra, sbase + (wave * A_INSTR + q) * 1024, (uint32_t)row * a_pitch + c * 16);
        }
#pragma unroll
        for (int q = 0; q < B_INSTR; ++q) {
            const int row = (wave * B_INSTR + q) * B_RPB + lane / CPR;
            const int c = (lane % CPR) ^ bswz(row);
            load_to_lds16(rb, sbase + A_BYTES + (wave * B_INSTR + q) * 1024, (uint32_t)row * b_pitch + c * 16);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    uint4 fa[2][FM], fb[2][FN];
    auto read_frags = [&](int buf, int ks, int slot) {
        const char *As = lds + buf * STAGE_BYTES;
        const char *Bs = As + A_BYTES;
        const int c = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wr * WM + i * 32 + (lane & 31);
            fa[slot][i] = *(const uint4 *)(As + row * BKB + ((c ^ aswz(row)) * 16));
        }
        const int G4 = lane >> 4, jl = lane & 15;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = wc * WN + j * 32 + (G4 & 1) * 16 + (jl & 3) * 4;
            uint2 h2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = ks * 16 + (G4 >> 1) * 8 + h * 4 + (jl >> 2);
                const int p = (n >> 3) ^ bswz(k);
                const char *addr = Bs + k * RBB + p * 16 + ((n >> 2) & 1) * 8;
                if constexpr (DT == MM_BFLOAT16)
                    h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                          (__attribute__((address_space(3))) bf16x4 *)(addr)));
                else
                    h2[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                                          (__attribute__((address_space(3))) fp16x4 *)(addr)));
            }
            fb[slot][j] = make_uint4(h2[0].x, h2[0].y, h2[1].x, h2[1].y);
        }
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if constexpr (DT == MM_BFLOAT16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[slot][j]),
                                                                       __builtin_bit_cast(bf16x8, fa[slot][i]),
                                                                       acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fb[slot][j]),
                                                                      __builtin_bit_cast(f16x8, fa[slot][i]),
                                                                      acc[i][j], 0, 0, 0);
            }
    };
    // Epilogue through the stage buffer just consumed, in WGM passes of the
    // WM rows of one row of waves.  Element r of a lane's accumulator block
    // (i, j) is row lane % 32 and column 8 (r / 4) + 4 (lane / 32) + r % 4
    // of the block, so r = 4q .. 4q + 3 are four consecutive columns of one
    // row: one 8-byte LDS write.  Tile row r keeps its 16-byte chunk c at
    // c ^ (r % OCPR); the workgroup then stores whole 16-byte chunks of
    // output rows.  Every thread issues exactly NST stores per tile, so the
    // wait for the next tile's first stage can count them.
    constexpr int OCPR = BN * ES / 16;
    constexpr int PASS_CHUNKS = WM * OCPR;
    static_assert(PASS_CHUNKS % (64 * WGM * WGN) == 0 && WM * BN * ES <= STAGE_BYTES, "epilogue passes");
    constexpr int NST = WGM * PASS_CHUNKS / (64 * WGM * WGN);
    static_assert(NST < 64, "stores counted by vmcnt");
    auto store_tile = [&](const Tile &T, int buf) {
        typedef int i32x4v __attribute__((ext_vector_type(4)));
        // An opaque zero keeps the tile-independent LDS and store offsets
        // below from being hoisted out of the tile loop (where they would
        // stay live in registers across the whole K loop).
        int oz;
        asm volatile("s_mov_b32 %0, 0" : "=s"(oz));
        char *tile = lds + buf * STAGE_BYTES + oz;
        const S *Yt = (const S *)a.Y + ((int64_t)T.b * M + T.m0) * a.ldy + T.n0;
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void *)Yt, (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int pass = 0; pass < WGM; ++pass) {
            if (pass > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (wr == pass) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int rl = i * 32 + (lane & 31);
                    char *trow = tile + rl * (BN * ES);
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int cl = wc * WN + j * 32 + 8 * q + 4 * (lane >> 5);
                            const int ch = (cl / VE) ^ (rl & (OCPR - 1));
                            const f32x16 &v = acc[i][j];
                            *(uint2 *)(trow + ch * 16 + (cl % VE) * ES) =
                                make_uint2(E::pack2(v[4 * q], v[4 * q + 1]), E::pack2(v[4 * q + 2], v[4 * q + 3]));
                        }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int it = 0; it < PASS_CHUNKS / (64 * WGM * WGN); ++it) {
                const int idx = it * 64 * WGM * WGN + tid;
                const int rl = idx / OCPR, c = idx % OCPR;
                const uint4 v = *(const uint4 *)(tile + rl * (BN * ES) + (c ^ (rl & (OCPR - 1))) * 16);
                const int row = pass * WM + rl;
                const uint32_t voff = (uint32_t)(((int64_t)row * a.ldy + c * VE) * ES) + (uint32_t)oz;
                // aux 2: non-temporal
                __builtin_amdgcn_raw_buffer_store_b128(i32x4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ry, (int)voff, 0, 2);
            }
        }
    };

    Tile cur = tile_at(0);
    Tile nxt = cur;
    issue(cur, 0, 0);
    const int total_gs = ntiles * nk;
    int st = 0;
    int j = 0;
    bool stored = false;  // the previous step ended a tile (its NST stores follow this step's loads)
    for (int gs = 0; gs < total_gs; ++gs) {
        // This wave's loads of stage gs are complete once at most the stores
        // issued after them are outstanding.
        if (stored) wait_vmcnt<NST>();
        else wait_vmcnt<0>();
        stored = false;
        // After the barrier every wave's loads of stage gs have landed and
        // every wave has finished reading the other buffer, refilled next.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int buf = gs & 1;
        if (gs + 1 < total_gs) {
            if (st + 1 < nk) {
                issue(cur, st + 1, buf ^ 1);
            } else {
                nxt = tile_at(j + 1);
                issue(nxt, 0, buf ^ 1);
            }
        }
        constexpr int RPS = FM + FN * 2;  // LDS reads per step
        constexpr int MPS = FM * FN;      // MFMAs per step
        read_frags(buf, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) read_frags(buf, ks + 1, (ks + 1) & 1);
            mfmas(ks & 1);
            if (ks + 1 < KS) {
#pragma unroll
                for (int q = 0; q < RPS / 2; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
                if constexpr (MPS > RPS / 2) __builtin_amdgcn_sched_group_barrier(0x008, MPS - RPS / 2, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, MPS, 0);
            }
        }
        if (st + 1 < nk) {
            ++st;
            continue;
        }
        // Every wave has finished reading this stage's buffer before the
        // epilogue reuses it.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        store_tile(cur, buf);
        stored = true;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
        st = 0;
        ++j;
        cur = nxt;
    }
#endif
}

template <int DT, int BM, int BN, int WGM, int WGN, int BKB, int STAGES, int PW, int KG, bool TA = false, bool TB = false,
          bool GEMM = false, bool PERS = false>
static hipError_t launch_tile(bool vec, bool split, const KArgs &a, hipStream_t s) {
    const int64_t tiles = a.batch * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * (split ? a.split : 1);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 g((unsigned)tiles);
    // Buffer offsets are 32-bit: one tile's rows of A and one stage's rows of
    // B must each span less than 2 GiB.
    constexpr int ES = (int)sizeof(typename Elem<DT>::S);
    const int64_t a_span = TA ? (int64_t)(BKB / ES) * a.lda : (int64_t)BM * a.lda;  // stored rows one tile stage spans
    const int64_t b_span = TB ? (int64_t)BN * a.ldb : (int64_t)(BKB / ES) * a.ldb;
    const bool fits = a_span * ES < 0x7fff0000LL && b_span * ES < 0x7fff0000LL;
    if constexpr (DT == MM_INT8) {
        // INT8 runs only this kernel (split-K on the 128 x 128 entry); the
        // plan and execute layer send other cases to the direct integer kernel.
        if (!(vec && fits)) return hipErrorInvalidValue;
        const dim3 blk(64 * WGM * WGN * KG);
        if (split) {
            if constexpr (BM * BN <= 128 * 128) {
                switch ((a.flip_a ? 1 : 0) | (a.flip_b ? 2 : 0)) {
                case 0: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, true, TA, TB, false, 0>), g, blk, 0, s, a); break;
                case 1: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, true, TA, TB, false, 1>), g, blk, 0, s, a); break;
                case 2: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, true, TA, TB, false, 2>), g, blk, 0, s, a); break;
                default: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, true, TA, TB, false, 3>), g, blk, 0, s, a); break;
                }
                return hipGetLastError();
            } else {
                return hipErrorInvalidValue;
            }
        }
        switch ((a.flip_a ? 1 : 0) | (a.flip_b ? 2 : 0)) {
        case 0: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, false, TA, TB, false, 0>), g, blk, 0, s, a); break;
        case 1: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, false, TA, TB, false, 1>), g, blk, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, false, TA, TB, false, 2>), g, blk, 0, s, a); break;
        default: hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, false, TA, TB, false, 3>), g, blk, 0, s, a); break;
        }
        return hipGetLastError();
    } else if (vec && fits) {
        const dim3 blk(64 * WGM * WGN * KG);
        constexpr bool kPackable = sizeof(typename Elem<DT>::S) == 2 && !TA && !TB && !GEMM;
        constexpr bool kPersist = PERS && sizeof(typename Elem<DT>::S) == 2 && !TA && !TB && !GEMM && STAGES == 2 && KG == 1;
        if constexpr (kPersist) {
            // Whole tiles and stages, 32-bit tile origins, output rows of
            // whole 16-byte chunks inside one buffer range.
            const bool whole = a.M % BM == 0 && a.N % BN == 0 && a.K % (BKB / 2) == 0;
            const bool small = a.M < 0x7fff0000LL && a.N < 0x7fff0000LL;
            if (!split && !a.b_packed && a.y_vec && whole && small && (int64_t)BM * a.ldy * 2 < 0x7fff0000LL) {
                constexpr int64_t kWgsPerCu = (160 * 1024) / (STAGES * (BM + BN) * BKB);
                const int64_t grid = tiles < kNumCUs * kWgsPerCu ? tiles : kNumCUs * kWgsPerCu;
                hipLaunchKernelGGL((k_gemm_persist<DT, BM, BN, WGM, WGN, BKB, PW>), dim3((unsigned)grid), blk, 0, s, a);
                return hipGetLastError();
            }
        }
        // Split-K partials take no epilogue (the reduction applies it).
        if (split) hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, true, TA, TB, false>), g, blk, 0, s, a);
        else if (kPackable && a.b_packed)
            hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, false, TA, TB, false, 0, kPackable>),
                               g, blk, 0, s, a);
        else hipLaunchKernelGGL((k_gemm_lds_dma<DT, BM, BN, WGM, WGN, BKB, STAGES, PW, KG, false, TA, TB, GEMM>), g, blk, 0, s, a);
    } else {
        // The register-staged kernel needs at least 64 x 64 (2 x 2 waves of
        // 32 x 32): narrower entries fall back to 64-wide tiles on their own grid.
        constexpr int GM = BM < 64 ? 64 : BM, GN = BN < 64 ? 64 : BN;
        const int64_t gt = a.batch * ((a.M + GM - 1) / GM) * ((a.N + GN - 1) / GN) * (split ? a.split : 1);
        if (gt > 0x7fffffff) return hipErrorInvalidValue;
        const dim3 gg((unsigned)gt), blk(256);
        // The register-staged kernel reads transposed operands element-wise.
        if (vec && !TA && !TB) {
            if (split) hipLaunchKernelGGL((k_gemm_generic<DT, GM, GN, true, true>), gg, blk, 0, s, a);
            else hipLaunchKernelGGL((k_gemm_generic<DT, GM, GN, true, false>), gg, blk, 0, s, a);
        } else {
            if (split) hipLaunchKernelGGL((k_gemm_generic<DT, GM, GN, false, true>), gg, blk, 0, s, a);
            else hipLaunchKernelGGL((k_gemm_generic<DT, GM, GN, false, false>), gg, blk, 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace mm
