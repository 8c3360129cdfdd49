// plan.cpp -- host-side MatMul plan: shape resolution, broadcast strides,
// batch collapsing/folding and algorithm selection.  The only GPU calls are
// the device query and allocation of a split plan's workspace, and a host
// without a GPU skips them, so the whole layer is testable there.
//
// Page "MatMul Kernel Design", section "Shape and plan model": the plan
// resolves the complete output shape before execution (rank-one promotion and
// squeeze, multidirectional batch broadcasting, precomputed batch strides
// with zeros for broadcast dimensions, empty outputs that read nothing).
// Page "Gemm and MatMul Performance Roadmap", section "Phase 4: complete
// MatMul": collapse contiguous batch dimensions, dispatch independent batches
// together, dedicated kernels for M == 1 / N == 1.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>

#include "internal.h"
#include "plan.h"
#include "tiles.h"

namespace mm {

static thread_local std::string g_last_error;

mm_status fail(mm_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

void clear_error() { g_last_error.clear(); }

int tile_count(int dtype) {
    if (dtype == MM_FLOAT) return kNumTiles32;
    if (dtype == MM_FLOAT16 || dtype == MM_BFLOAT16) return kNumTiles16;
    if (dtype == MM_DOUBLE) return kNumTiles64;
    if (dtype == MM_INT8 || dtype == MM_UINT8 || dtype == MM_INT32) return kNumTiles8;
    return 0;
}

const TileCfg *tile_entry(int dtype, int index) {
    if (index < 0 || index >= tile_count(dtype)) return nullptr;
    if (dtype == MM_DOUBLE) return &kTiles64[index];
    if (dtype == MM_INT8 || dtype == MM_UINT8 || dtype == MM_INT32) return &kTiles8[index];
    return dtype == MM_FLOAT ? &kTiles32[index] : &kTiles16[index];
}

int elem_size(int dtype) {
    if (dtype == MM_INT8 || dtype == MM_UINT8) return 1;
    return dtype == MM_DOUBLE ? 8 : (dtype == MM_FLOAT || dtype == MM_INT32) ? 4 : 2;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Relative per-CU throughput of a tile entry (bigger tiles reuse each LDS
// byte more often); used only to rank entries against each other.
static double tile_quality(int dtype, int index) {
    static const double q16[kNumTiles16] = {1.0, 0.85, 0.7, 0.55, 0.4, 0.9, 0.8, 0.8, 0.35, 0.5, 0.0, 0.0, 0.0, 0.0};
    static const double q32[kNumTiles32] = {0.95, 1.0, 0.8, 1.0, 1.1, 0.85, 1.15, 0.0};
    static const double q64[kNumTiles64] = {1.0, 0.8, 0.0};
    static const double q8[kNumTiles8] = {1.0, 0.75, 1.0, 0.0, 0.0};
    if (dtype == MM_DOUBLE) return q64[index];
    if (dtype == MM_INT32) return q8[index];
    return dtype == MM_FLOAT ? q32[index] : q16[index];
}

// Estimated useful fraction of the machine for a tile entry: wave
// quantization over the CUs, tile padding at the edges, and tile quality.
static double tile_score(int dtype, int index, int64_t batch, int64_t M, int64_t N) {
    const TileCfg *t = tile_entry(dtype, index);
    int64_t tm = cdiv(M, t->bm), tn = cdiv(N, t->bn);
    double tiles = (double)batch * (double)tm * (double)tn;
    double waves = ceil(tiles / kNumCUs);
    double occ = tiles / (waves * kNumCUs);
    double pad = ((double)M * (double)N) / ((double)(tm * t->bm) * (double)(tn * t->bn));
    return occ * pad * tile_quality(dtype, index);
}

// Tile entries a plan may use: every entry, except that Gemm plans have
// kernels only for the kTransTiles subset.
static bool tile_allowed(int dtype, int index, bool gemm) {
    if (!gemm) return true;
    if (dtype == MM_FLOAT) {
        for (int t : kTransTiles32)
            if (t == index) return true;
    } else {
        for (int t : kTransTiles16)
            if (t == index) return true;
    }
    return false;
}

// 16-bit entries for products of at most 64 rows (see choose_tile).  The
// last three entries of the table serve such products only: the selector
// takes them by the rules below, never by ranking or time estimate.
constexpr int kT16Small2 = 8, kT16Small = 4, kT16Row32 = 11, kT16Row32Wide = 12, kT16Row64 = 13;
static_assert(kTiles16[kT16Small2].bm == 64 && kTiles16[kT16Small2].bn == 64 && kTiles16[kT16Small2].kgroups == 2,
              "64 x 64 entry with two K groups");
static_assert(kTiles16[kT16Small].bm == 64 && kTiles16[kT16Small].bn == 64 && kTiles16[kT16Small].kgroups == 1,
              "64 x 64 entry with one K group");
static_assert(kTiles16[kT16Row32].bm == 32 && kTiles16[kT16Row32].bn == 128 && kTiles16[kT16Row32Wide].bm == 32 &&
                  kTiles16[kT16Row32Wide].bn == 256 && kTiles16[kT16Row64].bm == 64 && kTiles16[kT16Row64].bn == 128 &&
                  kNumTiles16 == kT16Row64 + 1 && kT16Row32Wide == kT16Row32 + 1 && kT16Row64 == kT16Row32 + 2,
              "the small-row entries close the 16-bit table");
static_assert(kTransTiles16[2] == kT16Small, "the 64 x 64 entry has a Gemm kernel");

constexpr int kT32Row32 = 7;  // FLOAT 32 x 128, two K groups (see float_small_rows)
constexpr int kT8Row64 = 3;    // INT8 64 x 128, three stages (MatMulInteger over at most 64 rows)
constexpr int kT8Deep128 = 4;  // INT8 128 x 128, three stages (split-K that fills the CUs exactly)
constexpr int kT64Row32 = 2;  // DOUBLE 32 x 128 (see double_small_rows)
static_assert(kTiles64[kT64Row32].bm == 32 && kTiles64[kT64Row32].bn == 128 && kNumTiles64 == kT64Row32 + 1,
              "the DOUBLE small-row entry closes its table");
static_assert(kTiles8[kT8Row64].bm == 64 && kTiles8[kT8Row64].bn == 128 && kTiles8[kT8Row64].stages == 3 &&
                  kTiles8[kT8Deep128].bm == 128 && kTiles8[kT8Deep128].bn == 128 &&
                  kTiles8[kT8Deep128].stages == 3 && kNumTiles8 == kT8Deep128 + 1,
              "the INT8 split entries close their table");
static_assert(kTiles32[kT32Row32].bm == 32 && kTiles32[kT32Row32].bn == 128 && kTiles32[kT32Row32].kgroups == 2 &&
                  kNumTiles32 == kT32Row32 + 1,
              "the FLOAT small-row entry closes its table");

static bool small_m_entry(int dtype, int index) {
    return ((dtype == MM_FLOAT16 || dtype == MM_BFLOAT16) && index >= kT16Row32) ||
           (dtype == MM_FLOAT && index == kT32Row32) ||
           ((dtype == MM_INT8 || dtype == MM_UINT8 || dtype == MM_INT32) && index >= kT8Row64) ||
           (dtype == MM_DOUBLE && index == kT64Row32);
}

static int choose_tile(int dtype, int64_t batch, int64_t M, int64_t N, bool gemm = false) {
    // MatMulInteger over at most 64 rows, up to one 128-column tile per CU:
    // the three-stage 64 x 128 INT8 entry, 37-41 % faster than the two-stage
    // 128 x 128 one the ranking picks (UINT8 x INT8, M = 1..64, N = 28672,
    // K = 4096 and 8192: [16,8192]x[8192,28672] 85.6 -> 51.7 us).  Past
    // one round (N = 65536) the 128 x 128 entry stays ahead.
    if (dtype == MM_INT32 && M <= 64 && batch * cdiv(N, kTiles8[kT8Row64].bn) <= kNumCUs) return kT8Row64;
    if ((dtype == MM_FLOAT16 || dtype == MM_BFLOAT16) && M <= 64) {
        // At most 64 rows: each tile is a K-long chain of B stages, not MFMA
        // work, so the quality ranking above does not apply.  Measured for
        // M = 1..64, K = 4096: up to one 64 x 64 tile per CU, the entry
        // with two K groups (shorter chain) wins.  Beyond that, tiles one
        // row tile high and 128 columns wide (32 rows for M <= 32, else 64)
        // stream B 6-27 % faster than the 64 x 64 and 128 x 64 tiles
        // (BF16, M = 16..64, K = 2048..8192, N = 20480..128256); for
        // M <= 32, 256-column tiles (one per CU) gain another 4-15 % when
        // every round fills at least three quarters of the CUs (N = 49152,
        // 65536, 128256), and lose up to 45 % when a round is less full.
        // Gemm has the single-group 64 x 64 entry only.
        const int64_t t64 = batch * cdiv(N, 64);
        if (gemm) return kT16Small;
        if (t64 <= kNumCUs) return kT16Small2;
        if (M > 32) return kT16Row64;
        const int64_t t256 = batch * cdiv(N, 256), last = t256 % kNumCUs;
        if (t256 >= 3 * kNumCUs / 4 && (last == 0 || last >= 3 * kNumCUs / 4)) return kT16Row32Wide;
        return kT16Row32;
    }
    int best = -1;
    double best_s = -1.0;
    for (int i = 0; i < tile_count(dtype); ++i) {
        if (!tile_allowed(dtype, i, gemm) || small_m_entry(dtype, i)) continue;
        double s = tile_score(dtype, i, batch, M, N);
        if (s > best_s + 1e-9) {
            best_s = s;
            best = i;
        }
    }
    return best;
}

// LDS bytes of a tile entry's stage buffers, and the workgroups of that
// entry one CU holds (160 KB of LDS per CU).
static int64_t tile_lds_bytes(const TileCfg *t) { return (int64_t)t->stages * t->bkb * (t->bm + t->bn); }
static int64_t tile_wgs_per_cu(const TileCfg *t) { return std::max<int64_t>(1, (160 * 1024) / tile_lds_bytes(t)); }

static int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        const int64_t r = a % b;
        a = b;
        b = r;
    }
    return a;
}

// Time model of the tile entries of FLOAT16 / BFLOAT16 and of FLOAT, each
// fitted (least squares on log time) to forced-tile timings on one MI355X:
// every entry on 48 BF16 products (M 256-8192, K and N 1024-14336) and on
// 35 FP32 products (M 256-4096, K and N 1024-11008).  A launch costs
// launch_us; each round of workgroups then costs, per 4096 of K, the
// entry's round time at the occupancy of its busiest CU (1 up to the
// workgroups one CU holds); a last round of at most one workgroup per CU is
// cheaper in proportion to the idle CUs (slope).  Root-mean-square error
// 7 % (16-bit) and 2 % (FP32); the model ranks entries, its absolute values
// belong to that GPU.  The quality ranking above mispriced the 16-bit
// 128 x 128 entries against the 256 x 256 one by up to 30 % (e.g.
// [2048,4096]x[4096,14336]: 272 against 210 us).
struct RoundCost {
    double us[3];  // round time at occupancy 1, 2, 3 (levels past the entry's limit unused)
};
constexpr RoundCost kRound16[] = {
    {{98.6, 0.0, 0.0}},   // 256 x 256, 2 stages (one workgroup per CU)
    {{71.3, 0.0, 0.0}},   // 256 x 128, 3 stages
    {{43.0, 0.0, 0.0}},   // 128 x 128, 3 stages
    {{30.3, 49.7, 0.0}},  // 128 x 64, 3 stages (two per CU)
    {{23.3, 36.5, 43.4}}, // 64 x 64, 3 stages (three per CU)
    {{56.0, 68.8, 0.0}},  // 128 x 128, 2 stages (two per CU)
    {{74.6, 0.0, 0.0}},   // 128 x 256, 2 stages
    {{74.4, 0.0, 0.0}},   // 256 x 128 (4 x 2 waves), 2 stages
    {{23.3, 37.2, 43.4}}, // 64 x 64, two K groups
    {{56.5, 69.2, 0.0}},  // 128 x 128, two K groups
    {{0.0, 0.0, 0.0}},    // persistent twin of entry 0: chosen by plan_persistent only
    {{0.0, 0.0, 0.0}},    // 32 x 128, 32 x 256, 64 x 128: products of at most 64 rows,
    {{0.0, 0.0, 0.0}},    // chosen by choose_tile and choose_split_tile
    {{0.0, 0.0, 0.0}},
};
constexpr RoundCost kRound32[] = {
    {{272.8, 0.0, 0.0}},    // 128 x 128, 3 stages (one workgroup per CU)
    {{153.2, 260.6, 0.0}},  // 128 x 64, 3 stages (two per CU)
    {{85.8, 150.9, 198.8}}, // 64 x 64, 3 stages (three per CU)
    {{485.1, 0.0, 0.0}},    // 256 x 128, 3 stages
    {{279.0, 495.5, 0.0}},  // 128 x 128, 2 stages (two per CU)
    {{83.3, 155.9, 198.6}}, // 64 x 64, two K groups
    {{254.8, 480.8, 0.0}},  // 128 x 128, two K groups
    {{0.0, 0.0, 0.0}},      // 32 x 128, two K groups: at most 32 rows, chosen by float_small_rows
};
static_assert(sizeof(kRound16) / sizeof(kRound16[0]) == kNumTiles16, "one round cost per 16-bit entry");
static_assert(sizeof(kRound32) / sizeof(kRound32[0]) == kNumTiles32, "one round cost per FLOAT entry");
struct TimeModel {
    const RoundCost *round;
    double launch_us, slope;
};
constexpr TimeModel kModel16 = {kRound16, 6.4, 0.12}, kModel32 = {kRound32, 6.7, 0.054};

static double est_us(int dtype, int index, int64_t tiles, int64_t K) {
    const TimeModel &m = dtype == MM_FLOAT ? kModel32 : kModel16;
    const TileCfg *t = tile_entry(dtype, index);
    const int64_t w = std::min<int64_t>(tile_wgs_per_cu(t), 3);
    const RoundCost &c = m.round[index];
    const int64_t slots = kNumCUs * w;
    const int64_t full = tiles / slots, rem = tiles % slots;
    double us = (double)full * c.us[w - 1];
    if (rem > 0) {
        const int64_t o = cdiv(rem, kNumCUs);
        double r = c.us[o - 1];
        if (o == 1) r *= 1.0 - m.slope + m.slope * (double)rem / kNumCUs;
        us += r;
    }
    return m.launch_us + us * (double)K / 4096.0;
}

// The entry of least estimated time for a rectangle (FLOAT16, BFLOAT16 or
// FLOAT; persistent entries are left to plan_persistent).
static int choose_tile_timed(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K, bool gemm) {
    int best = -1;
    double best_us = 0.0;
    for (int i = 0; i < tile_count(dtype); ++i) {
        const TileCfg *t = tile_entry(dtype, i);
        if (!tile_allowed(dtype, i, gemm) || t->persistent || small_m_entry(dtype, i)) continue;
        const double us = est_us(dtype, i, batch * cdiv(M, t->bm) * cdiv(N, t->bn), K);
        if (best < 0 || us < best_us * (1.0 - 1e-9)) {
            best = i;
            best_us = us;
        }
    }
    return best;
}

// The general path's entry: the time model for FLOAT and for 16-bit
// products of more than 64 rows (smaller ones keep choose_tile's measured
// rule), the quality ranking for DOUBLE and INT8.
static int choose_general_tile(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K, bool gemm) {
    if (dtype == MM_FLOAT || ((dtype == MM_FLOAT16 || dtype == MM_BFLOAT16) && M > 64))
        return choose_tile_timed(dtype, batch, M, N, K, gemm);
    return choose_tile(dtype, batch, M, N, gemm);
}

constexpr int kT16Large = 0, kT16Persist = 10;  // the 256 x 256 entry and its persistent twin
// Split-K on the 256 x 256 entry for a 16-bit product the general path
// would run in at most half a round of that entry with a long K: the K
// chunks fill one round, and the FP32 partials they write and the reduction
// reads cost about kSplitUsPerMB per MB of partials (measured on 18 BF16
// products of 2-8 M outputs and K 4096-14336: about 35 us for 67 MB).
// Returns the split count, or 0 when the estimate does not gain 5 % over
// the general plan's.  E.g. [2048,14336]x[14336,4096]: general 256 us,
// two chunks of 256 x 256 tiles 218 us; [2048,4096]x[4096,4096]: general
// 77 us, split 90 us.
constexpr double kSplitUsPerMB = 0.55;
static int large_tile_split16(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K, bool gemm) {
    if (!(dtype == MM_FLOAT16 || dtype == MM_BFLOAT16) || M <= 64 || !tile_allowed(dtype, kT16Large, gemm)) return 0;
    // Measured gains start at K = 8192; below it the estimate can pick a
    // split that loses ([1296,6464]x[6464,4480]: 105 against 93.5 us).
    if (K < 8192) return 0;
    const TileCfg *t0 = tile_entry(dtype, kT16Large);
    const int64_t n0 = batch * cdiv(M, t0->bm) * cdiv(N, t0->bn);
    if (n0 > kNumCUs / 2) return 0;
    const int64_t s = std::min<int64_t>(kNumCUs / n0, K / 1024);
    if (s < 2) return 0;
    const int gt = choose_general_tile(dtype, batch, M, N, K, gemm);
    const TileCfg *g = tile_entry(dtype, gt);
    const double t_gen = est_us(dtype, gt, batch * cdiv(M, g->bm) * cdiv(N, g->bn), K);
    const double part_mb = (double)s * batch * M * N * 4.0 / 1e6;
    const double t_split = est_us(dtype, kT16Large, n0 * s, cdiv(K, s)) + kSplitUsPerMB * part_mb;
    return t_split < 0.95 * t_gen ? (int)s : 0;
}

// Gemm as a linear layer (B transposed: [N][K], each B row K-long) over at
// most 64 rows, 16-bit, A not transposed: split-K on the 64 x 128 entry in
// s chunks, s the largest power of two with at most two workgroups per CU,
// and at most K / 512 and 8, when those chunks give every CU at least one
// workgroup and the tiles are at most half a round (N <= 16384).  Read from
// B's [N][K] layout, each tile's B panel is 128-byte rows whatever its
// width, and its time follows the workgroups streaming B at once: measured
// on 39 BF16 products (M = 16..64, K = 1024..14336, N = 2048..65536),
// forced tiles and chunk counts, the rule is within 3.2 % of the best tried
// (geometric mean) where the plans before it were 9.3 % off: e.g.
// [16,4096]x[12288,4096]^T 33.9 -> 27.9 us, [64,14336]x[4096,14336]^T
// 36.8 -> 31.1 us, [16,8192]x[8192,8192]^T 38.8 -> 32.6 us; the largest
// loss, [64,4096]x[14336,4096]^T, 35.7 -> 36.6 us.  Returns the chunk
// count, or 0.
static int gemm_linear_split16(const mm_plan_s *p, int64_t M, int64_t N, int64_t K) {
    if (!p->is_gemm || !p->tb || p->ta || (p->dtype != MM_FLOAT16 && p->dtype != MM_BFLOAT16) || M > 64) return 0;
    const int64_t tiles = cdiv(N, kTiles16[kT16Row64].bn);
    if (tiles > kNumCUs / 2) return 0;
    int64_t s = 1;
    while (2 * s * tiles <= 2 * kNumCUs) s *= 2;
    s = std::min<int64_t>(s, std::min<int64_t>(K / 512, 8));
    if (s < 2 || tiles * s < kNumCUs) return 0;
    return (int)s;
}

// FP32 MatMul and Gemm over at most 32 rows (where skinny-M does not take
// a MatMul): the 32 x 128 entry with two K groups.  With 64-row tiles the
// FP32 matrix cores did twice or more the useful work; one 32-row tile per
// column block halves that and leaves B's stream as the bound.  Up to one tile per CU
// the plan splits K in s chunks, s the largest power of two (at least 2)
// with at most one workgroup per CU beyond the first two chunks, and at
// most K / 256; past one tile per CU it runs the tiles whole.  Measured on
// FP32 products of 16 and 32 rows (K 1024-11008, N 2048-28672), forced
// tiles and chunk counts: [16,4096]x[4096,11008] 76.5 -> 47.2 us,
// [16,8192]x[8192,8192] 86.4 -> 58.4 us, [32,11008]x[11008,4096] 62.5 ->
// 43.4 us, [16,4096]x[4096,28672] 147.7 -> 94.7 us.  Returns the chunk
// count (1: the general path on this entry), or 0 when the rule does not
// apply.
static int float_small_rows(const mm_plan_s *p, int64_t M, int64_t N, int64_t K) {
    if (p->dtype != MM_FLOAT || M > 32) return 0;
    const int64_t tiles = p->batch * cdiv(N, kTiles32[kT32Row32].bn);
    if (tiles > kNumCUs) return 1;
    int64_t s = 2;
    while (2 * s * tiles <= kNumCUs) s *= 2;
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, K / 256));
}

// DOUBLE over at most 32 rows (DOUBLE has no skinny kernels): the 32 x 128
// entry, which halves the FP64 matrix-core work that 64-row tiles pad in.
// Up to one tile per CU it splits K in s chunks, s the largest power of two
// (at least 2) with at most three workgroups per CU (the FP64 kernel's
// small LDS footprint holds several), at most K / 512 and at most 8; past
// one tile per CU it runs the tiles whole.  Forced tiles and chunk counts
// on 12 products (M = 1..32; K, N 4096-28672): [16,4096]x[4096,11008]
// 175.6 -> 81.0 us (8 chunks), [16,11008]x[11008,4096] 150.1 -> 91.8 us,
// [16,4096]x[4096,28672] 345 -> 204 us (2 chunks).  Returns the chunk
// count (1: the general path on this entry), or 0.
static int double_small_rows(const mm_plan_s *p, int64_t M, int64_t N, int64_t K) {
    if (p->dtype != MM_DOUBLE || M > 32) return 0;
    const int64_t tiles = p->batch * cdiv(N, kTiles64[kT64Row32].bn);
    if (tiles > kNumCUs) return 1;
    int64_t s = 2;
    while (2 * s * tiles <= 3 * kNumCUs) s *= 2;
    return (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(s, 8), K / 512));
}

// FP32 products of 33-512 rows: split-K when the time model says it pays.
// Each candidate is priced by est_us: the general path's timed tile run
// whole, or a two-K-group entry (64 x 64 or 128 x 128) in 2, 3 or a power
// of two up to 256 chunks of at least 256, plus kSplitUsPerMB per MB of
// FP32 partials and kReduceLaunchUs for the reduction's launch.  The
// cheapest is taken.  Without the launch cost the estimate took three
// chunks over [512,2048]x[2048,2048] for a 1 % gain (measured 48.4 against
// 44.3 us).  Measured on 24 FP32 products (M 64-512; K, N 1024-11008),
// forced tiles and chunk counts: the choice is within 1.4 % of the best
// tried (geometric mean), where the occupancy rules before it were 9.4 %
// off.  E.g. [128,4096]x[4096,11008] 176 -> 122 us (two chunks of 64 x 64
// tiles, not three chunks of 128 x 128 ones that put 258 workgroups on 256
// CUs), [256,2048]x[2048,2048] 44.2 -> 30.8 us, [512,11008]x[11008,4096]
// 396 -> 356 us.  Returns the chunk count (the entry in *tile), or 0 for
// the general path.
constexpr double kReduceLaunchUs = 3.0;
static int float_timed_split(const mm_plan_s *p, int64_t M, int64_t N, int64_t K, int *tile) {
    const int gt = choose_general_tile(MM_FLOAT, p->batch, M, N, K, p->is_gemm);
    const TileCfg *g = tile_entry(MM_FLOAT, gt);
    double best = est_us(MM_FLOAT, gt, p->batch * cdiv(M, g->bm) * cdiv(N, g->bn), K);
    int best_s = 0;
    const int bk = stage_k(MM_FLOAT);
    for (int i = 0; i < kNumTiles32; ++i) {
        const TileCfg *t = tile_entry(MM_FLOAT, i);
        if (t->kgroups != 2 || small_m_entry(MM_FLOAT, i) || !tile_allowed(MM_FLOAT, i, p->is_gemm)) continue;
        const int64_t tiles = p->batch * cdiv(M, t->bm) * cdiv(N, t->bn);
        for (int s : {2, 3, 4, 8, 16, 32, 64, 128, 256}) {
            if (K / s < 256) break;
            const int64_t kc = cdiv(cdiv(K, bk), s) * bk;
            const double part_mb = (double)s * p->batch * M * N * 4.0 / 1e6;
            const double us = est_us(MM_FLOAT, i, tiles * s, kc) + kSplitUsPerMB * part_mb + kReduceLaunchUs;
            if (us < best) {
                best = us;
                best_s = s;
                *tile = i;
            }
        }
    }
    return best_s;
}

// Last-round balancing for a large tile (one workgroup per CU).  When the
// tiles leave the last round of workgroups less than half full, the leading
// output columns are covered by whole rounds of the chosen tile and the
// remaining columns by a second launch with the tile that suits that
// narrower rectangle best -- if the estimate (in units of one chosen-tile
// duration, scaled by tile area and relative tile throughput) gains at
// least 3 %.  The roadmap page's participation sizing ("Parallel
// execution") makes the same trade between partition count and workers.
static void plan_tail(mm_plan_s *p) {
    p->tail_col = 0;
    p->tail_tile = -1;
    // The small-row entries span M in one row tile: choose_tile already
    // balanced their rounds.
    if (p->dtype == MM_DOUBLE || small_m_entry(p->dtype, p->tile)) return;
    const TileCfg *t = tile_entry(p->dtype, p->tile);
    if (tile_wgs_per_cu(t) != 1) return;
    const int64_t rows = p->batch * cdiv(p->kernel_m, t->bm);
    const int64_t tn = cdiv(p->N, t->bn);
    const int64_t T = rows * tn;
    const int64_t rem = T % kNumCUs;
    if (T <= kNumCUs || rem == 0 || rem > kNumCUs / 2) return;
    const int64_t step = kNumCUs / gcd64(rows % kNumCUs == 0 ? kNumCUs : rows % kNumCUs, kNumCUs);
    const int64_t c_main = ((tn - 1) / step) * step;  // whole rounds, at least one column left over
    if (c_main <= 0) return;
    const int64_t n_rem = p->N - c_main * t->bn;
    const int rt = choose_general_tile(p->dtype, p->batch, p->kernel_m, n_rem, p->K, p->is_gemm);
    const TileCfg *r = tile_entry(p->dtype, rt);
    const int64_t T_rem = p->batch * cdiv(p->kernel_m, r->bm) * cdiv(n_rem, r->bn);
    const double without = (double)cdiv(T, kNumCUs);
    const double with_split = (double)(rows * c_main) / kNumCUs +
                              (double)cdiv(T_rem, kNumCUs * tile_wgs_per_cu(r)) * ((double)r->bm * r->bn) /
                                  ((double)t->bm * t->bn) * tile_quality(p->dtype, p->tile) /
                                  tile_quality(p->dtype, rt);
    if (with_split < 0.97 * without) {
        p->tail_col = c_main * t->bn;
        p->tail_tile = rt;
    }
}

// The persistent twin of the 256 x 256 entry: one workgroup per CU walks
// its tiles with the stage pipeline running on across tile boundaries, so
// a tile's first loads overlap the previous tile's last stage and its
// output stores drain under the next tile's MFMAs.  Measured against the
// one-tile-per-workgroup kernel (BF16, same bits): K = 128 with 32 rounds
// of tiles 18 % faster, K = 256 8 %, K = 512 5 %, K = 1024 4 %, K = 2048
// even, K = 4096 5 % slower -- so short K with at least two rounds.  The
// kernel takes whole tiles and stages only.
static_assert(kTiles16[kT16Persist].persistent == 1 && kTiles16[kT16Large].persistent == 0 &&
                  kTiles16[kT16Persist].bm == kTiles16[kT16Large].bm && kTiles16[kT16Persist].bn == kTiles16[kT16Large].bn &&
                  kTiles16[kT16Persist].bkb == kTiles16[kT16Large].bkb,
              "persistent twin of the 256 x 256 entry");
static void plan_persistent(mm_plan_s *p) {
    if ((p->dtype != MM_FLOAT16 && p->dtype != MM_BFLOAT16) || p->is_gemm || p->tile != kT16Large || p->tail_col > 0)
        return;
    const TileCfg *t = tile_entry(p->dtype, p->tile);
    const int64_t bk = t->bkb / 2;
    if (p->kernel_m % t->bm != 0 || p->N % t->bn != 0 || p->K % bk != 0 || p->K > 1024) return;
    const int64_t tiles = p->batch * (p->kernel_m / t->bm) * (p->N / t->bn);
    if (tiles >= 2 * kNumCUs) p->tile = kT16Persist;
}

// Tile for split-K (its output is small by construction): the smallest
// edge padding, and among equally padded tiles the one of higher relative
// throughput.  Tiles above 128 x 128 are left out: with so few of them the
// plan would need many short K chunks, whose FP32 partials (split x M x N x
// 4 bytes) can outweigh the inputs.  FLOAT uses its two-K-group entries,
// and weighs the padding by the share of the CUs the split
// fills: plan_split aims at one workgroup per
// CU with at least 256 K elements per chunk, so a large tile over a small
// output can leave most CUs idle (e.g. [128,2048]x[2048,2048]: 128 x 128
// tiles in 8 chunks fill 128 CUs, 29.7 us; 64 x 64 tiles in 4 chunks fill
// 256, 20.2 us).
static int choose_split_tile(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K, bool gemm = false) {
    if ((dtype == MM_FLOAT16 || dtype == MM_BFLOAT16) && M <= 64 && !gemm) {
        // At most 64 rows: the 64 x 64 tiles in cdiv(CUs, tiles) chunks,
        // unless those chunks overfill the CUs or stay K-long (>= 3072);
        // then the 128-column tiles one row tile high, whose chunks
        // plan_split keeps to one workgroup per CU.  Measured on 28 BF16
        // products (M = 16..64, K = 1024..14336, N = 2048..11008): within
        // 0.9 % of the best tile and chunk count tried (geometric mean),
        // against 6.9 % for the 64 x 64 tiles alone; e.g.
        // [64,4096]x[4096,11008] 33.4 -> 27.6 us, [16,14336]x[14336,4096]
        // 32.0 -> 29.1 us.
        const int64_t t64 = batch * cdiv(N, 64);
        const int64_t s64 = std::min<int64_t>(cdiv(kNumCUs, t64), std::max<int64_t>(1, K / 256));
        if (t64 * s64 > kNumCUs || K / s64 >= 3072) return M <= 32 ? kT16Row32 : kT16Row64;
    }
    // MatMulInteger over at most 64 rows: the three-stage 64 x 128 entry.
    // Its short K chunks (a few 128-byte stages each) run 5-25 % faster
    // than on the two-stage 128 x 128 entry (UINT8 x INT8, M = 1..64, K
    // 4096-11008): [16,8192]x[8192,8192] 31.7 -> 23.9 us, [16,4096]x
    // [4096,11008] 23.6 -> 20.2 us.
    if (dtype == MM_INT32 && M <= 64) return kT8Row64;
    // More rows: the three-stage 128 x 128 entry (one workgroup per CU)
    // when the rounded-up chunk count fills the CUs exactly (the tile count
    // divides them): 16-22 % faster than the two-stage entry on the K-long
    // products of 96-256 rows measured (e.g. [128,8192]x[8192,8192] 42.4
    // -> 33.8 us).  Otherwise a 257th workgroup would start a second round
    // on one CU, and the two-stage entry (two per CU) stays ([128,4096]x
    // [4096,11008], 86 tiles: 40.8 us or more on three-stage chunks,
    // against 32.1 us).
    if (dtype == MM_INT32) {
        const int64_t tiles = batch * cdiv(M, kTiles8[kT8Deep128].bm) * cdiv(N, kTiles8[kT8Deep128].bn);
        if (tiles <= kNumCUs && kNumCUs % tiles == 0) return kT8Deep128;
    }
    int best = -1;
    double best_s = -1.0;
    for (int i = 0; i < tile_count(dtype); ++i) {
        if (!tile_allowed(dtype, i, gemm) || small_m_entry(dtype, i)) continue;
        const TileCfg *t = tile_entry(dtype, i);
        if (t->bm * t->bn > 128 * 128) continue;
        // FLOAT: the two-K-group entries (the measured split tiles).
        if (dtype == MM_FLOAT && (t->kgroups != 2 || small_m_entry(dtype, i))) continue;
        double score = ((double)M * N) / ((double)cdiv(M, t->bm) * t->bm * (double)cdiv(N, t->bn) * t->bn);
        if (dtype == MM_FLOAT) {
            const int64_t tiles = batch * cdiv(M, t->bm) * cdiv(N, t->bn);
            const int64_t s = std::min<int64_t>(cdiv(kNumCUs, tiles), std::max<int64_t>(1, K / 256));
            score *= (double)std::min<int64_t>(kNumCUs, tiles * s) / kNumCUs;
        }
        const bool tie = best >= 0 && fabs(score - best_s) <= 1e-9;
        if (score > best_s + 1e-9 || (tie && tile_quality(dtype, i) > tile_quality(dtype, best))) {
            best_s = score;
            best = i;
        }
    }
    return best;
}

// Resolve shapes, strides, collapse and fold into `p`.
static mm_status resolve(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank,
                         mm_plan_s *p) {
    if (a_rank < 1 || b_rank < 1)
        return fail(MM_ERR_RANK, "input rank must be >= 1 (got A rank %d, B rank %d)", a_rank, b_rank);
    if (a_rank > MM_MAX_RANK || b_rank > MM_MAX_RANK)
        return fail(MM_ERR_RANK, "input rank must be <= %d (got A rank %d, B rank %d)", MM_MAX_RANK,
                    a_rank, b_rank);
    for (int i = 0; i < a_rank; ++i)
        if (a_shape[i] < 0) return fail(MM_ERR_NEG_DIM, "A dimension %d is negative (%lld)", i, (long long)a_shape[i]);
    for (int i = 0; i < b_rank; ++i)
        if (b_shape[i] < 0) return fail(MM_ERR_NEG_DIM, "B dimension %d is negative (%lld)", i, (long long)b_shape[i]);

    p->a_rank = a_rank;
    p->b_rank = b_rank;
    p->b_numel = 1;
    for (int i = 0; i < b_rank; ++i) p->b_numel *= b_shape[i];
    memcpy(p->a_shape, a_shape, sizeof(int64_t) * a_rank);
    memcpy(p->b_shape, b_shape, sizeof(int64_t) * b_rank);

    // Rank-one promotion: A [K] -> [1, K]; B [K] -> [K, 1].
    const bool a_vec = a_rank == 1, b_vec = b_rank == 1;
    const int64_t M = a_vec ? 1 : a_shape[a_rank - 2];
    const int64_t Ka = a_shape[a_rank - 1];
    const int64_t Kb = b_vec ? b_shape[0] : b_shape[b_rank - 2];
    const int64_t N = b_vec ? 1 : b_shape[b_rank - 1];
    if (Ka != Kb)
        return fail(MM_ERR_K_MISMATCH, "inner dimensions differ: A has K=%lld, B has K=%lld", (long long)Ka,
                    (long long)Kb);
    const int64_t K = Ka;
    const int abr = a_vec ? 0 : a_rank - 2;  // batch ranks
    const int bbr = b_vec ? 0 : b_rank - 2;
    const int r = std::max(abr, bbr);
    if (r > MM_MAX_BATCH_DIMS)
        return fail(MM_ERR_RANK, "at most %d batch dimensions are supported", MM_MAX_BATCH_DIMS);

    // Right-aligned broadcast of the batch dimensions, with dense row-major
    // strides (in elements) of each operand, zero where it broadcasts.
    int64_t da[MM_MAX_BATCH_DIMS], db[MM_MAX_BATCH_DIMS], dout[MM_MAX_BATCH_DIMS];
    for (int d = 0; d < r; ++d) {
        int ai = d - (r - abr), bi = d - (r - bbr);
        da[d] = ai >= 0 ? a_shape[ai] : 1;
        db[d] = bi >= 0 ? b_shape[bi] : 1;
        if (da[d] == db[d]) dout[d] = da[d];
        else if (da[d] == 1) dout[d] = db[d];
        else if (db[d] == 1) dout[d] = da[d];
        else
            return fail(MM_ERR_BROADCAST, "batch dimension %d cannot be broadcast: A has %lld, B has %lld", d,
                        (long long)da[d], (long long)db[d]);
    }
    int64_t sa[MM_MAX_BATCH_DIMS], sb[MM_MAX_BATCH_DIMS];
    {
        int64_t ma = M * K, mb = K * N;  // element stride of the innermost batch dim
        for (int d = r - 1; d >= 0; --d) {
            sa[d] = da[d] == 1 ? 0 : ma;
            sb[d] = db[d] == 1 ? 0 : mb;
            ma *= da[d];
            mb *= db[d];
        }
    }

    // Output shape: batch ++ [M unless A was rank one] ++ [N unless B was].
    p->out_rank = 0;
    int64_t batch = 1;
    for (int d = 0; d < r; ++d) {
        p->out_shape[p->out_rank++] = dout[d];
        batch *= dout[d];
    }
    if (!a_vec) p->out_shape[p->out_rank++] = M;
    if (!b_vec) p->out_shape[p->out_rank++] = N;
    p->M = M;
    p->N = N;
    p->K = K;
    p->out_numel = batch * M * N;
    p->total_batch = batch;

    // Collapse: drop size-1 dims, then merge neighbours whose strides stay
    // linear for both operands.
    BatchDesc bd;
    memset(&bd, 0, sizeof(bd));
    for (int d = 0; d < r; ++d) {
        if (dout[d] == 1) continue;
        if (bd.nb > 0) {
            int q = bd.nb - 1;
            // merging the new dim d into q: q's stride must equal stride_d * dim_d
            if (bd.sa[q] == sa[d] * dout[d] && bd.sb[q] == sb[d] * dout[d]) {
                bd.dim[q] *= dout[d];
                bd.sa[q] = sa[d];
                bd.sb[q] = sb[d];
                continue;
            }
        }
        bd.dim[bd.nb] = dout[d];
        bd.sa[bd.nb] = sa[d];
        bd.sb[bd.nb] = sb[d];
        bd.nb++;
    }
    // Fold: B shared by every batch (all its strides zero) and A dense over
    // the (single collapsed) batch dim -> one product with batch*M rows.
    p->folded = 0;
    p->kernel_m = M;
    p->batch = batch;
    if (bd.nb == 1 && bd.sb[0] == 0 && bd.sa[0] == M * K && batch > 1) {
        p->folded = 1;
        p->kernel_m = batch * M;
        p->batch = 1;
        bd.nb = 0;
    }
    if (batch == 0) bd.nb = 0;
    p->bd = bd;
    return MM_OK;
}

// Split count and chunk for SPLIT_K.
static void plan_split(mm_plan_s *p, int requested) {
    const int bk = stage_k(p->dtype);
    const TileCfg *t = tile_entry(p->dtype, p->tile);
    int64_t tiles = p->batch * cdiv(p->kernel_m, t->bm) * cdiv(p->N, t->bn);
    int64_t kblocks = cdiv(p->K, bk);
    int64_t s;
    if (requested > 0) {
        s = requested;
    } else {
        // Aim for about one workgroup per CU, with at least 256 K elements
        // per partition (the partials then stay small next to the inputs).
        int64_t want = cdiv((int64_t)kNumCUs, std::max<int64_t>(tiles, 1));
        // The 16-bit and FP32 entries for few rows: never more workgroups
        // than CUs (BF16 [48,4096]x[4096,11008] on 64 x 128 tiles: 2 chunks
        // 26.5 us, 3 chunks -- two workgroups on two CUs -- 32.1 us).  The
        // INT8 split entry keeps the rounded-up count (3 or 4 chunks of
        // [16,4096]x[4096,11008]: 20.2 and 20.0 us).
        if (small_m_entry(p->dtype, p->tile) && p->dtype != MM_INT32)
            want = std::max<int64_t>(1, kNumCUs / std::max<int64_t>(tiles, 1));
        // FP32 and DOUBLE: one partition fewer when that still fills three
        // quarters of the CUs and the rounded-up count would put a second
        // workgroup on a few of them (their long MFMA chains make that
        // second one a slow last round; measured on 70 shapes, 0.64-0.89 of
        // the time).  The 16-bit tiles gain nothing from it.
        const bool long_chains = p->dtype == MM_FLOAT || p->dtype == MM_DOUBLE;
        if (long_chains && want > 2 && tiles * want > kNumCUs && tiles * (want - 1) >= 3 * kNumCUs / 4) --want;
        int64_t max_s = std::max<int64_t>(1, p->K / 256);
        s = std::min(want, max_s);
    }
    s = std::max<int64_t>(1, std::min(s, kblocks));
    int64_t chunk_blocks = cdiv(kblocks, s);
    p->kchunk = chunk_blocks * bk;
    p->split = (int32_t)cdiv(p->K, p->kchunk);
    const int64_t part_bytes = p->dtype == MM_DOUBLE ? 8 : 4;  // partials: FP32, or double for DOUBLE
    p->workspace_bytes = (int64_t)p->split * p->batch * p->kernel_m * p->N * part_bytes;
}

// K chunks of the skinny-M kernel.  Its workgroups each cover 64 lanes x 16
// bytes of columns for one group of rows (the launcher's row groups: 1, 2,
// 4, 8 or 16 rows); when those are fewer than one per CU, K is cut into
// chunks of whole 64-row blocks so that the grid holds at most two
// workgroups per CU (a third on some CUs would make a slow last round),
// with at most kSkinnyMaxSplit chunks.  Measured over M = 1..8, K =
// 1024..16384 and 1..120 column workgroups, that count is within 5 %
// (geometric mean) of the best chunk count.  The FP32 partials (split x rows
// x N) stay small next to B, which holds K rows of N.
constexpr int64_t kSkinnyMaxSplit = 64;

static void plan_skinny_split(mm_plan_s *p, int requested) {
    const int64_t M = p->kernel_m, N = p->N, K = p->K;
    const int64_t mt = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    const int64_t wgs = p->batch * cdiv(M, mt) * cdiv(N, 64 * (16 / elem_size(p->dtype)));
    const int64_t kblocks = cdiv(K, 64);
    int64_t s;
    if (requested > 0) {
        s = requested;
    } else {
        s = wgs >= kNumCUs ? 1 : std::min(2 * (int64_t)kNumCUs / std::max<int64_t>(wgs, 1), kSkinnyMaxSplit);
    }
    s = std::max<int64_t>(1, std::min(s, kblocks));
    p->kchunk = cdiv(kblocks, s) * 64;
    p->split = (int32_t)cdiv(K, p->kchunk);
    p->workspace_bytes = p->split > 1 ? (int64_t)p->split * p->batch * M * N * 4 : 0;
}

static mm_status check_limits(const mm_plan_s *p) {
    const int64_t lim = INT32_MAX;
    if (p->kernel_m > lim || p->N > lim || p->K > lim || p->batch > lim)
        return fail(MM_ERR_TOO_LARGE, "M, N, K and batch must each be below 2^31");
    return MM_OK;
}

static mm_status select_algo(mm_plan_s *p, const mm_plan_options *opt) {
    const int64_t M = p->kernel_m, N = p->N, K = p->K;
    p->tile = -1;
    p->tail_col = 0;
    p->tail_tile = -1;
    p->split = 1;
    p->kchunk = K;
    p->workspace_bytes = 0;
    if (p->out_numel == 0) {
        p->algo = MM_ALGO_EMPTY;
        return MM_OK;
    }
    if (K == 0) {
        // MatMul: the empty sum.  Gemm: Y = beta * C (or alpha * 0), formed by
        // the direct kernel without reading A or B.
        p->algo = p->is_gemm ? MM_ALGO_DIRECT : MM_ALGO_ZERO_FILL;
        return MM_OK;
    }
    mm_status st = check_limits(p);
    if (st != MM_OK) return st;

    int algo = opt ? opt->force_algo : MM_ALGO_AUTO;
    int rule_split = 0, rule_tile = -1;  // a plan fixed by a rule below: split chunks (1: none) and tile
    if (algo == MM_ALGO_AUTO) {
        const double flops = 2.0 * (double)p->batch * M * N * K;
        // Tiles of the smallest block tile in the table: the most workgroups
        // the tiled kernel can put on the GPU (64-row tiles: the 32-row
        // entries serve at most 32 rows, where they count the same).
        int64_t small_tiles = 0;
        for (int i = 0; i < tile_count(p->dtype); ++i) {
            const TileCfg *t = tile_entry(p->dtype, i);
            if (t->bm < 64) continue;
            small_tiles = std::max(small_tiles, p->batch * cdiv(M, t->bm) * cdiv(N, t->bn));
        }
        // Workgroups of the skinny-M kernel (one per 64 lanes x 16 bytes of
        // columns per batch): with few of them the GEMV cannot fill the GPU.
        const int64_t skm_wgs = p->batch * cdiv(N, 64 * (16 / elem_size(p->dtype)));
        const bool has_skinny = p->dtype != MM_DOUBLE && !p->is_gemm && !p->is_int;
        // Direct-kernel limits (measured): for the 16-bit types the tiled
        // MFMA kernel wins from K = 64 on, and from about 2^18 outputs at
        // K = 16; for FP32 the direct kernel stays ahead of the FP32 tiles up
        // to K = 512 and about 2^25 FLOPs.
        const bool t16 = p->dtype == MM_FLOAT16 || p->dtype == MM_BFLOAT16;
        const double direct_flops = p->dtype == MM_FLOAT && !p->is_gemm ? 33554432.0 : 16777216.0;
        const int64_t direct_k = t16 ? (p->batch * M * N <= 262144 ? 32 : 0) : 512;
        // The 16-bit eight-column skinny-N kernel gives each of its 8 waves
        // 512 elements of K: below K = 1024 most waves idle and the tiles win.
        const bool skn_short = t16 && N == 8 && K < 1024;
        // Workgroups of the tile the general path would choose.
        auto general_tiles = [&]() -> int64_t {
            // FLOAT: the entry the general path would run; the 16-bit
            // thresholds below were measured with the quality ranking, and
            // for at most 64 rows with the 64-column tiles of that time.
            if (t16 && M <= 64) return p->batch * cdiv(N, 64);
            const int gt = p->dtype == MM_FLOAT ? choose_general_tile(p->dtype, p->batch, M, N, K, p->is_gemm)
                                                : choose_tile(p->dtype, p->batch, M, N, p->is_gemm);
            const TileCfg *t = tile_entry(p->dtype, gt);
            return p->batch * cdiv(M, t->bm) * cdiv(N, t->bn);
        };
        // Skinny-M with K cut over workgroups (measured against split-K and
        // the tiles for M = 1..15, K = 1024..16384, N = 256..30720): FP32
        // up to 8 rows wins everywhere (64-row tiles padded M to 64 rows of
        // FP32 MFMA work), by up to 3x.  It also won for 9-15 rows with
        // K >= 4096 and N >= 4096 until the 32-row FP32 entry: split on that
        // entry, 12 and 15 rows run 1.11-1.37x faster than skinny-M on 10
        // products (K, N 4096-28672), so float_small_rows takes them.  The
        // 16-bit types, whose tiles run at the 16-bit MFMA
        // rate, win for up to 4 rows with a long K and a large B (K >= 8192,
        // K * N >= 2^26), and for up to 8 rows with K >= 16384 and
        // N >= 8704 (packed dot products: 15-29 % faster than the tiles).
        // The 16-bit wins come from the packed-dot kernel, which needs rows
        // of A, B and Y in whole 16-byte chunks (K and N multiples of 8);
        // other 16-bit shapes keep the tiles or split-K.
        const bool rows16 = K % 8 == 0 && N % 8 == 0;
        const bool skm_split = has_skinny && K >= 1024 &&
                               ((p->dtype == MM_FLOAT && M <= 8) ||
                                (t16 && rows16 && M <= 4 && K >= 8192 && (double)K * N >= 67108864.0) ||
                                (t16 && rows16 && M <= 8 && K >= 16384 && N >= 8704));
        if (has_skinny && N < 16 && N <= M && K >= 64 && !skn_short) {
            algo = MM_ALGO_SKINNY_N;  // few columns: the rows of A stream in parallel, K split over waves
        } else if (flops <= direct_flops && K <= direct_k) {
            algo = MM_ALGO_DIRECT;  // tiny product with a short reduction: launch latency dominates
        } else if (has_skinny && N < 16 && N <= M && !skn_short) {
            algo = MM_ALGO_SKINNY_N;  // includes N == 1: never split-K
        } else if (has_skinny && M < 16 && skm_wgs >= kNumCUs / 2) {
            algo = MM_ALGO_SKINNY_M;  // GEMV over enough columns and batches to fill the GPU
        } else if (skm_split) {
            algo = MM_ALGO_SKINNY_M;  // GEMV over few columns: K cut into chunks
        } else if ((rule_split = float_small_rows(p, M, N, K)) > 0) {
            algo = rule_split > 1 ? MM_ALGO_SPLIT_K : MM_ALGO_GENERAL;  // FP32 over few rows: 32-row tiles
            rule_tile = kT32Row32;
        } else if ((rule_split = double_small_rows(p, M, N, K)) > 0) {
            algo = rule_split > 1 ? MM_ALGO_SPLIT_K : MM_ALGO_GENERAL;  // DOUBLE over few rows: 32-row tiles
            rule_tile = kT64Row32;
        } else if (p->dtype == MM_FLOAT && M > 32 && M <= 512) {
            // FP32 of 33-512 rows: split-K or general by the time model
            rule_split = float_timed_split(p, M, N, K, &rule_tile);
            algo = rule_split > 0 ? MM_ALGO_SPLIT_K : MM_ALGO_GENERAL;
        } else if ((rule_split = gemm_linear_split16(p, M, N, K)) > 0) {
            algo = MM_ALGO_SPLIT_K;  // a linear layer over few rows: B streamed by 64 x 128 chunks
            rule_tile = kT16Row64;
        } else if ((small_tiles < kNumCUs / 2 && K >= 1024) || (K >= 4096 && general_tiles() < 3 * kNumCUs / 4) ||
                   (t16 && !p->is_gemm && M <= 32 && K >= 4096 && general_tiles() <= kNumCUs)) {
            // Tiles cannot fill the GPU and K is long; with K >= 4096, also
            // when the tile the general path would take leaves a quarter of
            // the CUs idle (each of its tiles is then a chain of at least 64
            // stages, which outweighs the partials' round trip).  Also the
            // skinny shapes of DOUBLE and Gemm, which have no skinny kernels.
            // 16-bit MatMul of at
            // most 32 rows splits up to one 64-column tile per CU: two
            // chunks of 32 x 128 tiles stream B faster than one K-long
            // chain per 64 x 64 tile ([16,4096]x[4096,14336] BF16: 31.2
            // against 27.4 us; at 16384 columns 31.6 against 30.1 us).
            algo = MM_ALGO_SPLIT_K;
        } else if ((rule_split = large_tile_split16(p->dtype, p->batch, M, N, K, p->is_gemm)) > 0) {
            algo = MM_ALGO_SPLIT_K;  // a long K over at most half a round of large tiles
            rule_tile = kT16Large;
        } else {
            algo = MM_ALGO_GENERAL;
        }
        // MatMulInteger runs on the direct and tiled INT8 kernels; split-K
        // (INT32 partials) where the rules above split and the tiled kernel
        // can take the shape (K and N whole 16-byte chunks).
        if (p->is_int && algo != MM_ALGO_DIRECT)
            algo = algo == MM_ALGO_SPLIT_K && K % 16 == 0 && N % 16 == 0 ? MM_ALGO_SPLIT_K : MM_ALGO_GENERAL;
    }
    if (algo < MM_ALGO_DIRECT || algo > MM_ALGO_GENERAL)
        return fail(MM_ERR_BAD_OPTION, "force_algo %d is not a forcible algorithm", algo);
    if (p->dtype == MM_DOUBLE && (algo == MM_ALGO_SKINNY_M || algo == MM_ALGO_SKINNY_N))
        return fail(MM_ERR_BAD_OPTION, "DOUBLE has no skinny-M / skinny-N kernel (force GENERAL or DIRECT)");
    if (p->is_gemm && (algo == MM_ALGO_SKINNY_M || algo == MM_ALGO_SKINNY_N))
        return fail(MM_ERR_BAD_OPTION, "Gemm runs on the direct, general and split-K kernels only");
    if (p->is_int && algo != MM_ALGO_DIRECT && algo != MM_ALGO_GENERAL && algo != MM_ALGO_SPLIT_K)
        return fail(MM_ERR_BAD_OPTION, "MatMulInteger runs on the direct, general and split-K kernels only");
    p->algo = algo;

    if (algo == MM_ALGO_SKINNY_M) {
        const int sreq = opt ? opt->split_k : 0;
        if (sreq < 0) return fail(MM_ERR_BAD_OPTION, "split_k %d is negative", sreq);
        plan_skinny_split(p, sreq);
        const int64_t wgs = p->batch * cdiv(M, 16) * cdiv(N, 64);
        if (wgs * p->split > INT32_MAX)
            return fail(MM_ERR_TOO_LARGE, "too many workgroups (%lld x %d splits)", (long long)wgs, p->split);
    }
    if (algo == MM_ALGO_GENERAL || algo == MM_ALGO_SPLIT_K) {
        int req = opt ? opt->tile : 0;
        if (req < 0 || req > tile_count(p->dtype))
            return fail(MM_ERR_BAD_OPTION, "tile %d out of range 0..%d", req, tile_count(p->dtype));
        if (req > 0) {
            p->tile = req - 1;
            if (!tile_allowed(p->dtype, p->tile, p->is_gemm))
                return fail(MM_ERR_BAD_OPTION, "tile %d has no Gemm kernel", req);
        } else if (rule_tile >= 0) {
            p->tile = rule_tile;
        } else if (algo == MM_ALGO_GENERAL) {
            p->tile = choose_general_tile(p->dtype, p->batch, M, N, K, p->is_gemm);
        } else {
            p->tile = choose_split_tile(p->dtype, p->batch, M, N, K, p->is_gemm);
        }
        if (algo == MM_ALGO_GENERAL && req == 0) {
            plan_tail(p);
            plan_persistent(p);
        }
        const TileCfg *t = tile_entry(p->dtype, p->tile);
        const int64_t tiles = p->batch * cdiv(M, t->bm) * cdiv(N, t->bn);
        if (algo == MM_ALGO_SPLIT_K) {
            int sreq = opt ? opt->split_k : 0;
            if (sreq < 0) return fail(MM_ERR_BAD_OPTION, "split_k %d is negative", sreq);
            plan_split(p, sreq > 0 ? sreq : rule_split);
        }
        if (tiles * p->split > INT32_MAX)
            return fail(MM_ERR_TOO_LARGE, "too many workgroups (%lld tiles x %d splits)", (long long)tiles,
                        p->split);
    }
    return MM_OK;
}

}  // namespace mm

using namespace mm;

extern "C" {

mm_status mm_plan_create_ex(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank,
                            int dtype, const mm_plan_options *opt, mm_plan_t *out) {
    clear_error();
    if (!out) return fail(MM_ERR_NULL_ARG, "out is NULL");
    *out = nullptr;
    if ((!a_shape && a_rank > 0) || (!b_shape && b_rank > 0)) return fail(MM_ERR_NULL_ARG, "shape pointer is NULL");
    if (dtype != MM_FLOAT && dtype != MM_FLOAT16 && dtype != MM_BFLOAT16 && dtype != MM_DOUBLE)
        return fail(MM_ERR_DTYPE, "unknown element type %d", dtype);
    if (opt && opt->reserved != 0) return fail(MM_ERR_BAD_OPTION, "reserved option field must be 0");
    mm_plan_s *p = new (std::nothrow) mm_plan_s();
    if (!p) return fail(MM_ERR_ALLOC, "host allocation failed");
    p->dtype = dtype;
    mm_status st = resolve(a_shape, a_rank, b_shape, b_rank, p);
    if (st == MM_OK) st = select_algo(p, opt);
    if (st == MM_OK) st = alloc_workspace(p, true);
    if (st != MM_OK) {
        delete p;
        return st;
    }
    *out = p;
    return MM_OK;
}

mm_status mm_plan_create(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank, int dtype,
                         mm_plan_t *out) {
    return mm_plan_create_ex(a_shape, a_rank, b_shape, b_rank, dtype, nullptr, out);
}

mm_status mm_int_plan_create(const int64_t *a_shape, int a_rank, const int64_t *b_shape, int b_rank, int a_type,
                             int b_type, int a_zp_kind, int b_zp_kind, const mm_plan_options *opt, mm_plan_t *out) {
    clear_error();
    if (!out) return fail(MM_ERR_NULL_ARG, "out is NULL");
    *out = nullptr;
    if ((!a_shape && a_rank > 0) || (!b_shape && b_rank > 0)) return fail(MM_ERR_NULL_ARG, "shape pointer is NULL");
    auto int_type = [](int t) { return t == MM_UINT8 || t == MM_INT8; };
    if (!int_type(a_type) || !int_type(b_type))
        return fail(MM_ERR_DTYPE, "MatMulInteger takes UINT8 / INT8 operands (got %d, %d)", a_type, b_type);
    auto zp_ok = [](int z) { return z == MM_ZP_NONE || z == MM_ZP_SCALAR || z == MM_ZP_VECTOR; };
    if (!zp_ok(a_zp_kind) || !zp_ok(b_zp_kind)) return fail(MM_ERR_BAD_OPTION, "unknown zero-point kind");
    if (opt && opt->reserved != 0) return fail(MM_ERR_BAD_OPTION, "reserved option field must be 0");
    mm_plan_s *p = new (std::nothrow) mm_plan_s();
    if (!p) return fail(MM_ERR_ALLOC, "host allocation failed");
    p->dtype = MM_INT32;
    p->is_int = true;
    p->a_type = a_type;
    p->b_type = b_type;
    p->zpa_kind = a_zp_kind;
    p->zpb_kind = b_zp_kind;
    mm_status st = resolve(a_shape, a_rank, b_shape, b_rank, p);
    if (st == MM_OK) st = select_algo(p, opt);
    if (st != MM_OK) {
        delete p;
        return st;
    }
    // The tiled kernel needs the row sums of A' when zb' can be non-zero and
    // the column sums of B' when za' can be (a UINT8 operand has a non-zero
    // offset); it forms them itself, so no workspace is needed.
    p->need_ra = b_type == MM_UINT8 || b_zp_kind != MM_ZP_NONE;
    p->need_cb = a_type == MM_UINT8 || a_zp_kind != MM_ZP_NONE;
    // The 256 x 256 tile in the wave layout that holds fewer fragments of
    // the sign-flipped operand (entry 2: two A fragments per wave); the
    // last-round balancing planned for entry 0 holds for entry 2 (same
    // block tile).
    if (p->algo == MM_ALGO_GENERAL && !(opt && opt->tile > 0) && (p->tile == 0 || p->tile == 2))
        p->tile = a_type == MM_UINT8 && b_type == MM_INT8 ? 2 : 0;
    if (p->algo == MM_ALGO_SPLIT_K && tile_entry(MM_INT32, p->tile)->bm * tile_entry(MM_INT32, p->tile)->bn > 128 * 128) {
        delete p;
        return fail(MM_ERR_BAD_OPTION, "MatMulInteger split-K runs on the 128 x 128 tile only");
    }
    st = alloc_workspace(p, true);
    if (st != MM_OK) {
        delete p;
        return st;
    }
    *out = p;
    return MM_OK;
}

mm_status mm_gemm_plan_create(const mm_gemm_desc *d, int dtype, const mm_plan_options *opt, mm_plan_t *out) {
    clear_error();
    if (!out) return fail(MM_ERR_NULL_ARG, "out is NULL");
    *out = nullptr;
    if (!d) return fail(MM_ERR_NULL_ARG, "descriptor is NULL");
    if (dtype != MM_FLOAT && dtype != MM_FLOAT16 && dtype != MM_BFLOAT16)
        return fail(MM_ERR_DTYPE, "Gemm supports FLOAT, FLOAT16 and BFLOAT16 (got %d)", dtype);
    if (d->reserved != 0 || (opt && opt->reserved != 0)) return fail(MM_ERR_BAD_OPTION, "reserved field must be 0");
    if ((d->trans_a != 0 && d->trans_a != 1) || (d->trans_b != 0 && d->trans_b != 1))
        return fail(MM_ERR_BAD_OPTION, "trans_a / trans_b must be 0 or 1");
    if (d->c_rank < -1 || d->c_rank > 2) return fail(MM_ERR_BAD_OPTION, "c_rank %d is not -1, 0, 1 or 2", d->c_rank);
    if (d->a_rows < 0 || d->a_cols < 0 || d->b_rows < 0 || d->b_cols < 0)
        return fail(MM_ERR_NEG_DIM, "a Gemm operand dimension is negative");
    const int64_t M = d->trans_a ? d->a_cols : d->a_rows;
    const int64_t K = d->trans_a ? d->a_rows : d->a_cols;
    const int64_t Kb = d->trans_b ? d->b_cols : d->b_rows;
    const int64_t N = d->trans_b ? d->b_rows : d->b_cols;
    if (K != Kb)
        return fail(MM_ERR_K_MISMATCH, "inner dimensions differ: A' has K=%lld, B' has K=%lld", (long long)K,
                    (long long)Kb);
    // C right-aligned against (M, N); each dimension 1 or the output's.
    int c_mode = kBiasNone;
    int64_t cr = 1, cc = 1;
    if (d->c_rank >= 1) cc = d->c_shape[d->c_rank - 1];
    if (d->c_rank == 2) cr = d->c_shape[0];
    if (cr < 0 || cc < 0) return fail(MM_ERR_NEG_DIM, "a C dimension is negative");
    if (d->c_rank >= 0) {
        if ((cr != 1 && cr != M) || (cc != 1 && cc != N))
            return fail(MM_ERR_BROADCAST, "C [%lld, %lld] does not broadcast to [%lld, %lld]", (long long)cr,
                        (long long)cc, (long long)M, (long long)N);
        c_mode = (cr == 1 && cc == 1) ? kBiasScalar : cr == 1 ? kBiasRow : cc == 1 ? kBiasCol : kBiasFull;
    }
    mm_plan_s *p = new (std::nothrow) mm_plan_s();
    if (!p) return fail(MM_ERR_ALLOC, "host allocation failed");
    p->dtype = dtype;
    p->is_gemm = true;
    p->ta = d->trans_a;
    p->tb = d->trans_b;
    p->alpha = d->alpha;
    p->beta = d->beta;
    p->c_mode = c_mode;
    p->ldc = c_mode == kBiasFull ? N : 0;
    p->a_rank = p->b_rank = 2;
    p->a_shape[0] = d->a_rows;
    p->a_shape[1] = d->a_cols;
    p->b_shape[0] = d->b_rows;
    p->b_shape[1] = d->b_cols;
    p->b_numel = d->b_rows * d->b_cols;
    p->out_rank = 2;
    p->out_shape[0] = M;
    p->out_shape[1] = N;
    p->M = M;
    p->N = N;
    p->K = K;
    p->out_numel = M * N;
    p->total_batch = 1;
    p->batch = 1;
    p->kernel_m = M;
    p->folded = 0;
    mm_status st = select_algo(p, opt);
    if (st == MM_OK) st = alloc_workspace(p, true);
    if (st != MM_OK) {
        mm_plan_destroy(p);
        return st;
    }
    *out = p;
    return MM_OK;
}

mm_status mm_plan_output_shape(mm_plan_t p, int64_t *shape, int *rank) {
    if (!p || !rank || (!shape && p->out_rank > 0)) return fail(MM_ERR_NULL_ARG, "NULL argument");
    for (int i = 0; i < p->out_rank; ++i) shape[i] = p->out_shape[i];
    *rank = p->out_rank;
    return MM_OK;
}

int64_t mm_plan_output_numel(mm_plan_t p) { return p ? p->out_numel : -1; }

int mm_plan_algo(mm_plan_t p) { return p ? p->algo : -1; }

size_t mm_plan_workspace_bytes(mm_plan_t p) { return p ? (size_t)p->workspace_bytes : 0; }

mm_status mm_plan_get_info(mm_plan_t p, mm_plan_info *info) {
    if (!p || !info) return fail(MM_ERR_NULL_ARG, "NULL argument");
    memset(info, 0, sizeof(*info));
    info->dtype = p->dtype;
    info->algo = p->algo;
    info->M = p->M;
    info->N = p->N;
    info->K = p->K;
    info->batch = p->batch;
    info->kernel_m = p->kernel_m;
    info->folded = p->folded;
    info->batch_rank = p->bd.nb;
    for (int d = 0; d < p->bd.nb; ++d) {
        info->batch_dims[d] = p->bd.dim[d];
        info->a_batch_strides[d] = p->bd.sa[d];
        info->b_batch_strides[d] = p->bd.sb[d];
    }
    info->tile = p->tile >= 0 ? p->tile + 1 : 0;
    info->split_k = p->split;
    info->k_chunk = p->kchunk;
    info->workspace_bytes = p->workspace_bytes;
    info->tail_col = p->tail_col;
    info->tail_tile = p->tail_tile >= 0 ? p->tail_tile + 1 : 0;
    {
        std::lock_guard<std::mutex> lock(const_cast<mm_plan_s *>(p)->cb_mutex);
        info->constant_b_packed = p->cb_set && p->cbp_ok ? 1 : 0;
    }
    info->flops = 2.0 * (double)p->total_batch * (double)p->M * (double)p->N * (double)p->K;
    int64_t na = 1, nb = 1;
    for (int i = 0; i < p->a_rank; ++i) na *= p->a_shape[i];
    for (int i = 0; i < p->b_rank; ++i) nb *= p->b_shape[i];
    if (p->is_int)  // one-byte inputs, INT32 output
        info->min_bytes = (double)na + (double)nb + 4.0 * (double)p->out_numel;
    else
        info->min_bytes = (double)elem_size(p->dtype) * ((double)na + (double)nb + (double)p->out_numel);
    return MM_OK;
}

int mm_tile_count(int dtype) { return tile_count(dtype); }

mm_status mm_tile_config(int dtype, int index, int *bm, int *bn, int *bk) {
    const TileCfg *t = tile_entry(dtype, index);
    if (!t) return fail(MM_ERR_BAD_OPTION, "no tile %d for dtype %d", index, dtype);
    if (bm) *bm = t->bm;
    if (bn) *bn = t->bn;
    // K elements per stage: INT8 tiles stage one-byte elements (the table is
    // shared by the MM_UINT8 / MM_INT8 / MM_INT32 codes).
    const bool int_code = dtype == MM_INT8 || dtype == MM_UINT8 || dtype == MM_INT32;
    if (bk) *bk = t->bkb / (int_code ? 1 : elem_size(dtype));
    return MM_OK;
}

const char *mm_status_string(mm_status s) {
    switch (s) {
    case MM_OK: return "ok";
    case MM_ERR_NULL_ARG: return "null argument";
    case MM_ERR_RANK: return "invalid rank";
    case MM_ERR_NEG_DIM: return "negative dimension";
    case MM_ERR_K_MISMATCH: return "inner dimension mismatch";
    case MM_ERR_BROADCAST: return "batch dimensions not broadcastable";
    case MM_ERR_DTYPE: return "unsupported element type";
    case MM_ERR_BAD_OPTION: return "invalid option";
    case MM_ERR_TOO_LARGE: return "size too large";
    case MM_ERR_ALLOC: return "allocation failed";
    case MM_ERR_HIP: return "HIP runtime error";
    case MM_ERR_SIZE: return "constant B size differs from the planned B";
    case MM_ERR_NO_CONSTANT_B: return "plan owns no constant B";
    }
    return "unknown status";
}

const char *mm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
