// Launch planning: which kernel configuration runs a shape, and how its
// output tiles and K chunks are spread over the workgroups.
//
// Scheduling follows the persistent Stream-K scheme described on "Beyond
// Kernel 7: Closing the Gap to cuBLAS on an H100 FP32 GEMM", section
// "Kernel 14 and Stream-K": the work is the stream of (output tile, K chunk)
// steps; whole tiles are handed out in full waves first, and only the tiles
// left over are split, evenly, over a grid of resident workgroups.  Tile
// counts that fill whole waves run purely data-parallel (one workgroup per
// tile), which is the plain tiling of the other pages.
#include "plan.h"

#include "sgemm_f32.h"

namespace sgemm {

const CfgInfo kCfgs[] = {
    {SGEMM_CFG_AUTO, 0, 0, 0, 0, kKindValu, 0, false, false, "auto"},
    {SGEMM_CFG_MFMA_256x256x16, 256, 256, 16, 512, kKindMfma, 1, false, false, "mfma_256x256x16"},
    {SGEMM_CFG_MFMA_128x128x32, 128, 128, 32, 256, kKindMfma, 2, false, false, "mfma_128x128x32"},
    {SGEMM_CFG_MFMA_256x256x32, 256, 256, 32, 256, kKindMfma, 1, false, false, "mfma_256x256x32"},
    {SGEMM_CFG_MFMA_256x128x32, 256, 128, 32, 256, kKindMfma, 1, false, false, "mfma_256x128x32"},
    {SGEMM_CFG_VALU_128x128x8, 128, 128, 8, 256, kKindValu, 2, false, false, "valu_128x128x8"},
    {SGEMM_CFG_MFMA_256x256x32_W8, 256, 256, 32, 512, kKindMfma, 1, false, false, "mfma_256x256x32_w8"},
    {SGEMM_CFG_MFMA_128x128x32_W8, 128, 128, 32, 512, kKindMfma, 2, false, false, "mfma_128x128x32_w8"},
    {SGEMM_CFG_MFMA_64x64x32, 64, 64, 32, 256, kKindMfma, 4, false, false, "mfma_64x64x32"},
    {SGEMM_CFG_MFMA_128x64x32, 128, 64, 32, 256, kKindMfma, 2, false, false, "mfma_128x64x32"},
    {SGEMM_CFG_MFMA_64x64x64, 64, 64, 64, 256, kKindMfma, 2, false, false, "mfma_64x64x64"},
    {SGEMM_CFG_MFMA_128x128x64, 128, 128, 64, 256, kKindMfma, 1, false, false, "mfma_128x128x64"},
    {SGEMM_CFG_MFMA_64x64x128, 64, 64, 128, 256, kKindMfma, 1, false, false, "mfma_64x64x128"},
    {SGEMM_CFG_DL_64x64x32, 64, 64, 32, 256, kKindMfmaDl, 2, true, true, "dl_64x64x32"},
    {SGEMM_CFG_DL_64x64x64_K2, 64, 64, 64, 512, kKindMfmaDl, 1, false, false, "dl_64x64x64_k2"},
    {SGEMM_CFG_DL_128x128x32, 128, 128, 32, 512, kKindMfmaDl, 1, true, true, "dl_128x128x32"},
    {SGEMM_CFG_DL_256x256x16, 256, 256, 16, 512, kKindMfmaDl, 1, true, true, "dl_256x256x16"},
    {SGEMM_CFG_DL_64x64x32_K2, 64, 64, 32, 512, kKindMfmaDl, 2, false, false, "dl_64x64x32_k2"},
    {SGEMM_CFG_DL_128x128x32_K2, 128, 128, 32, 512, kKindMfmaDl, 1, false, false, "dl_128x128x32_k2"},
    {SGEMM_CFG_DL_64x64x64, 64, 64, 64, 256, kKindMfmaDl, 1, true, true, "dl_64x64x64"},
    {SGEMM_CFG_DL_128x256x16, 128, 256, 16, 256, kKindMfmaDl, 2, false, false, "dl_128x256x16"},
    {SGEMM_CFG_DL_256x128x16, 256, 128, 16, 256, kKindMfmaDl, 2, false, false, "dl_256x128x16"},
    {SGEMM_CFG_GENERIC_64x64x16, 64, 64, 16, 256, kKindGeneric, 2, true, true, "generic_64x64x16"},
    {SGEMM_CFG_SKINNY_16x256, 16, 256, kSkinnyBlock, 512, kKindSkinny, 1, true, true, "skinny_16x256"},
    {SGEMM_CFG_ROWDOT_N8, 8, 8, 0, 512, kKindRowdot, 2, true, true, "rowdot_n8"},
    {SGEMM_CFG_VALU_256x128x8, 256, 128, 8, 256, kKindValu, 2, false, false, "valu_256x128x8"},
};
const int kNumCfgs = SGEMM_NUM_CFGS;

static_assert(sizeof(kCfgs) / sizeof(kCfgs[0]) == SGEMM_NUM_CFGS, "config table size");

const FixedShapeInfo kFixedShapes[] = {
    {4096, 4096, 4096, SGEMM_CFG_DL_256x256x16, 4},
    {2048, 2048, 2048, SGEMM_CFG_DL_128x128x32, 4},
    {1024, 1024, 1024, SGEMM_CFG_DL_64x64x64, 4},
    {1024, 1024, 16384, SGEMM_CFG_DL_64x64x64, 4},
};
const int kNumFixedShapes = sizeof(kFixedShapes) / sizeof(kFixedShapes[0]);

int64_t workspace_bytes(int grid, int sk_tiles, int bm, int bn) {
    if (sk_tiles <= 0) return 0;
    return (int64_t)grid * 2 * bm * bn * 4;
}

static bool divides(const CfgInfo &c, int M, int N, int K) {
    return M % c.bm == 0 && N % c.bn == 0 && K % c.bk == 0;
}

// Whether configuration c can run the shape: the generic kernel runs
// anything; the others need the aligned fast-path layout, and a tile that
// divides the shape unless they mask ragged edges.
// The skinny kernel: at most 16 rows, B stored K x N (A and C read and
// written one float at a time; B too where it is off the 16-byte grid).
static bool skinny_fits(const PlanRequest &r) { return r.M <= 16 && !r.trans_b; }

// The row-dot kernel: at most 8 columns, A stored M x K (B and C read and
// written one float at a time; A too where it is off the 16-byte grid).
static bool rowdot_fits(const PlanRequest &r) { return r.N >= 1 && r.N <= 8 && !r.trans_a; }

static bool fits(const CfgInfo &c, int M, int N, int K, bool aligned, bool transposed) {
    if (c.kind == kKindGeneric) return true;
    if (!aligned || (transposed && !c.layouts)) return false;
    return c.edge || divides(c, M, N, K);
}

static int occ_of(const PlanRequest &r, int cfg) {
    int o = r.occupancy ? r.occupancy[cfg] : kCfgs[cfg].default_occ;
    return o > 0 ? o : 1;
}

// Tile-order grouping for a run of R consecutive tiles (one XCD's share):
// groups of g tile rows, walked column by column, so that a run covers about
// g rows x R/g columns; g minimises the panels touched, g + R/g.
static int pick_group_m(int tiles_m, int run) {
    int best = 1, best_cost = 1 + run;
    for (int g = 2; g <= tiles_m && g <= run; g *= 2) {
        if (tiles_m % g) continue;
        int cost = g + (run + g - 1) / g;
        if (cost < best_cost) { best = g; best_cost = cost; }
    }
    return best;
}

// Automatic choice of the kernel family:
//   * at most 2 columns (or 8 once A has 2^26 elements, or when the tiled
//     kernels cannot load the layout), A stored M x K, M and K at least 256:
//     the row-dot kernel (per-row dot products streaming A; y = A x).
//     16384 x 1 x 16384: 209 us against 1190 on the general kernel and 216
//     for hipBLASLt; 16384 x 8 x 16384: 231 against 264 on the tiled kernel.
//     At 4096 x 8 x 4096 the tiled kernel is faster (26 against 41 us):
//     staging B per workgroup costs as much as the little A each one streams;
//   * at most 16 rows, B stored K x N, N and K at least 256 (9-16 rows:
//     also B above 2^22 elements or a layout the tiled kernels cannot
//     load): the skinny kernel, which streams B without computing the empty
//     rows of a 64-row tile (1 x 16384 x 16384: 6.35 TB/s of B against 4.4
//     for the tiled kernel and 5.6 for hipBLASLt; 8 x 8192 x 28672: 5.6
//     against 4.3 and 4.9; 16 x 16384 x 16384, on 16 x 16 x 4 matrix-core
//     steps: 4.97 against 4.3 and 5.75);
//   * layouts the vector kernels cannot load: the general kernel;
//   * everything else: the direct-to-LDS tiles, configuration and schedule
//     by the cost model below (kTiledChoice).
constexpr int kTiledChoice = -1;
static int auto_config(const PlanRequest &r, bool aligned) {
    const int M = r.M, N = r.N, K = r.K;
    // 9-16 rows with B of at most 2^22 elements: the tiled kernel, 1-2 us
    // faster there (16 x 2048 x 2048: 17.2 against 18.8 us), where it can
    // load the layout.
    if (skinny_fits(r) && N >= 256 && K >= 256 && (M <= 8 || !aligned || (int64_t)N * K > ((int64_t)1 << 22)))
        return SGEMM_CFG_SKINNY_16x256;
    if (rowdot_fits(r) && M >= 256 && K >= 256 && (N <= 2 || !aligned || (int64_t)M * K >= ((int64_t)1 << 26)) &&
        (r.sched != SGEMM_SCHED_DP || K <= kRowdotFloats / rowdot_cols(N)))
        return SGEMM_CFG_ROWDOT_N8;
    if (!aligned) return SGEMM_CFG_GENERIC_64x64x16;
    return kTiledChoice;
}

// Cost model of the automatic choice among the direct-to-LDS configurations
// and their schedules, in microseconds of kernel time.  A tile's K chunk
// takes 2 BM BN BK FLOPs at the CU's matrix-core rate (256 FLOPs per clock at
// 2.3 GHz) times the configuration's efficiency, and each tile a workgroup
// runs adds a fixed cost (its first loads, the C store), hidden in part when
// a second workgroup shares the CU.  Data-parallel: the CU with the most
// tiles sets the time.  Split: the full waves of whole tiles, then the
// longest split range, with a tile's fixed cost for every tile that range
// touches, then the summing kernel (a launch, and its traffic: every partial
// tile read, the split tiles of C written).  Writing C bounds
// the time from below.  On a narrow C (at most 8 tiles of 64 across a side,
// at least two waves of them) the 64x64x32 configuration, two workgroups per
// CU, keeps more loads in flight while the long operand streams with little
// reuse, and its efficiency is scaled up by 3% (fits gave 2-3%; alternating
// rounds on four such shapes measured it 1-5% faster than 64x64x64).
// The coefficients are least-squares fits (on log time) to back-to-back
// timings of both schedules of each configuration on 236 seeded shapes,
// sides log-uniform in 64..16384, on one MI355X.  With the fit to any three
// of the four sweeps, the choice on the fourth came within 0.3-0.8% of its
// fastest candidate (geometric mean per shape), where the earlier fixed
// rules were 3.6-15% off (worst single shape 1.18x against 3.8x, at small K,
// where splitting tiles cost more than it balanced).  The values below are
// the fit to all four; tuning/fit_cost_model.py reproduces them from the
// sweeps' timings in tuning/plan_sweeps.csv.
struct CostCoef {
    int cfg;
    double eff;       // fraction of the matrix-core rate in the K loop
    double tile_us;   // fixed cost of one tile
};
static const CostCoef kCostCoefs[] = {
    {SGEMM_CFG_DL_256x256x16, 1.014, 3.855},
    {SGEMM_CFG_DL_128x128x32, 0.9906, 3.097},
    {SGEMM_CFG_DL_64x64x64, 0.9407, 1.909},
    {SGEMM_CFG_DL_64x64x32, 0.9069, 1.684},
};
constexpr double kCuFlopsPerUs = 256.0 * 2300.0;
constexpr double kNarrowEff64x64x32 = 1.03;  // 64x64x32 on a narrow C
constexpr double kSumLaunchUs = 3.776;       // summing kernel: launch and fixed cost
constexpr double kSumBytesPerUs = 5.609e6;   // summing kernel: partial tiles read, C written
constexpr double kStoreBytesPerUs = 3.05e6;  // C written by the GEMM kernel

static int64_t ceil_div(int64_t a, int64_t b) { return b > 0 ? (a + b - 1) / b : 0; }

double plan_cost(const Plan &p, int M, int N, int cus, int occ) {
    const CostCoef *cc = nullptr;
    for (const CostCoef &x : kCostCoefs)
        if (x.cfg == p.config) cc = &x;
    if (!cc || cus < 1) return -1.0;
    if (occ < 1) occ = 1;
    double eff = cc->eff;
    const int64_t tm64 = ceil_div(M, 64), tn64 = ceil_div(N, 64);
    if (p.config == SGEMM_CFG_DL_64x64x32 && (tm64 <= 8 || tn64 <= 8) && tm64 * tn64 >= 2 * (int64_t)cus)
        eff *= kNarrowEff64x64x32;
    const double chunk_us = 2.0 * p.bm * p.bn * p.bk / (kCuFlopsPerUs * eff);
    double t;
    if (p.sk_tiles == 0) {
        const int64_t n = ceil_div(p.dp_tiles, cus);
        t = (double)n * p.ipt * chunk_us + (double)ceil_div(n, occ) * cc->tile_us;
    } else {
        const int64_t waves = p.dp_tiles > 0 && p.grid > 0 ? p.dp_tiles / p.grid : 0;
        const int64_t longest = ceil_div(p.sk_iters, p.sk_grid);
        int64_t segments = ceil_div(longest, p.ipt) + (p.ipt > 0 && longest % p.ipt ? 1 : 0);
        if (segments > p.sk_tiles) segments = p.sk_tiles;
        t = (double)waves * (p.ipt * chunk_us + cc->tile_us) + (double)longest * chunk_us +
            (double)segments * cc->tile_us;
        const double tile_bytes = 4.0 * p.bm * p.bn;
        t += kSumLaunchUs + ((double)p.sk_grid + 2.0 * p.sk_tiles) * tile_bytes / kSumBytesPerUs;
    }
    const double c_us = 4.0 * M * N / kStoreBytesPerUs;
    return t > c_us ? t : c_us;
}

int staged_equivalent(int cfg) {
    switch (cfg) {
    case SGEMM_CFG_DL_64x64x32:
    case SGEMM_CFG_DL_64x64x32_K2: return SGEMM_CFG_MFMA_64x64x32;
    case SGEMM_CFG_DL_64x64x64:
    case SGEMM_CFG_DL_64x64x64_K2: return SGEMM_CFG_MFMA_64x64x64;
    case SGEMM_CFG_DL_128x128x32:
    case SGEMM_CFG_DL_128x128x32_K2: return SGEMM_CFG_MFMA_128x128x32;
    case SGEMM_CFG_DL_256x256x16: return SGEMM_CFG_MFMA_256x256x16;
    default: return cfg;
    }
}

bool dl_offsets_fit(int cfg, bool edge, int64_t lda, int64_t ldb, bool trans_a, bool trans_b) {
    if (kCfgs[cfg].kind != kKindMfmaDl) return true;
    const int64_t lim = (int64_t)1 << (edge ? 31 : 32);
    // Rows a lane's offset spans from the operand's base: the tile's rows of
    // a k-contiguous operand, the chunk's k rows of an m/n-contiguous one.
    const int64_t rows_a = trans_a ? kCfgs[cfg].bk : kCfgs[cfg].bm;
    const int64_t rows_b = trans_b ? kCfgs[cfg].bn : kCfgs[cfg].bk;
    return rows_a * lda * 4 < lim && rows_b * ldb * 4 < lim;
}

// The skinny kernel's plan, in the terms of the tiled ones: a "tile" is a
// strip of 256 columns (one tile row, 16 rows high), its "K chunks" are the
// KS splits of K, and every workgroup owns exactly one (strip, split) step,
// so KS > 1 is a Stream-K plan whose every tile is split.  KS keeps the
// grid within one workgroup per CU (8 waves: two per SIMD), with at least
// 256 k per split; the data-parallel schedule forces KS = 1.  Rounding KS
// down leaves some CUs idle but runs one round: 65 strips x 3 splits took
// 204 us at 1 x 16385 x 16384 where 65 x 4 (four workgroups in a second
// round) took 259.
static int plan_skinny(const PlanRequest &req, int cus, Plan *out) {
    if (!skinny_fits(req)) return SGEMM_ERR_CONFIG;
    const CfgInfo &c = kCfgs[SGEMM_CFG_SKINNY_16x256];
    Plan p{};
    p.config = SGEMM_CFG_SKINNY_16x256;
    p.bm = c.bm; p.bn = c.bn; p.threads = c.threads;
    p.tiles_m = (req.M + c.bm - 1) / c.bm;
    p.tiles_n = (req.N + c.bn - 1) / c.bn;
    p.edge = 1;
    const int strips = p.tiles_n;
    int ks = 1;
    if (req.sched != SGEMM_SCHED_DP && strips > 0 && req.K > 0) {
        ks = cus / strips > 1 ? cus / strips : 1;
        const int by_k = req.K / 256 > 1 ? req.K / 256 : 1;
        if (ks > by_k) ks = by_k;
        if (req.sched == SGEMM_SCHED_STREAMK && ks < 2 && req.K >= 2) ks = 2;
    }
    p.bk = req.K > 0 ? (req.K + ks - 1) / ks : 1;   // k per split (dealt to it in blocks of up to 512)
    p.ipt = req.K > 0 ? (req.K + p.bk - 1) / p.bk : 0;
    const int tiles = p.tiles_m * p.tiles_n;
    if (tiles == 0 || p.ipt == 0 || (p.ipt == 1 && req.sched != SGEMM_SCHED_STREAMK)) {
        p.dp_tiles = tiles; p.sk_tiles = 0; p.sk_grid = 0; p.grid = tiles;
        p.sched = SGEMM_SCHED_DP;
    } else {
        p.dp_tiles = 0; p.sk_tiles = tiles;
        p.sk_iters = (int64_t)tiles * p.ipt;
        p.sk_grid = (int)p.sk_iters; p.grid = p.sk_grid;
        p.sched = SGEMM_SCHED_STREAMK;
        p.workspace_bytes = (int64_t)p.ipt * 16 * strips * c.bn * 4;   // [KS][16][strips * 256]
    }
    p.xcd_remap = 0;
    p.group_m = 1;
    *out = p;
    return SGEMM_OK;
}

// The row-dot kernel's plan, in the same terms: a "tile" is a block of
// rows (all 8 columns), its "K chunks" are the KS splits of K, every
// workgroup owns one (block, split) step.  KS is at least what fits B's
// split in LDS; beyond that, blocks and splits stay within the resident
// workgroups of one round (two per CU); a data-parallel schedule needs B's
// whole K range to fit.
static int plan_rowdot(const PlanRequest &req, int cus, int occ, Plan *out) {
    if (!rowdot_fits(req)) return SGEMM_ERR_CONFIG;
    const CfgInfo &c = kCfgs[SGEMM_CFG_ROWDOT_N8];
    const int M = req.M, K = req.K;
    const int kb = kRowdotFloats / rowdot_cols(req.N);   // k of one split at most
    int ks = K > 0 ? (K + kb - 1) / kb : 1;
    if (req.sched == SGEMM_SCHED_DP && ks > 1) return SGEMM_ERR_CONFIG;
    const int64_t target = (int64_t)cus * occ;
    const int64_t rb_max = M > 0 ? (M + 7) / 8 : 0;   // blocks of at least a row per wave
    int64_t rb = target / ks > 1 ? target / ks : 1;
    if (rb > rb_max) rb = rb_max;
    if (req.sched != SGEMM_SCHED_DP && rb > 0 && rb * ks < target) {
        // Few rows: split K further (at least 256 k per split), within one
        // resident round.
        int64_t more = target / rb;
        const int64_t by_k = K / 256 > 1 ? K / 256 : 1;
        if (more > by_k) more = by_k;
        if (more > ks) ks = (int)more;
    }
    if (req.sched == SGEMM_SCHED_STREAMK && ks < 2 && K >= 8) ks = 2;
    Plan p{};
    p.config = SGEMM_CFG_ROWDOT_N8;
    p.threads = c.threads;
    p.bn = c.bn;
    p.bm = rb > 0 ? (int)((M + rb - 1) / rb) : c.bm;
    p.tiles_m = M > 0 ? (M + p.bm - 1) / p.bm : 0;
    p.tiles_n = req.N > 0 ? 1 : 0;
    p.bk = K > 0 ? rowdot_k_per(K, ks) : 1;
    p.ipt = K > 0 ? (K + p.bk - 1) / p.bk : 0;
    p.edge = 1;
    const int tiles = p.tiles_m * p.tiles_n;
    if (tiles == 0 || p.ipt == 0 || (p.ipt == 1 && req.sched != SGEMM_SCHED_STREAMK)) {
        p.dp_tiles = tiles; p.sk_tiles = 0; p.sk_grid = 0; p.grid = tiles;
        p.sched = SGEMM_SCHED_DP;
    } else {
        p.dp_tiles = 0; p.sk_tiles = tiles;
        p.sk_iters = (int64_t)tiles * p.ipt;
        p.sk_grid = (int)p.sk_iters; p.grid = p.sk_grid;
        p.sched = SGEMM_SCHED_STREAMK;
        p.workspace_bytes = (int64_t)p.sk_grid * p.bm * c.bn * 4;   // [KS][rows][8], rows padded to blocks
    }
    p.xcd_remap = 0;
    p.group_m = 1;
    *out = p;
    return SGEMM_OK;
}

// The compile-time-shape kernel for a request: the data-parallel plan of
// the same configuration, which must be the one a kFixedShapes entry was
// compiled for (shape, configuration, tile order, one workgroup per tile).
static int plan_fixed(const PlanRequest &req, Plan *out) {
    PlanRequest r = req;
    r.sched = SGEMM_SCHED_DP;
    Plan p;
    const int st = make_plan(r, &p);
    if (st != SGEMM_OK) return st;
    if (!req.aligned || req.trans_a || req.trans_b || p.edge || p.sk_tiles) return SGEMM_ERR_CONFIG;
    for (int i = 0; i < kNumFixedShapes; ++i) {
        const FixedShapeInfo &f = kFixedShapes[i];
        if (f.M == req.M && f.N == req.N && f.K == req.K && f.config == p.config && f.group_m == p.group_m &&
            p.xcd_remap && p.grid == p.tiles_m * p.tiles_n) {
            p.fixed = i + 1;
            *out = p;
            return SGEMM_OK;
        }
    }
    return SGEMM_ERR_CONFIG;
}

// Internal schedule of the automatic choice: whole tiles in full waves, the
// remainder split (what SGEMM_SCHED_AUTO runs when it splits).
constexpr int kSchedSplitRest = -100;

// Plan of a tiled configuration (not the skinny or row-dot kernels) under
// `sched`: SGEMM_SCHED_AUTO (the rules below), SGEMM_SCHED_DP,
// SGEMM_SCHED_STREAMK (every tile split) or kSchedSplitRest.
static int plan_tiled(const PlanRequest &req, int cfg, int sched, int cus, Plan *out) {
    const int M = req.M, N = req.N, K = req.K;
    const bool aligned = req.aligned != 0, transposed = req.trans_a || req.trans_b;
    const CfgInfo &c = kCfgs[cfg];
    if (!fits(c, M, N, K, aligned, transposed)) return SGEMM_ERR_CONFIG;

    Plan p{};
    p.config = cfg;
    p.bm = c.bm; p.bn = c.bn; p.bk = c.bk; p.threads = c.threads;
    p.tiles_m = (M + c.bm - 1) / c.bm;
    p.tiles_n = (N + c.bn - 1) / c.bn;
    p.ipt = (K + c.bk - 1) / c.bk;
    p.edge = (c.kind == kKindGeneric || !divides(c, M, N, K)) ? 1 : 0;
    const int tiles = p.tiles_m * p.tiles_n;
    const int occ = occ_of(req, cfg);
    // Split workgroups per CU: one by default (measured faster than filling
    // every resident slot, which multiplies partial tiles), else as asked.
    const int sk_per_cu = req.sk_wg_per_cu > 0 ? req.sk_wg_per_cu : 1;
    const int cap = cus * (sk_per_cu < occ ? sk_per_cu : occ);

    if (tiles == 0 || p.ipt == 0) sched = SGEMM_SCHED_DP;  // nothing to split
    if (sched == SGEMM_SCHED_AUTO) {
        if (tiles >= cus && tiles % cus == 0) sched = SGEMM_SCHED_DP;
        else if (tiles < cus && p.ipt < 2 * kMinSkIters) sched = SGEMM_SCHED_DP;  // too short to split
        else if (tiles > cus && tiles <= (int64_t)occ * cus && 100 * (int64_t)tiles >= 85 * (int64_t)occ * cus)
            sched = SGEMM_SCHED_DP;   // one resident wave, nearly full: every tile runs at once
        else sched = kSchedSplitRest;
    }

    if (sched == SGEMM_SCHED_DP) {
        p.dp_tiles = tiles;
        p.sk_tiles = 0;
        p.sk_grid = 0;
        p.grid = tiles;
    } else {
        // Whole tiles in full waves first, the remainder split.  The split
        // part runs on the first sk_grid logical workgroups, each owning a
        // contiguous run of at least kMinSkIters (tile, K chunk) steps when
        // there are that many.
        int dp = sched == SGEMM_SCHED_STREAMK ? 0 : (tiles / cap) * cap;
        if (dp == cap) {
            // One full wave and a remainder: split everything instead when
            // that ends sooner.  The remainder alone spreads over at most
            // (its steps / kMinSkIters) workgroups, so with few K chunks per
            // tile its split part can take longer than the whole product
            // spread over the full grid (64x64 tiles at 1024x1028x2048: 94
            // TFLOP/s split whole against 89).
            const int64_t rest = (int64_t)(tiles - dp) * p.ipt;
            int64_t g = rest / kMinSkIters;
            if (g > cap) g = cap;
            if (g < 1) g = 1;
            const int64_t hybrid = p.ipt + (rest + g - 1) / g;
            const int64_t whole = ((int64_t)tiles * p.ipt + cap - 1) / cap;
            if (whole < hybrid) dp = 0;
        }
        p.dp_tiles = dp;
        p.sk_tiles = tiles - dp;
        int64_t sk_iters = (int64_t)p.sk_tiles * p.ipt;
        int64_t g = sk_iters / kMinSkIters;
        if (g > cap) g = cap;
        if (g < 1) g = 1;
        if (sk_iters == 0) g = 0;
        p.sk_grid = (int)g;
        p.grid = dp > 0 ? cap : (int)g;
        // The kernel's split bookkeeping is 32-bit; beyond that range run
        // whole tiles only.
        if ((sk_iters + 1) * g >= ((int64_t)1 << 31)) {
            p.dp_tiles = tiles;
            p.sk_tiles = 0;
            p.sk_grid = 0;
            p.grid = tiles;
        }
    }
    p.sk_iters = (int64_t)p.sk_tiles * p.ipt;
    p.sched = p.sk_tiles > 0 ? SGEMM_SCHED_STREAMK : SGEMM_SCHED_DP;
    p.xcd_remap = (p.grid >= 8 && p.grid % 8 == 0) ? 1 : 0;
    int run = p.xcd_remap ? p.grid / 8 : p.grid;
    if (run < 1) run = 1;
    p.group_m = pick_group_m(p.tiles_m > 0 ? p.tiles_m : 1, run);
    // A narrow C: few tile columns and a B that fits one XCD's L2 (4 MiB)
    // go row by row, so the tiles that share an A panel run side by side
    // and A streams through once (49152x192x4096: 139 TFLOP/s against 134
    // with 16-row groups); few tile rows and a small A, column by column.
    if (p.tiles_n <= 8 && (int64_t)K * N * 4 <= ((int64_t)4 << 20)) p.group_m = 1;
    else if (p.tiles_m <= 8 && (int64_t)M * K * 4 <= ((int64_t)4 << 20)) p.group_m = p.tiles_m > 0 ? p.tiles_m : 1;
    p.workspace_bytes = workspace_bytes(p.sk_grid, p.sk_tiles, p.bm, p.bn);
    *out = p;
    return SGEMM_OK;
}

// The automatic choice among the direct-to-LDS configurations: the plan of
// least modelled time (plan_cost) over each configuration's data-parallel
// and split schedules (only the one asked for when the call fixes the
// schedule); ties go to the larger tile.
static const int kTiled[] = {SGEMM_CFG_DL_256x256x16, SGEMM_CFG_DL_128x128x32, SGEMM_CFG_DL_64x64x64,
                             SGEMM_CFG_DL_64x64x32};

// The inputs of one automatic choice: the request's values (the occupancy of
// the four configurations, not the pointer to it).
struct CostKey {
    int M, N, K, sched, cus, sk_wg_per_cu, aligned, trans_a, trans_b;
    int occ[4];
    bool operator==(const CostKey &o) const {
        return M == o.M && N == o.N && K == o.K && sched == o.sched && cus == o.cus &&
               sk_wg_per_cu == o.sk_wg_per_cu && aligned == o.aligned && trans_a == o.trans_a &&
               trans_b == o.trans_b && occ[0] == o.occ[0] && occ[1] == o.occ[1] && occ[2] == o.occ[2] &&
               occ[3] == o.occ[3];
    }
};

static int plan_by_cost_uncached(const PlanRequest &req, int cus, Plan *out);

// The automatic choice weighs eight plans (~0.3 us); calls that repeat a
// shape take it from a few per-thread entries instead.
static int plan_by_cost(const PlanRequest &req, int cus, Plan *out) {
    CostKey key{req.M, req.N, req.K, req.sched, cus, req.sk_wg_per_cu, req.aligned, req.trans_a, req.trans_b, {}};
    for (int i = 0; i < 4; ++i) key.occ[i] = occ_of(req, kTiled[i]);
    constexpr int kEntries = 4;
    struct Entry {
        bool used;
        CostKey key;
        Plan plan;
    };
    thread_local Entry cache[kEntries] = {};
    thread_local int next = 0;
    for (const Entry &e : cache)
        if (e.used && e.key == key) {
            *out = e.plan;
            return SGEMM_OK;
        }
    const int st = plan_by_cost_uncached(req, cus, out);
    if (st == SGEMM_OK) {
        cache[next] = Entry{true, key, *out};
        next = (next + 1) % kEntries;
    }
    return st;
}

static int plan_by_cost_uncached(const PlanRequest &req, int cus, Plan *out) {
    int scheds[2] = {SGEMM_SCHED_DP, kSchedSplitRest};
    int n_sched = 2;
    if (req.sched == SGEMM_SCHED_DP || req.sched == SGEMM_SCHED_STREAMK) {
        scheds[0] = req.sched;
        n_sched = 1;
    }
    bool have = false;
    double best = 0.0;
    for (const int cfg : kTiled) {
        for (int i = 0; i < n_sched; ++i) {
            Plan p;
            if (plan_tiled(req, cfg, scheds[i], cus, &p) != SGEMM_OK) continue;
            const double t = plan_cost(p, req.M, req.N, cus, occ_of(req, cfg));
            if (t >= 0.0 && (!have || t < best)) {
                best = t;
                *out = p;
                have = true;
            }
        }
    }
    return have ? SGEMM_OK : SGEMM_ERR_CONFIG;
}

int make_plan(const PlanRequest &req, Plan *out) {
    const int M = req.M, N = req.N, K = req.K;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_SHAPE;
    if (req.config < 0 || req.config >= kNumCfgs) return SGEMM_ERR_CONFIG;
    if (req.sched < SGEMM_SCHED_AUTO || req.sched > SGEMM_SCHED_FIXED) return SGEMM_ERR_CONFIG;
    if (req.sched == SGEMM_SCHED_FIXED) return plan_fixed(req, out);
    const int cus = req.num_cus > 0 ? req.num_cus : 1;

    int cfg = req.config;
    if (cfg == SGEMM_CFG_AUTO) {
        cfg = auto_config(req, req.aligned != 0);
        if (cfg == kTiledChoice) return plan_by_cost(req, cus, out);
    }
    const CfgInfo &c = kCfgs[cfg];
    if (c.kind == kKindSkinny) return plan_skinny(req, cus, out);
    if (c.kind == kKindRowdot) return plan_rowdot(req, cus, occ_of(req, cfg), out);
    return plan_tiled(req, cfg, req.sched, cus, out);
}

}  // namespace sgemm
