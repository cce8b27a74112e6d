// Host-side launch planning for sgemm_f32: configuration choice, tile grid,
// and the data-parallel / Stream-K split.  Pure C++ with no HIP dependency so
// that it runs (and is tested) on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

namespace sgemm {

enum CfgKind {
    kKindValu = 0,      // scalar VALU FMAs
    kKindMfma = 1,      // matrix cores, tiles staged through registers
    kKindMfmaDl = 2,    // matrix cores, tiles loaded straight into LDS
    kKindGeneric = 3,   // matrix cores, element-wise bounds-checked loads (any shape/alignment)
    kKindSkinny = 4,    // scalar VALU FMAs over the M <= 16 rows only, B streamed
    kKindRowdot = 5,    // per-row dot products for N <= 8 columns, A streamed
};

// K values of A staged in LDS at a time by the skinny kernel.
constexpr int kSkinnyBlock = 512;

// The row-dot kernel (N <= 8): floats of B held in LDS per workgroup
// (64 KiB), for its columns rounded up to 1, 2, 4 or 8, and the k of one K
// split (rounded up to a multiple of 4, so splits start on 16-byte
// boundaries of A's rows).
constexpr int kRowdotFloats = 16384;
inline int rowdot_cols(int N) { return N <= 2 ? (N < 1 ? 1 : N) : N <= 4 ? 4 : 8; }
inline int rowdot_k_per(int K, int splits) { return ((K + splits - 1) / splits + 3) & ~3; }

struct CfgInfo {
    int id;
    int bm, bn, bk;     // output tile and K chunk
    int threads;        // threads per workgroup
    int kind;           // CfgKind: which kernel family runs it
    int default_occ;    // workgroups per CU expected from its LDS/VGPR use
    bool edge;          // runs shapes that are not multiples of its tile
    bool layouts;       // runs transposed A and/or B (else only A M x K, B K x N)
    const char *name;
};

// Indexed by SGEMM_CFG_* (entry 0 is a placeholder for AUTO).
extern const CfgInfo kCfgs[];
extern const int kNumCfgs;

// Shape granule accepted by the library: every M, N, K >= 0 (ragged edges are
// masked; see make_plan).
constexpr int kGranM = 1, kGranN = 1, kGranK = 1;

// Smallest number of K chunks a Stream-K workgroup should own.
constexpr int kMinSkIters = 8;

struct PlanRequest {
    int M, N, K;
    int config;          // SGEMM_CFG_*
    int sched;           // SGEMM_SCHED_*
    int num_cus;
    const int *occupancy;  // [kNumCfgs] or nullptr
    int sk_wg_per_cu;    // Stream-K grid = num_cus * this (0: occupancy)
    int aligned;         // 16-byte aligned A, B, C; lda, ldb, ldc and the contiguous
                         // extents of A, B, C multiples of 4
    int trans_a = 0;     // A stored K x M
    int trans_b = 0;     // B stored N x K
};

struct Plan {
    int config, sched;
    int bm, bn, bk, threads;
    int tiles_m, tiles_n, ipt;
    int dp_tiles, sk_tiles, grid, sk_grid;
    int xcd_remap, group_m;
    int edge;            // the shape is not a multiple of the tile: masked loads and stores
    int64_t sk_iters;
    int64_t workspace_bytes;
    int fixed = 0;       // 1 + index into kFixedShapes: the kernel compiled for this product
};

// Products that have a kernel compiled for their exact shape
// (SGEMM_SCHED_FIXED): dense row-major A (M x K), B (K x N), C (M x N), the
// configuration and tile-row grouping the automatic choice gives them.  The
// instances in gemm_mfma_dl.hip follow this order.
struct FixedShapeInfo {
    int M, N, K;
    int config;
    int group_m;
};
extern const FixedShapeInfo kFixedShapes[];
extern const int kNumFixedShapes;

// Returns an SGEMM_* status; fills *out on success.
int make_plan(const PlanRequest &req, Plan *out);

// Modelled kernel time (microseconds) of a plan of a direct-to-LDS
// configuration that the automatic choice weighs (negative for any other),
// on `cus` compute units with `occ` workgroups of it resident per CU.
double plan_cost(const Plan &p, int M, int N, int cus, int occ);

// The configurations that load tiles straight into LDS address a lane's
// source as a 32-bit byte offset from the tile's first row (an operand stored
// k-contiguous: A M x K, B N x K) or the chunk's first k row (stored
// m/n-contiguous): they need BM * lda or BK * lda, and BK * ldb or BN * ldb,
// under 2^30 floats (2^29 for the edge-masking variants, whose offsets mark a
// masked lane with the top bit).
bool dl_offsets_fit(int cfg, bool edge, int64_t lda, int64_t ldb, bool trans_a = false, bool trans_b = false);

// The register-staged configuration with the same tile as `cfg` (itself
// for those).
int staged_equivalent(int cfg);

// Workspace of a Stream-K launch: sk_grid * 2 partial tiles of bm*bn floats
// (a split workgroup leaves a partial for at most two tiles: the first and
// the last it touches).
int64_t workspace_bytes(int grid, int sk_tiles, int bm, int bn);

}  // namespace sgemm
