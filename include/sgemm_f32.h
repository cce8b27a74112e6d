/*
 * sgemm_f32: single-precision GEMM for AMD Instinct MI355X (gfx950):
 * C = A * B (sgemm_f32) and C = alpha * op(A) * op(B) + beta * C
 * (sgemm_f32_gemm).
 *
 * The operation (page "Beyond Kernel 7: Closing the Gap to cuBLAS on an H100
 * FP32 GEMM", section "The operation: GEMM and the precision of the
 * comparison"): for row-major FP32 matrices A (M x K) and B (K x N),
 *
 *     C[m][n] = sum over k of A[m][k] * B[k][n]
 *
 * with FP32 inputs and FP32 arithmetic throughout (fused multiply-adds, one
 * rounding each; no reduced-precision input rounding of any kind).  Any
 * shape is accepted: that page restricts itself to multiples of the tile;
 * ragged edges are handled as the pages "Vectorized Memory Access: Pushing
 * CUDA SGEMM to 29 TFLOPS on H100" and "2D Block Tiling: Scaling Matrix
 * Multiplication on NVIDIA H100" describe in their sections 5: values
 * beyond the matrix read as zero, results beyond it are not written.
 *
 * Fast and general layouts
 *   When the stored row lengths of A and B (K and N for sgemm_f32) and N
 *   are multiples of 4, lda, ldb and ldc are multiples of 4 and A, B, C are
 *   16-byte aligned, the 16-byte vector kernels run (tile edges masked
 *   where the shape is not a multiple of the tile).  Any other layout runs
 *   on a general kernel with element-wise bounds checks, except that with
 *   the automatic configuration and M * N * K at least 2^25,
 *   A and B are first copied on `stream` into zero-padded aligned buffers
 *   of the library (each only when its own layout does not qualify) and the
 *   product runs on the vector kernels, which then write C in place (one
 *   float at a time when C's layout does not qualify; results as unpadded,
 *   C's padding untouched).  Thin products have kernels of their own that
 *   take any layout: at most 16 rows with B stored K x N
 *   (SGEMM_CFG_SKINNY_16x256); at most 8 rows with B stored N x K (as in
 *   x W^T with W row-major) run transposed, C^T = B A^T, on the row-dot
 *   kernel, and at most 16 columns with A stored K x M (as in X^T v) on the
 *   skinny kernel, each when that kernel would take the transposed shape;
 *   at most 2 columns, or 8 for large A or a
 *   layout the tiled kernels cannot load, with A stored M x K
 *   (SGEMM_CFG_ROWDOT_N8).
 *
 * Memory and ownership
 *   A, B, C are device pointers, caller-owned, allocated on the HIP device
 *   that is current when the call is made.  The library never frees or keeps
 *   them.  Layout is row-major with leading dimensions:
 *       A[m * lda + k],  B[k * ldb + n],  C[m * ldc + n].
 *   Only the logical M x N region of C is written; the ldc padding is left
 *   untouched.  sgemm_f32 overwrites C without reading it (sgemm_f32_gemm
 *   reads it when beta != 0).  C must not overlap A or B.
 *
 * Asynchrony
 *   Every call only enqueues work on `stream` (0 = the null stream) and
 *   returns without synchronising the host.  Faults during execution surface
 *   at the caller's next synchronisation, as usual for HIP.
 *
 * Errors
 *   Arguments are fully checked before anything is enqueued, so on any error
 *   C is untouched.  Return values are the SGEMM_* status codes below.
 *
 * Workspace
 *   Split-K ("Stream-K") schedules keep partial tiles in a workspace owned
 *   by the library, one per (device, stream), grown on demand with
 *   hipMalloc and kept until sgemm_f32_release() or process exit; a second
 *   kernel, enqueued on the same stream right after the GEMM kernel, adds
 *   them into C.  Repacked calls (see above) keep their copies in a buffer
 *   of the same (device, stream), held and freed the same way.  Calls on
 *   different streams therefore never share one.
 *   Calls that run concurrently on the SAME stream are impossible by stream
 *   order; calls from several host threads on one stream are serialised by
 *   the stream as well.
 *
 * Graph capture
 *   A call only enqueues kernels (no memset, no copy), so it can be captured
 *   into a HIP graph, provided it allocates nothing during capture: make one
 *   eager call with the same stream and a shape at least as large first (the
 *   Stream-K workspace and the repacking buffer are then in place; aligned
 *   shapes that run whole tiles need neither).  Replays use the workspace the capturing stream had at capture
 *   time: replays of graphs captured on one stream must not run
 *   concurrently, and a later call on that stream that needs a larger
 *   workspace (it replaces the buffers) or sgemm_f32_release() invalidates
 *   those graphs — size the workspace with the largest shape before
 *   capturing.  sgemm_f32_gemm_noalloc (below) needs no eager call: it
 *   never allocates.
 *
 * Environment (read on every call; for tuning and measurement, not needed
 * for correct results):
 *   SGEMM_F32_SK_WG_PER_CU  split workgroups per compute unit in Stream-K
 *                           schedules (default 1, capped by occupancy);
 *   SGEMM_F32_XCD_REMAP     0 turns off the remapping of workgroup ids that
 *                           gives each XCD a contiguous run of tiles;
 *   SGEMM_F32_GROUP_M       tile rows per group of the tile order (default:
 *                           chosen by the planner);
 *   SGEMM_F32_REPACK_MIN_MACS  products of at least this many multiply-adds
 *                           whose layout the vector kernels cannot load are
 *                           run on aligned copies (default 2^25; -1: never).
 */
#ifndef SGEMM_F32_H
#define SGEMM_F32_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SGEMM_OK            0  /* success (also for M == 0 or N == 0: nothing to do) */
#define SGEMM_ERR_SHAPE     1  /* M, N or K negative */
#define SGEMM_ERR_LD        2  /* lda < K, ldb < N or ldc < N */
#define SGEMM_ERR_ALIGN     3  /* a pointer not aligned to a float (4 bytes) */
#define SGEMM_ERR_NULL      4  /* a required pointer is NULL */
#define SGEMM_ERR_ALIAS     5  /* the C region overlaps the A or B region */
#define SGEMM_ERR_HIP       6  /* a HIP runtime call failed: see sgemm_f32_last_hip_error() */
#define SGEMM_ERR_POINTER   7  /* a pointer is not device memory of the current device, or
                                  the matrix extent runs past the end of its allocation */
#define SGEMM_ERR_CONFIG    8  /* unknown kernel configuration/schedule, or a forced one that
                                  cannot run this shape or layout */
#define SGEMM_ERR_SCRATCH   9  /* sgemm_f32_gemm_noalloc: the scratch the call needs (repacked
                                  copies, or split partials of a kernel that cannot run
                                  unsplit) exceeds SGEMM_F32_NOALLOC_SCRATCH_BYTES */

/* Kernel configurations (sgemm_f32_ex / sgemm_f32_plan).  "MFMA" configs
 * run the product on the FP32 matrix cores (v_mfma_f32_32x32x2_f32: full
 * FP32 inputs, FP32 accumulation); the "VALU" config runs it as a
 * register-tiled outer product of scalar FP32 fused multiply-adds. */
#define SGEMM_CFG_AUTO              0
#define SGEMM_CFG_MFMA_256x256x16   1  /* 512 threads, 8 waves of 64x128 */
#define SGEMM_CFG_MFMA_128x128x32   2  /* 256 threads, 4 waves of 64x64  */
#define SGEMM_CFG_MFMA_256x256x32   3  /* 256 threads, 4 waves of 128x128 */
#define SGEMM_CFG_MFMA_256x128x32   4  /* 256 threads, 4 waves of 128x64 */
#define SGEMM_CFG_VALU_128x128x8    5  /* 256 threads, 8x8 outputs per lane */
#define SGEMM_CFG_MFMA_256x256x32_W8 6 /* 512 threads, 8 waves of 64x128 */
#define SGEMM_CFG_MFMA_128x128x32_W8 7 /* 512 threads, 8 waves of 32x64 */
#define SGEMM_CFG_MFMA_64x64x32     8  /* 256 threads, 4 waves of 32x32 */
#define SGEMM_CFG_MFMA_128x64x32    9  /* 256 threads, 4 waves of 64x32 */
#define SGEMM_CFG_MFMA_64x64x64     10 /* 256 threads, 4 waves of 32x32 */
#define SGEMM_CFG_MFMA_128x128x64   11 /* 256 threads, 4 waves of 64x64 */
#define SGEMM_CFG_MFMA_64x64x128    12 /* 256 threads, 4 waves of 32x32 */
/* Tiles loaded straight from global memory into LDS (no register staging),
 * with a ring of LDS stages; _k2: two groups of waves split each chunk's K
 * range (two waves per SIMD with one tile per CU).  DL_64x64x32,
 * DL_64x64x64, DL_128x128x32 and DL_256x256x16 also run shapes their tile
 * does not divide and A / B in either storage order (sgemm_f32_gemm), when
 * the stored row lengths of A and B, N and every leading dimension are
 * multiples of 4 and A, B, C are 16-byte aligned.  The automatic choice
 * (SGEMM_CFG_AUTO) uses these four (the one, and the schedule, of least
 * modelled time), the skinny and row-dot kernels for thin products, and the
 * general kernel. */
#define SGEMM_CFG_DL_64x64x32       13 /* 256 threads, 4 waves of 32x32, 4 stages */
#define SGEMM_CFG_DL_64x64x64_K2    14 /* 512 threads, 2 x 4 waves of 32x32, 3 stages */
#define SGEMM_CFG_DL_128x128x32     15 /* 512 threads, 4 waves of 64x64 and 4 that load, 3 stages */
#define SGEMM_CFG_DL_256x256x16     16 /* 512 threads, 8 waves of 64x128, 3 stages */
#define SGEMM_CFG_DL_64x64x32_K2    17 /* 512 threads, 2 x 4 waves of 32x32, 4 stages */
#define SGEMM_CFG_DL_128x128x32_K2  18 /* 512 threads, 2 x 4 waves of 64x64, 3 stages */
#define SGEMM_CFG_DL_64x64x64       19 /* 256 threads, 4 waves of 32x32, 3 stages */
#define SGEMM_CFG_DL_128x256x16     20 /* 256 threads, 4 waves of 64x128, 3 stages */
#define SGEMM_CFG_DL_256x128x16     21 /* 256 threads, 4 waves of 128x64, 3 stages */
/* Element-wise bounds-checked loads: any shape, leading dimension and
 * (4-byte) alignment. */
#define SGEMM_CFG_GENERIC_64x64x16  22 /* 256 threads, 4 waves of 32x32 */
/* At most 16 rows (M <= 16), B stored K x N (any layout; 16-byte loads
 * where B's rows and N are on the 16-byte grid): multiply-adds over the M
 * rows only (vector ALU up to 8 rows, 16 x 16 x 4 matrix-core steps for
 * 9-16), B streamed once, K split over the grid.  The automatic choice
 * takes it for such products with N, K >= 256 (for M > 8: and N * K > 2^22,
 * or a layout the tiled kernels cannot load). */
#define SGEMM_CFG_SKINNY_16x256     23 /* 512 threads, 8 waves over 256 columns */
/* At most 8 columns (N <= 8, y = A x among them), A stored M x K (any
 * layout; 16-byte loads where A's rows are on the 16-byte grid): per-row
 * dot products, A streamed once, B held in LDS.  The automatic choice takes
 * it for such products with M, K >= 256 and N <= 2, or N <= 8 once
 * M * K >= 2^26 or when the layout rules out the tiled kernels. */
#define SGEMM_CFG_ROWDOT_N8         24 /* 512 threads, 8 waves over rows of A */
/* The register-tiled outer product of scalar FP32 fused multiply-adds with a
 * 16 x 8 tile per lane (0.75 bytes of LDS operands per multiply-add) and the
 * next k step's operands read during the current one. */
#define SGEMM_CFG_VALU_256x128x8    25 /* 256 threads, 16x8 outputs per lane */
#define SGEMM_NUM_CFGS              26 /* configurations are 1 .. SGEMM_NUM_CFGS-1 */
/* The configurations not named above as running other shapes or storage
 * orders need A stored M x K, B stored K x N, the vector layout and a shape
 * their tile divides. */

/* Schedules. */
#define SGEMM_SCHED_AUTO     0  /* the planner's: data-parallel, or whole tiles in full waves and the rest split */
#define SGEMM_SCHED_DP       1  /* one workgroup per output tile, full K each */
#define SGEMM_SCHED_STREAMK  2  /* every tile's K range split evenly over a resident grid */
/* Data-parallel, on the automatic configuration's kernel compiled for this
 * exact product (every size, leading dimension and the tile order fixed at
 * compile time; "Beyond Kernel 7: Closing the Gap to cuBLAS on an H100 FP32
 * GEMM", section "Kernel 13", the size-specialised build).  Compiled for
 * M x N x K = 4096^3, 2048^3, 1024^3 and 1024 x 1024 x 16384, with lda = K,
 * ldb = ldc = N, 16-byte aligned A, B, C and the plain product (sgemm_f32,
 * or sgemm_f32_gemm with alpha = 1, beta = 0, no transposes); anything else
 * returns SGEMM_ERR_CONFIG.  Results are those of SGEMM_SCHED_DP bit for
 * bit (same kernel body, same summation order). */
#define SGEMM_SCHED_FIXED    3

/*
 * C = A * B.  Requirements: M, N, K >= 0; lda >= K, ldb >= N, ldc >= N;
 * A, B, C device pointers aligned to a float.  K == 0 writes zeros to C (the
 * empty sum); A, B, lda and ldb are then not used or checked.  Returns an
 * SGEMM_* status code.
 */
int sgemm_f32(int M, int N, int K,
              const float *A, int lda,
              const float *B, int ldb,
              float *C, int ldc,
              hipStream_t stream);

/*
 * As sgemm_f32, with the kernel configuration and schedule forced (for
 * tests and benchmarks).  config = SGEMM_CFG_*, sched = SGEMM_SCHED_*;
 * SGEMM_CFG_AUTO / SGEMM_SCHED_AUTO select as sgemm_f32 does.  Returns
 * SGEMM_ERR_CONFIG if the forced configuration cannot run this shape.
 */
int sgemm_f32_ex(int M, int N, int K,
                 const float *A, int lda,
                 const float *B, int ldb,
                 float *C, int ldc,
                 hipStream_t stream, int config, int sched);

/*
 * General matrix multiply in the BLAS form, row-major:
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * op(A) is M x K: A stored M x K (A[m * lda + k], lda >= K) when trans_a
 * is 0, or stored K x M (A[k * lda + m], lda >= M) when trans_a is 1, so
 * that op(A) = A^T; likewise op(B) is K x N: B stored K x N (ldb >= N) or,
 * with trans_b = 1, N x K (B[n * ldb + k], ldb >= K).  C is M x N, ldc >= N.
 * The kernels of "Vectorized Memory Access: Pushing CUDA SGEMM to 29 TFLOPS
 * on H100" and "2D Block Tiling: Scaling Matrix Multiplication on NVIDIA
 * H100" take the same alpha and beta (their sections 5 show the scaled
 * store); sgemm_f32 is the alpha = 1, beta = 0, untransposed case.
 *
 * Conventions (as in BLAS): beta == 0 means C is not read (it may hold
 * anything); alpha == 0 or K == 0 means A and B are not read (they and
 * their leading dimensions are then not checked) and C = beta * C.  The
 * sum is computed once and scaled once per element; with Stream-K the
 * partial sums are combined first.  Accepts every shape and layout; the
 * 16-byte vector kernels need the contiguous extent (K or M of A, N or K
 * of B, N of C) and every leading dimension to be multiples of 4 and the
 * operands 16-byte aligned, else the general kernel runs.  trans_a or
 * trans_b outside {0, 1}: SGEMM_ERR_CONFIG.  Other errors as sgemm_f32.
 */
int sgemm_f32_gemm(int trans_a, int trans_b, int M, int N, int K, float alpha,
                   const float *A, int lda,
                   const float *B, int ldb, float beta,
                   float *C, int ldc,
                   hipStream_t stream);

/* sgemm_f32_gemm with the configuration and schedule forced (tests and
 * benchmarks), as sgemm_f32_ex. */
int sgemm_f32_gemm_ex(int trans_a, int trans_b, int M, int N, int K, float alpha,
                      const float *A, int lda,
                      const float *B, int ldb, float beta,
                      float *C, int ldc,
                      hipStream_t stream, int config, int sched);

/*
 * sgemm_f32_gemm that allocates no memory, for callers that cannot call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and errors as
 * sgemm_f32_gemm (automatic configuration and schedule), except where
 * sgemm_f32_gemm would take device memory:
 *   - Stream-K partial tiles and repacked copies of A and B (see "Fast and
 *     general layouts") go to a fixed scratch array of
 *     SGEMM_F32_NOALLOC_SCRATCH_BYTES in the library's code object, one per
 *     device, held from the library's load on that device until the process
 *     ends (its address is looked up on the first call on each device);
 *   - a split schedule whose partial tiles do not fit (or do not fit beside
 *     the repacked copies) runs data-parallel instead: whole tiles, no
 *     partials (results within the same tolerance; exact on integer inputs);
 *     where the kernel cannot run unsplit (the row-dot kernel when B's K
 *     range exceeds its LDS), the call is refused with SGEMM_ERR_SCRATCH;
 *   - repacked copies that do not fit the array are refused with
 *     SGEMM_ERR_SCRATCH, both before anything is enqueued.
 * Nothing needs clearing between calls: every partial tile and every padded
 * copy is written in full before it is read.  Every call on a device shares
 * that device's array and leaves its contents behind: calls on one stream
 * are ordered by the stream (also from several host threads), but calls
 * whose execution overlaps on one GPU (on different streams, or graphs
 * replayed concurrently) race on the array and give wrong results.
 */
#define SGEMM_F32_NOALLOC_SCRATCH_BYTES (64LL << 20)   /* 64 MiB per device */
int sgemm_f32_gemm_noalloc(int trans_a, int trans_b, int M, int N, int K, float alpha,
                           const float *A, int lda,
                           const float *B, int ldb, float beta,
                           float *C, int ldc,
                           hipStream_t stream);

/* Shape multiples accepted by sgemm_f32: 1, 1, 1 (any shape; any pointer
 * may be NULL). */
void sgemm_f32_granule(int *gm, int *gn, int *gk);

/* Human-readable text for a status code (static storage, never NULL). */
const char *sgemm_f32_status_string(int status);

/* hipError_t of the most recent SGEMM_ERR_HIP in the calling thread (0 if none). */
int sgemm_f32_last_hip_error(void);

/*
 * The launch plan the library would use, computed on the host only (no HIP
 * call): which configuration, the tile, the grid, how many tiles are done
 * whole and how many are split, and the workspace size.  num_cus is the
 * compute-unit count; occupancy[c] is the number of workgroups of
 * configuration c that fit on one compute unit (NULL: the library's
 * built-in figures); sk_wg_per_cu is the number of split workgroups per CU
 * (0: the library's default, one), capped by the occupancy.  The plan
 * assumes dense operands (lda = K, ldb = ldc = N) on 16-byte boundaries;
 * where such a call would run on repacked copies (see "Fast and general
 * layouts"), it is the plan of the padded product and `repacked` is 1.
 * Returns an SGEMM_* status code; *out is filled on success.
 */
typedef struct sgemm_f32_plan_t {
    int config;          /* SGEMM_CFG_* chosen */
    int sched;           /* SGEMM_SCHED_DP or SGEMM_SCHED_STREAMK (DP+split mix reports STREAMK) */
    int tile_m, tile_n, tile_k;
    int threads;         /* threads per workgroup */
    int tiles_m, tiles_n;
    int iters_per_tile;  /* K chunks per tile: ceil(K / tile_k) */
    int dp_tiles;        /* tiles computed whole, first in tile order */
    int sk_tiles;        /* remaining tiles, K-split over the grid */
    int grid;            /* workgroups launched */
    int sk_grid;         /* logical workgroups 0 .. sk_grid-1 share the split tiles */
    int xcd_remap;       /* 1: workgroup ids are remapped so each XCD gets a contiguous run */
    int group_m;         /* tile order: groups of group_m tile rows, column-major inside */
    long long sk_iters;  /* sk_tiles * iters_per_tile */
    long long workspace_bytes;
    int repacked;        /* 1: A and B are first copied to padded buffers; the
                            fields above describe the padded product */
    int transposed;      /* 1: the product runs transposed, C^T = op(B)^T op(A)^T
                            (few rows with B stored N x K on the row-dot
                            kernel, few columns with A stored K x M on the
                            skinny kernel); the fields above describe it */
    int fixed_shape;     /* 1: SGEMM_SCHED_FIXED, the kernel compiled for this product */
    double model_us;     /* the planner's modelled kernel time (microseconds) of this plan,
                            by which the automatic choice ranks the direct-to-LDS
                            configurations DL_64x64x32, DL_64x64x64, DL_128x128x32
                            and DL_256x256x16 and their schedules; -1 for any other
                            configuration */
} sgemm_f32_plan_t;

int sgemm_f32_plan(int M, int N, int K, int config, int sched, int num_cus,
                   const int *occupancy, int sk_wg_per_cu, sgemm_f32_plan_t *out);

/* sgemm_f32_plan for the BLAS form (sgemm_f32_gemm) with A and B in the
 * storage orders trans_a / trans_b (0 or 1, as there), dense operands (each
 * leading dimension equal to its stored row length) on 16-byte boundaries.
 * SGEMM_ERR_CONFIG for a transpose flag outside {0, 1}. */
int sgemm_f32_gemm_plan(int trans_a, int trans_b, int M, int N, int K, int config, int sched,
                        int num_cus, const int *occupancy, int sk_wg_per_cu,
                        sgemm_f32_plan_t *out);

/*
 * Free every workspace the library holds (all devices, all streams).  The
 * caller must ensure no sgemm call is still executing.  Returns SGEMM_OK or
 * SGEMM_ERR_HIP.
 */
int sgemm_f32_release(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_H */
