// Host-callable launchers of the GEMM kernels (one per source file).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "sgemm_f32.h"

namespace sgemm {

struct KernelArgs;

hipError_t launch_mfma(int cfg, const KernelArgs &a, hipStream_t s);
hipError_t occupancy_mfma(int cfg, int *wg_per_cu);
hipError_t launch_mfma_dl(int cfg, const KernelArgs &a, hipStream_t s);
hipError_t occupancy_mfma_dl(int cfg, int *wg_per_cu);
// The direct-to-LDS kernel compiled for the product kFixedShapes[idx].
hipError_t launch_mfma_dl_fixed(int idx, const KernelArgs &a, hipStream_t s);
hipError_t launch_generic(int cfg, const KernelArgs &a, hipStream_t s);
hipError_t occupancy_generic(int cfg, int *wg_per_cu);
hipError_t launch_valu(int cfg, const KernelArgs &a, hipStream_t s);
// The skinny kernel (M <= 16) and, for a K-split plan, the sum of its splits.
// trans_c: C stored N x M, element (m, n) at C[n * ldc + m] (the transposed
// product of a call with few columns and A stored K x M).
hipError_t launch_skinny(int cfg, const KernelArgs &a, hipStream_t s, int trans_c = 0);
hipError_t occupancy_skinny(int cfg, int *wg_per_cu);
// The row-dot kernel (N <= 8) and, for a K-split plan, the sum of its splits.
// trans_c: C stored N x M, element (m, n) at C[n * ldc + m] (the transposed
// product of a call with few rows and B stored N x K).
hipError_t launch_rowdot(int cfg, const KernelArgs &a, hipStream_t s, int trans_c = 0);
hipError_t occupancy_rowdot(int cfg, int *wg_per_cu);
hipError_t occupancy_valu(int cfg, int *wg_per_cu);
// Sum of the split tiles of a Stream-K launch (tile bm x bn) into C; after
// the GEMM kernel on the same stream.
hipError_t launch_sk_fixup(const KernelArgs &a, int bm, int bn, hipStream_t s);
hipError_t launch_scale_c(float *C, int M, int N, int64_t ldc, float beta, hipStream_t s);
// One copy of a repacking launch: dst (drows x dcols, leading dimension
// ldd) = src (rows x cols, leading dimension lds) with zeros outside it.
struct PackJob {
    const float *src;
    int64_t lds;
    int rows, cols;
    float *dst;
    int64_t ldd;
    int drows, dcols;
};
// Up to two copies in one launch (jobs with no rows or columns skipped).
hipError_t launch_pack(const PackJob *jobs, int njobs, hipStream_t s);

}  // namespace sgemm
