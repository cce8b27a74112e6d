// Repacking of operands whose layout the 16-byte direct-to-LDS kernels
// cannot load (a pointer off a 16-byte boundary, a leading dimension or a
// stored row length not a multiple of 4): a plain 2-D copy into a padded,
// aligned buffer, zeros in the padding.  HBM-bound: each element is read
// once and written once, lanes along the contiguous dimension.  One launch
// copies up to two operands (grid z selects the job).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace sgemm {

namespace {

constexpr int kRowsPerThread = 4;

// dst[r * ldd + c] for r < drows, c < dcols: src[r * lds + c] inside
// rows x cols, zero outside.  Block (x, y) covers columns [256 x, 256 x +
// 256) and rows [4 y', 4 y' + 4) for y' = y, y + gridDim.y, ...; each thread
// one column of those rows, all four loads issued before the stores.
__device__ __forceinline__ void pack_job(const PackJob &j) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= j.dcols) return;
    const bool col_in = c < j.cols;
    for (int r0 = blockIdx.y * kRowsPerThread; r0 < j.drows; r0 += gridDim.y * kRowsPerThread) {
        float v[kRowsPerThread];
#pragma unroll
        for (int u = 0; u < kRowsPerThread; ++u) {
            const int r = r0 + u;
            v[u] = (col_in && r < j.rows) ? j.src[(int64_t)r * j.lds + c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kRowsPerThread; ++u)
            if (r0 + u < j.drows) j.dst[(int64_t)(r0 + u) * j.ldd + c] = v[u];
    }
}

__global__ __launch_bounds__(256) void sgemm_pack_kernel(PackJob j0, PackJob j1) {
    pack_job(blockIdx.z == 0 ? j0 : j1);
}

}  // namespace

hipError_t launch_pack(const PackJob *jobs, int njobs, hipStream_t s) {
    PackJob j[2] = {};
    int n = 0, gx = 0, gy = 0;
    for (int i = 0; i < njobs && n < 2; ++i) {
        if (jobs[i].drows <= 0 || jobs[i].dcols <= 0) continue;
        j[n++] = jobs[i];
        const int x = (jobs[i].dcols + 255) / 256;
        const int y = (jobs[i].drows + kRowsPerThread - 1) / kRowsPerThread;
        gx = x > gx ? x : gx;
        gy = y > gy ? y : gy;
    }
    if (n == 0) return hipSuccess;
    if (gy > 1024) gy = 1024;   // the kernel strides over the rest
    void *params[] = {&j[0], &j[1]};
    return hipLaunchKernel((const void *)sgemm_pack_kernel, dim3(gx, gy, n), dim3(256), params, 0, s);
}

}  // namespace sgemm
