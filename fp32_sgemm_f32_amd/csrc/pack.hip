// Repacking of operands whose layout the 16-byte direct-to-LDS kernels
// cannot load (a pointer off a 16-byte boundary, a leading dimension or a
// stored row length not a multiple of 4): a plain 2-D copy into a padded,
// aligned buffer, zeros in the padding, and the copy of the result back.
// HBM-bound: each element is read once and written once, lanes along the
// contiguous dimension.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace sgemm {

// dst[r * ldd + c] for r < drows, c < dcols: src[r * lds + c] inside
// rows x cols, zero outside.  Grid x walks columns in blocks of 256, grid y
// strides over rows.
__global__ __launch_bounds__(256) void sgemm_pack_kernel(const float *src, int64_t lds, int rows, int cols,
                                                         float *dst, int64_t ldd, int drows, int dcols) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= dcols) return;
    for (int r = blockIdx.y; r < drows; r += gridDim.y) {
        const float v = (r < rows && c < cols) ? src[(int64_t)r * lds + c] : 0.0f;
        dst[(int64_t)r * ldd + c] = v;
    }
}

hipError_t launch_pack(const float *src, int64_t lds, int rows, int cols, float *dst, int64_t ldd, int drows,
                       int dcols, hipStream_t s) {
    if (drows <= 0 || dcols <= 0) return hipSuccess;
    const int gx = (dcols + 255) / 256;
    const int gy = drows < 1024 ? drows : 1024;
    void *params[] = {&src, &lds, &rows, &cols, &dst, &ldd, &drows, &dcols};
    return hipLaunchKernel((const void *)sgemm_pack_kernel, dim3(gx, gy), dim3(256), params, 0, s);
}

}  // namespace sgemm
