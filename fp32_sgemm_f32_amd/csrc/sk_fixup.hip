// The second kernel of a Stream-K launch: the sum of the split tiles'
// partials, in a fixed contributor order, with the epilogue ("Beyond Kernel
// 7: Closing the Gap to cuBLAS on an H100 FP32 GEMM", section "Kernel 14 and
// Stream-K": the partial tiles of a split output tile are combined before
// the tile is written).  HBM-bound: each partial is read once, each output
// of a split tile written once.
#include "gemm_common.h"
#include "kernels.h"

namespace sgemm {

template <int BM, int BN>
__global__ __launch_bounds__(256) void sgemm_sk_fixup_kernel(KernelArgs a) {
    sk_fixup<BM, BN>(a);
}

template <int BM, int BN>
hipError_t launch_fixup_tile(const KernelArgs &a, hipStream_t s) {
    const int64_t threads = (int64_t)a.sk_tiles * (BM * BN / 4);
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;   // the kernel strides over the rest
    KernelArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel((const void *)sgemm_sk_fixup_kernel<BM, BN>, dim3((unsigned)blocks), dim3(256), params,
                           0, s);
}

hipError_t launch_sk_fixup(const KernelArgs &a, int bm, int bn, hipStream_t s) {
    if (a.sk_tiles <= 0) return hipSuccess;
#define SGEMM_FIXUP_TILE(M_, N_) \
    if (bm == M_ && bn == N_) return launch_fixup_tile<M_, N_>(a, s);
    SGEMM_FIXUP_TILE(64, 64)
    SGEMM_FIXUP_TILE(128, 64)
    SGEMM_FIXUP_TILE(64, 128)
    SGEMM_FIXUP_TILE(128, 128)
    SGEMM_FIXUP_TILE(256, 128)
    SGEMM_FIXUP_TILE(128, 256)
    SGEMM_FIXUP_TILE(256, 256)
#undef SGEMM_FIXUP_TILE
    return hipErrorInvalidValue;
}

}  // namespace sgemm
