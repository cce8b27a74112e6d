// FP32 GEMM on the vector ALUs: a register-tiled outer product of scalar
// fused multiply-adds (v_fma_f32), one rounding per multiply-add.
//
// Geometry after "Vectorized Memory Access: Pushing CUDA SGEMM to 29 TFLOPS
// on H100" (sections 2-4: a 128x128 output tile, K chunks of 8, 256 threads
// with 8x8 outputs each, one 128-bit load of A and one of B per thread per
// chunk, A stored transposed in shared memory) and "2D Block Tiling" (section
// 1 and 4: the 8x8 register outer product, 16 operand reads per 64
// multiply-adds), re-laid for 64-wide waves:
//   * each lane's 8 rows are two runs of 4 (ty*4 and 64 + ty*4) and its 8
//     columns likewise (tx*4 and 64 + tx*4), so every LDS operand read is one
//     ds_read_b128: the 16 lanes of a row read 256 contiguous bytes of B and
//     the four distinct A addresses of a wave are broadcasts;
//   * two LDS stages (ping-pong) with the next chunk's global loads in
//     registers while the current chunk is multiplied, one barrier per chunk;
//   * C is written as float4s, 16 lanes covering 256 contiguous bytes of a
//     row.
#include "gemm_common.h"
#include "kernels.h"

namespace sgemm {

struct Valu128x128x8 {
    static constexpr int BM = 128, BN = 128, BK = 8;
    static constexpr int NT = 256;
    static constexpr int LDT = BM + 4;           // LDS row stride of A^T (k rows)
    static constexpr int LDB_S = BN + 4;         // LDS row stride of B (k rows)
    static constexpr int A_STAGE = BK * LDT;
    static constexpr int STAGE = A_STAGE + BK * LDB_S;
    static constexpr int LDS_FLOATS = 2 * STAGE;
    static constexpr int TILE_FLOATS = BM * BN;

    float acc[8][8];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    }

    __device__ __forceinline__ void mainloop(const KernelArgs &a, float *lds, int tm, int tn,
                                             int k0, int k1) {
        const int tid = threadIdx.x;
        // One float4 of A (row tid/2, k 4*(tid%2)) and one of B (k row tid/32,
        // columns 4*(tid%32)) per chunk.
        const int a_row = tid >> 1, a_c4 = tid & 1;
        const int b_row = tid >> 5, b_c4 = tid & 31;
        const float *ga = a.A + ((int64_t)tm * BM + a_row) * a.lda + (int64_t)k0 * BK + a_c4 * 4;
        const float *gb = a.B + ((int64_t)k0 * BK + b_row) * a.ldb + (int64_t)tn * BN + b_c4 * 4;
        const int64_t gb_chunk = (int64_t)BK * a.ldb;
        const int sa = (a_c4 * 4) * LDT + a_row;
        const int sb = A_STAGE + b_row * LDB_S + b_c4 * 4;
        const int tx = tid & 15, ty = tid >> 4;

        f32x4 ra, rb;
        auto load_global = [&]() {
            ra = *(const f32x4 *)ga;
            rb = *(const f32x4 *)gb;
        };
        auto store_lds = [&](int stage) {
            float *s = lds + stage * STAGE;
            s[sa + 0 * LDT] = ra.x;        // A stored transposed: [k][m]
            s[sa + 1 * LDT] = ra.y;
            s[sa + 2 * LDT] = ra.z;
            s[sa + 3 * LDT] = ra.w;
            *(f32x4 *)(s + sb) = rb;
        };
        auto compute = [&](int stage) {
            const float *s = lds + stage * STAGE;
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                const f32x4 a0 = *(const f32x4 *)(s + k * LDT + ty * 4);
                const f32x4 a1 = *(const f32x4 *)(s + k * LDT + 64 + ty * 4);
                const f32x4 b0 = *(const f32x4 *)(s + A_STAGE + k * LDB_S + tx * 4);
                const f32x4 b1 = *(const f32x4 *)(s + A_STAGE + k * LDB_S + 64 + tx * 4);
                const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
            }
        };

        const int nch = k1 - k0;
        load_global();
        __syncthreads();
        store_lds(0);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            const int cur = c & 1;
            const bool more = c + 1 < nch;
            if (more) {
                ga += BK;
                gb += gb_chunk;
                load_global();
            }
            compute(cur);
            if (more) store_lds(cur ^ 1);
            __syncthreads();
        }
    }

    // Output row of accumulator row i: ty*4 + i (i < 4) or 64 + ty*4 + i-4;
    // output column of j: tx*4 + j (j < 4) or 64 + tx*4 + j-4.
    __device__ __forceinline__ void store_c(const KernelArgs &a, int tm, int tn) {
        const int tid = threadIdx.x;
        const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = tm * BM + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
            float *c = a.C + (int64_t)row * a.ldc + (int64_t)tn * BN + tx * 4;
            *(f32x4 *)c = epilogue(a, f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]}, c);
            *(f32x4 *)(c + 64) = epilogue(a, f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]}, c + 64);
        }
    }

    // The same mapping into a dense row-major BM x BN tile (a split tile's
    // partial sum).
    __device__ __forceinline__ void store_tile(float *p) {
        const int tid = threadIdx.x;
        const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float *q = p + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4)) * BN + tx * 4;
            *(f32x4 *)q = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
            *(f32x4 *)(q + 64) = f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
        }
    }
};

template <bool SPLIT>
__global__ __launch_bounds__(Valu128x128x8::NT) void sgemm_valu_kernel(KernelArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[Valu128x128x8::LDS_FLOATS];
    run_gemm<Valu128x128x8, SPLIT>(a, lds);
}

hipError_t launch_valu(int cfg, const KernelArgs &a, hipStream_t s) {
    if (cfg != SGEMM_CFG_VALU_128x128x8) return hipErrorInvalidValue;
    KernelArgs args = a;
    void *params[] = {&args};
    const void *f = a.sk_tiles > 0 ? (const void *)sgemm_valu_kernel<true>
                                   : (const void *)sgemm_valu_kernel<false>;
    return hipLaunchKernel(f, dim3(a.grid), dim3(Valu128x128x8::NT), params, 0, s);
}

hipError_t occupancy_valu(int cfg, int *wg_per_cu) {
    if (cfg != SGEMM_CFG_VALU_128x128x8) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        wg_per_cu, (const void *)sgemm_valu_kernel<true>, Valu128x128x8::NT, 0);
}

// C := 0 over the logical M x N region (the empty sum, K == 0).
// C = beta * C over the M x N region (the product is empty, K == 0, or
// scaled by alpha == 0); beta == 0 writes zeros without reading C.
__global__ void sgemm_scale_c_kernel(float *C, int M, int N, int64_t ldc, float beta) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / N, c = i - r * N;
        float *p = C + r * ldc + c;
        *p = beta == 0.0f ? 0.0f : beta * *p;
    }
}

hipError_t launch_scale_c(float *C, int M, int N, int64_t ldc, float beta, hipStream_t s) {
    int64_t total = (int64_t)M * N;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) return hipSuccess;
    void *params[] = {&C, &M, &N, &ldc, &beta};
    return hipLaunchKernel((const void *)sgemm_scale_c_kernel, dim3(blocks), dim3(256), params, 0, s);
}

}  // namespace sgemm
