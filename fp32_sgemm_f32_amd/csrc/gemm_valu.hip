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

// acc += a * b, one rounding, as v_fmac_f32 acc, b, a: a (the operand
// fixed along a row of accumulators) is the instruction's second source.
// Measured on MI355X with independent chains: when the accumulator and the
// second source lie in the same VGPR bank (register number mod 4) the
// multiply-adds run 27% slower (74 against 101 TFLOP/s); the first source
// may share the accumulator's bank at no cost.  Left to itself the compiler
// makes b the second source and allocates b_j and the accumulators of
// column j in the same bank, almost every multiply-add; with a there, at
// most 2 of a row's 8 accumulators can share a's bank.
__device__ __forceinline__ void fmac_rowwise(float &acc, float a, float b) {
    asm("v_fmac_f32 %0, %1, %2" : "+v"(acc) : "v"(b), "v"(a));
}

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
                    for (int j = 0; j < 8; ++j) fmac_rowwise(acc[i][j], av[i], bv[j]);
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
            *(f32x4 *)(c + 64) =
                epilogue(a, f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]}, c + 64);
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

// A 256 x 128 output tile, K chunks of 8, 256 threads with 16 x 8 outputs
// each ("Beyond Kernel 7", section "Kernel 11": the 16 x 8 register tile
// cut shared-memory loads threefold).  Per k step a lane reads 16 values of
// A and 8 of B for 128 multiply-adds: 0.75 bytes of LDS operands per
// multiply-add where the 8 x 8 tile above needs 1, which at the FP32 vector
// rate (128 multiply-adds per clock per CU) is the whole LDS bandwidth of
// 128 bytes per clock.  Register prefetch: the operands of step k+1 are read
// while step k's multiply-adds run (two operand register sets); the
// scheduler is held to that order, or it would read all eight steps at the
// start of the chunk (128 more VGPRs, half the waves).
//   * lane (tx, ty) of the 16 x 16 grid owns rows 64 q + 4 ty + i (q, i in
//     0..3) and columns 64 p + 4 tx + j (p in 0..1, j in 0..3): every operand
//     read is one ds_read_b128 (A: four addresses per wave, broadcast;
//     B: 256 contiguous bytes per 16 lanes);
//   * A is stored transposed ([k][m], rows padded by 4), B as is; two LDS
//     stages, the next chunk's global loads (two float4s of A, one of B per
//     thread) in registers while the current chunk is multiplied, one
//     barrier per chunk.
struct Valu256x128x8 {
    static constexpr int BM = 256, BN = 128, BK = 8;
    static constexpr int NT = 256;
    static constexpr int LDT = BM + 4;           // LDS row stride of A^T (k rows)
    static constexpr int LDB_S = BN + 4;         // LDS row stride of B (k rows)
    static constexpr int A_STAGE = BK * LDT;
    static constexpr int STAGE = A_STAGE + BK * LDB_S;
    static constexpr int LDS_FLOATS = 2 * STAGE;
    static constexpr int TILE_FLOATS = BM * BN;

    float acc[16][8];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    }

    __device__ __forceinline__ void mainloop(const KernelArgs &a, float *lds, int tm, int tn,
                                             int k0, int k1) {
        const int tid = threadIdx.x;
        // Per chunk: A rows tid/2 and 128 + tid/2, k 4*(tid%2); B k row tid/32,
        // columns 4*(tid%32).
        const int a_row = tid >> 1, a_c4 = tid & 1;
        const int b_row = tid >> 5, b_c4 = tid & 31;
        const float *ga = a.A + ((int64_t)tm * BM + a_row) * a.lda + (int64_t)k0 * BK + a_c4 * 4;
        const int64_t ga_half = (int64_t)128 * a.lda;
        const float *gb = a.B + ((int64_t)k0 * BK + b_row) * a.ldb + (int64_t)tn * BN + b_c4 * 4;
        const int64_t gb_chunk = (int64_t)BK * a.ldb;
        const int sa = (a_c4 * 4) * LDT + a_row;
        const int sb = A_STAGE + b_row * LDB_S + b_c4 * 4;
        const int tx = tid & 15, ty = tid >> 4;

        f32x4 ra0, ra1, rb;
        auto load_global = [&]() {
            ra0 = *(const f32x4 *)ga;
            ra1 = *(const f32x4 *)(ga + ga_half);
            rb = *(const f32x4 *)gb;
        };
        auto store_lds = [&](int stage) {
            float *s = lds + stage * STAGE;
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // A stored transposed: [k][m]
                s[sa + j * LDT] = ra0[j];
                s[sa + j * LDT + 128] = ra1[j];
            }
            *(f32x4 *)(s + sb) = rb;
        };
        auto read_step = [&](const float *s, int k, f32x4 (&av)[4], f32x4 (&bv)[2]) {
#pragma unroll
            for (int q = 0; q < 4; ++q) av[q] = *(const f32x4 *)(s + k * LDT + 64 * q + ty * 4);
#pragma unroll
            for (int p = 0; p < 2; ++p) bv[p] = *(const f32x4 *)(s + A_STAGE + k * LDB_S + 64 * p + tx * 4);
        };
        auto compute = [&](int stage) {
            const float *s = lds + stage * STAGE;
            f32x4 av[2][4], bv[2][2];
            read_step(s, 0, av[0], bv[0]);
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                if (k + 1 < BK) read_step(s, k + 1, av[(k + 1) & 1], bv[(k + 1) & 1]);
#pragma unroll
                for (int i = 0; i < 16; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        fmac_rowwise(acc[i][j], av[k & 1][i >> 2][i & 3], bv[k & 1][j >> 2][j & 3]);
            }
            // Issue order: step 0's reads, then per step the next step's
            // reads followed by this step's 128 multiply-adds.
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
            for (int k = 0; k < BK; ++k) {
                if (k + 1 < BK) __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 128, 0);
            }
        };

        // The loop body is one basic block (the scheduling order above holds
        // only within one): the last chunk loads and stores its own data
        // again instead of branching around the next chunk's loads; its stage
        // is not read after the last barrier.
        const int nch = k1 - k0;
        load_global();
        __syncthreads();
        store_lds(0);
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            const int cur = c & 1;
            const int step = c + 1 < nch ? 1 : 0;
            ga += step * BK;
            gb += step * gb_chunk;
            load_global();
            compute(cur);
            store_lds(cur ^ 1);
            __syncthreads();
        }
    }

    // Accumulator (4q + i, 4p + j) is row 64 q + 4 ty + i, column
    // 64 p + 4 tx + j of the tile.
    __device__ __forceinline__ void store_c(const KernelArgs &a, int tm, int tn) {
        const int tid = threadIdx.x;
        const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = tm * BM + 64 * (i >> 2) + ty * 4 + (i & 3);
            float *c = a.C + (int64_t)row * a.ldc + (int64_t)tn * BN + tx * 4;
            *(f32x4 *)c = epilogue(a, f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]}, c);
            *(f32x4 *)(c + 64) =
                epilogue(a, f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]}, c + 64);
        }
    }

    __device__ __forceinline__ void store_tile(float *p) {
        const int tid = threadIdx.x;
        const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float *q = p + (64 * (i >> 2) + ty * 4 + (i & 3)) * BN + tx * 4;
            *(f32x4 *)q = f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
            *(f32x4 *)(q + 64) = f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]};
        }
    }
};

template <class Core, bool SPLIT>
__global__ __launch_bounds__(Core::NT) void sgemm_valu_kernel(KernelArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[Core::LDS_FLOATS];
    run_gemm<Core, SPLIT>(a, lds);
}

template <class Core>
static hipError_t launch_core(const KernelArgs &a, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args};
    const void *f = a.sk_tiles > 0 ? (const void *)sgemm_valu_kernel<Core, true>
                                   : (const void *)sgemm_valu_kernel<Core, false>;
    return hipLaunchKernel(f, dim3(a.grid), dim3(Core::NT), params, 0, s);
}

hipError_t launch_valu(int cfg, const KernelArgs &a, hipStream_t s) {
    switch (cfg) {
    case SGEMM_CFG_VALU_128x128x8: return launch_core<Valu128x128x8>(a, s);
    case SGEMM_CFG_VALU_256x128x8: return launch_core<Valu256x128x8>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t occupancy_valu(int cfg, int *wg_per_cu) {
    switch (cfg) {
    case SGEMM_CFG_VALU_128x128x8:
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
            wg_per_cu, (const void *)sgemm_valu_kernel<Valu128x128x8, true>, Valu128x128x8::NT, 0);
    case SGEMM_CFG_VALU_256x128x8:
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
            wg_per_cu, (const void *)sgemm_valu_kernel<Valu256x128x8, true>, Valu256x128x8::NT, 0);
    default: return hipErrorInvalidValue;
    }
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
