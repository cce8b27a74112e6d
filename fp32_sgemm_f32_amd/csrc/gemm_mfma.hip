// FP32 GEMM on the gfx950 matrix cores: v_mfma_f32_32x32x2_f32.
//
// The instruction multiplies a 32x2 FP32 block of A by a 2x32 FP32 block of
// B and adds the 32x32 product into FP32 accumulators: full FP32 inputs, no
// reduced-precision rounding of the operands, so the arithmetic stays what
// the page "Beyond Kernel 7: Closing the Gap to cuBLAS on an H100 FP32 GEMM"
// (section "The operation: GEMM and the precision of the comparison")
// requires of the comparison: FP32 inputs and FP32 arithmetic.
//
// Structure of one workgroup (BM x BN output tile, K chunks of BK):
//   * global -> registers: each lane issues 128-bit loads (global_load_dwordx4)
//     of A rows and B rows, adjacent lanes on adjacent addresses; chunk c+1 is
//     in flight while chunk c is multiplied (register prefetch).
//   * registers -> LDS: two LDS stages (ping-pong), one barrier per chunk.
//     A is kept row-major (k contiguous) with rows padded to BK+4 floats; B is
//     kept row-major (n contiguous) with rows padded to BN+4 floats.  Both
//     paddings make the fragment reads below free of bank conflicts.
//   * LDS -> matrix cores: the waves tile the workgroup tile WAVES_M x
//     WAVES_N; a wave owns FM x FN blocks of 32x32.  Inside a chunk the K
//     index is permuted so that lane half h (lanes 32h .. 32h+31) works on
//     k in [h*BK/2, (h+1)*BK/2): each MFMA step p pairs k = p (half 0) with
//     k = BK/2 + p (half 1).  A sum is a sum, so the product is unchanged,
//     and a lane's A operands for consecutive steps are consecutive floats in
//     its LDS row: one ds_read_b128 feeds four steps.
//   * epilogue: each lane owns 16 values of each 32x32 block; a lane half
//     writes 32 consecutive floats of a C row per store.
#include "gemm_common.h"
#include "kernels.h"

namespace sgemm {

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WAVES_M, int WAVES_N>
struct MfmaCore {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WTM = BM / WAVES_M;      // wave tile rows
    static constexpr int WTN = BN / WAVES_N;      // wave tile columns
    static constexpr int FM = WTM / 32;           // 32x32 blocks per wave, down
    static constexpr int FN = WTN / 32;           // 32x32 blocks per wave, across
    static constexpr int KH = BK / 2;             // k values per lane half per chunk
    static constexpr int LDA_S = BK + 4;          // LDS row stride of the A tile
    static constexpr int LDB_S = BN + 4;          // LDS row stride of the B tile
    static constexpr int A_STAGE = BM * LDA_S;
    static constexpr int B_STAGE = BK * LDB_S;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_FLOATS = 2 * STAGE;
    static constexpr int A_VEC = BM * BK / 4 / NT;   // float4 loads of A per lane per chunk
    static constexpr int B_VEC = BK * BN / 4 / NT;   // float4 loads of B per lane per chunk
    static constexpr int A_ROWS_PER_PASS = NT / (BK / 4);
    static constexpr int B_ROWS_PER_PASS = NT / (BN / 4);
    static constexpr int TILE_FLOATS = BM * BN;

    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 8 == 0, "BK/2 must be a multiple of 4 (one b128 per four steps)");
    static_assert(A_VEC >= 1 && A_VEC * NT * 4 == BM * BK, "A tile must split evenly into float4s");
    static_assert(B_VEC >= 1 && B_VEC * NT * 4 == BK * BN, "B tile must split evenly into float4s");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");

    floatx16 acc[FM][FN];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

    __device__ __forceinline__ void mainloop(const KernelArgs &a, float *lds, int tm, int tn,
                                             int k0, int k1) {
        const int tid = threadIdx.x;
        const int64_t lda = a.lda, ldb = a.ldb;

        // Loader geometry (hoisted out of the K loop).
        const int a_row = tid / (BK / 4), a_c4 = tid % (BK / 4);
        const int b_row = tid / (BN / 4), b_c4 = tid % (BN / 4);
        const float *ga = a.A + ((int64_t)tm * BM + a_row) * lda + (int64_t)k0 * BK + a_c4 * 4;
        const float *gb = a.B + ((int64_t)k0 * BK + b_row) * ldb + (int64_t)tn * BN + b_c4 * 4;
        const int64_t ga_pass = (int64_t)A_ROWS_PER_PASS * lda;
        const int64_t gb_pass = (int64_t)B_ROWS_PER_PASS * ldb;
        const int64_t gb_chunk = (int64_t)BK * ldb;
        const int sa = a_row * LDA_S + a_c4 * 4;
        const int sb = A_STAGE + b_row * LDB_S + b_c4 * 4;

        // Fragment geometry.
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        const int lr = lane & 31, lh = lane >> 5;
        const int fa = (wm * WTM + lr) * LDA_S + lh * KH;
        const int fb = A_STAGE + lh * KH * LDB_S + wn * WTN + lr;

        f32x4 ra[A_VEC], rb[B_VEC];

        auto load_global = [&]() {
#pragma unroll
            for (int i = 0; i < A_VEC; ++i) ra[i] = *(const f32x4 *)(ga + i * ga_pass);
#pragma unroll
            for (int i = 0; i < B_VEC; ++i) rb[i] = *(const f32x4 *)(gb + i * gb_pass);
        };
        auto store_lds = [&](int stage) {
            float *s = lds + stage * STAGE;
#pragma unroll
            for (int i = 0; i < A_VEC; ++i)
                *(f32x4 *)(s + sa + i * A_ROWS_PER_PASS * LDA_S) = ra[i];
#pragma unroll
            for (int i = 0; i < B_VEC; ++i)
                *(f32x4 *)(s + sb + i * B_ROWS_PER_PASS * LDB_S) = rb[i];
        };
        auto compute = [&](int stage) {
            const float *s = lds + stage * STAGE;
#pragma unroll
            for (int p = 0; p < KH; p += 4) {
                f32x4 av[FM];
                float bv[FN][4];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    av[i] = *(const f32x4 *)(s + fa + i * 32 * LDA_S + p);
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) bv[j][q] = s[fb + (p + q) * LDB_S + j * 32];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                av[i][q], bv[j][q], acc[i][j], 0, 0, 0);
            }
        };

        const int nch = k1 - k0;
        load_global();
        __syncthreads();            // LDS may still be read by a previous tile
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

    // C element (row, col) of block (i, j), register r, for this lane:
    //   row = 32 i + 8 (r / 4) + 4 (lane / 32) + r % 4,  col = 32 j + lane % 32.
    __device__ __forceinline__ void store_c(const KernelArgs &a, int tm, int tn) {
        const int tid = threadIdx.x;
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        const int lr = lane & 31, lh = lane >> 5;
        float *c = a.C + ((int64_t)tm * BM + wm * WTM + 4 * lh) * a.ldc + (int64_t)tn * BN + wn * WTN + lr;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    c[(int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * a.ldc + j * 32] = acc[i][j][r];
    }

    // Thread-private layout: value v of this thread at p[v * NT + tid].
    __device__ __forceinline__ void store_partial(float *p) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    p[((i * FN + j) * 16 + r) * NT + tid] = acc[i][j][r];
    }

    // One 32x32 block (16 values per lane) at a time: the empty asm keeps the
    // compiler from hoisting every block's loads at once, which would need a
    // second full accumulator set of registers.
    __device__ __forceinline__ void add_partial(const float *p) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[i][j][r] += p[((i * FN + j) * 16 + r) * NT + tid];
                asm volatile("" ::: "memory");
            }
    }
};

template <class Core, bool SPLIT>
__global__ __launch_bounds__(Core::NT) void sgemm_mfma_kernel(KernelArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[Core::LDS_FLOATS];
    __shared__ int flag;
    run_gemm<Core, SPLIT>(a, lds, &flag);
}

using Mfma256x256x16 = MfmaCore<256, 256, 16, 4, 2>;
using Mfma128x128x32 = MfmaCore<128, 128, 32, 2, 2>;
using Mfma256x256x32 = MfmaCore<256, 256, 32, 2, 2>;
using Mfma256x128x32 = MfmaCore<256, 128, 32, 2, 2>;

template <class Core>
static hipError_t launch(const KernelArgs &a, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args};
    const void *f = a.sk_tiles > 0 ? (const void *)sgemm_mfma_kernel<Core, true>
                                   : (const void *)sgemm_mfma_kernel<Core, false>;
    return hipLaunchKernel(f, dim3(a.grid), dim3(Core::NT), params, 0, s);
}

// Workgroups per CU of the split instance (the larger register footprint of
// the two, so it bounds both).
template <class Core>
static hipError_t occ(int *n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        n, (const void *)sgemm_mfma_kernel<Core, true>, Core::NT, 0);
}

hipError_t launch_mfma(int cfg, const KernelArgs &a, hipStream_t s) {
    switch (cfg) {
    case SGEMM_CFG_MFMA_256x256x16: return launch<Mfma256x256x16>(a, s);
    case SGEMM_CFG_MFMA_128x128x32: return launch<Mfma128x128x32>(a, s);
    case SGEMM_CFG_MFMA_256x256x32: return launch<Mfma256x256x32>(a, s);
    case SGEMM_CFG_MFMA_256x128x32: return launch<Mfma256x128x32>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t occupancy_mfma(int cfg, int *wg_per_cu) {
    switch (cfg) {
    case SGEMM_CFG_MFMA_256x256x16: return occ<Mfma256x256x16>(wg_per_cu);
    case SGEMM_CFG_MFMA_128x128x32: return occ<Mfma128x128x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_256x256x32: return occ<Mfma256x256x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_256x128x32: return occ<Mfma256x128x32>(wg_per_cu);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sgemm
