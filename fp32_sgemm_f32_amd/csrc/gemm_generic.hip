// FP32 GEMM for any shape, any (4-byte) alignment and either storage order
// of A and B: the general path.
//
// The fast kernels load 16-byte vectors and assume rows that start on
// 16-byte boundaries; this one loads single floats, each checked against the
// matrix bounds (a zero stands in outside), so ragged edges in M, N and K,
// odd leading dimensions and misaligned pointers all work.  It is the
// zero-padded, bounds-checked path that "Vectorized Memory Access: Pushing
// CUDA SGEMM to 29 TFLOPS on H100" (section 5, unaligned tails and
// boundaries) and "2D Block Tiling: Scaling Matrix Multiplication on NVIDIA
// H100" (section 5, non-multiple shapes) use for boundary tiles, here used
// for the whole product when its layout rules out the vector kernels.
//
// Tile 64 x 64, K chunks of 16, four waves of 32 x 32 on v_mfma_f32_32x32x2_f32
// with the same K permutation and LDS layout as the register-staged core:
// A rows and B columns k-contiguous, row stride 20 floats (4 x odd words).
// Two LDS stages; the next chunk's loads are issued before the barrier.
#include "gemm_common.h"
#include "kernels.h"

namespace sgemm {

typedef float floatx16 __attribute__((ext_vector_type(16)));

struct GenericCore {
    static constexpr int BM = 64, BN = 64, BK = 16;
    static constexpr int NT = 256;
    static constexpr int LDK = BK + 4;
    static constexpr int A_STAGE = BM * LDK, B_STAGE = BN * LDK;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_FLOATS = 2 * STAGE;
    static constexpr int TILE_FLOATS = BM * BN;

    floatx16 acc;

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    }

    // Chunk c of tile (tm, tn): this thread's 4 A values (k-consecutive, for
    // one row) and 4 B values (k-consecutive for one column when B is stored
    // transposed, else column-consecutive for one k), each bounds-checked.
    // The thread map follows the stored layout so that neighbouring threads
    // read neighbouring addresses.
    __device__ __forceinline__ static void load(const KernelArgs &a, int tm, int tn, int c, float (&ra)[4],
                                                float (&rb)[4]) {
        const int t = threadIdx.x;
        if (!a.trans_a) {   // A[m * lda + k]: threads along k
            const int row = tm * BM + t / 4, ka = c * BK + 4 * (t % 4);
            const bool row_ok = row < a.M;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ra[j] = (row_ok && ka + j < a.K) ? a.A[(int64_t)row * a.lda + ka + j] : 0.0f;
        } else {            // A[k * lda + m]: threads along m
            const int row = tm * BM + t % 64, ka = c * BK + 4 * (t / 64);
            const bool row_ok = row < a.M;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ra[j] = (row_ok && ka + j < a.K) ? a.A[(int64_t)(ka + j) * a.lda + row] : 0.0f;
        }
        if (!a.trans_b) {   // B[k * ldb + n]: threads along n
            const int kb = c * BK + t / 16, col = tn * BN + 4 * (t % 16);
            const bool k_ok = kb < a.K;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                rb[j] = (k_ok && col + j < a.N) ? a.B[(int64_t)kb * a.ldb + col + j] : 0.0f;
        } else {            // B[n * ldb + k]: threads along k
            const int col = tn * BN + t / 4, kb = c * BK + 4 * (t % 4);
            const bool col_ok = col < a.N;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                rb[j] = (col_ok && kb + j < a.K) ? a.B[(int64_t)col * a.ldb + kb + j] : 0.0f;
        }
    }

    // A[row][k..k+3] of the thread's map to its LDS row; B likewise into
    // the k-contiguous row of its column (a transposing scatter when B is
    // stored k-major).
    __device__ __forceinline__ static void store(const KernelArgs &a, float *s, const float (&ra)[4],
                                                 const float (&rb)[4]) {
        const int t = threadIdx.x;
        const int am = a.trans_a ? t % 64 : t / 4, ak = a.trans_a ? 4 * (t / 64) : 4 * (t % 4);
        *(f32x4 *)(s + am * LDK + ak) = f32x4{ra[0], ra[1], ra[2], ra[3]};
        if (a.trans_b) {
            *(f32x4 *)(s + A_STAGE + (t / 4) * LDK + 4 * (t % 4)) = f32x4{rb[0], rb[1], rb[2], rb[3]};
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) s[A_STAGE + (4 * (t % 16) + j) * LDK + t / 16] = rb[j];
        }
    }

    __device__ __forceinline__ void mainloop(const KernelArgs &a, float *lds, int tm, int tn, int k0, int k1) {
        const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
        const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
        const int fa = (wm * 32 + lr) * LDK + 8 * lh, fb = A_STAGE + (wn * 32 + lr) * LDK + 8 * lh;
        float ra[4], rb[4];
        __syncthreads();   // a previous tile may still read the stages
        load(a, tm, tn, k0, ra, rb);
        for (int c = k0; c < k1; ++c) {
            float *s = lds + ((c - k0) & 1) * STAGE;
            store(a, s, ra, rb);
            if (c + 1 < k1) load(a, tm, tn, c + 1, ra, rb);
            __syncthreads();
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const f32x4 av = *(const f32x4 *)(s + fa + 4 * g);
                const f32x4 bv = *(const f32x4 *)(s + fb + 4 * g);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u], acc, 0, 0, 0);
            }
        }
    }

    // C element of register r: row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32.
    __device__ __forceinline__ void store_c(const KernelArgs &a, int tm, int tn) {
        const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
        const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
        const int col = tn * BN + wn * 32 + lr;
        if (col >= a.cn) return;
        const int row0 = tm * BM + wm * 32 + 4 * lh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = row0 + 8 * (r >> 2) + (r & 3);
            if (row < a.cm) {
                float *p = a.C + (int64_t)row * a.ldc + col;
                *p = epilogue(a, acc[r], p);
            }
        }
    }

    // The same mapping into a dense row-major BM x BN tile (a split tile's
    // partial sum).
    __device__ __forceinline__ void store_tile(float *p) {
        const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
        const int wm = wave >> 1, wn = wave & 1, lr = lane & 31, lh = lane >> 5;
        float *q = p + (wm * 32 + 4 * lh) * BN + wn * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) q[(8 * (r >> 2) + (r & 3)) * BN] = acc[r];
    }
};

template <bool SPLIT>
__global__ __launch_bounds__(GenericCore::NT) void sgemm_generic_kernel(KernelArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[GenericCore::LDS_FLOATS];
    run_gemm<GenericCore, SPLIT>(a, lds);
}

hipError_t launch_generic(int cfg, const KernelArgs &a, hipStream_t s) {
    if (cfg != SGEMM_CFG_GENERIC_64x64x16) return hipErrorInvalidValue;
    KernelArgs args = a;
    void *params[] = {&args};
    const void *f = a.sk_tiles > 0 ? (const void *)sgemm_generic_kernel<true> : (const void *)sgemm_generic_kernel<false>;
    return hipLaunchKernel(f, dim3(a.grid), dim3(GenericCore::NT), params, 0, s);
}

hipError_t occupancy_generic(int cfg, int *wg_per_cu) {
    if (cfg != SGEMM_CFG_GENERIC_64x64x16) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(wg_per_cu, (const void *)sgemm_generic_kernel<true>,
                                                        GenericCore::NT, 0);
}

}  // namespace sgemm
