// Products with at most 8 columns (N <= 8), A stored M x K: HBM-bound on A
// (y = A x is the case N = 1).  Each output is the dot product of a row of
// A with a column of B, so the lanes of a wave stream a row of A along K
// (one 16-byte load per lane, 1 KiB per wave per load: the coalesced access
// of "Vectorized Memory Access: Pushing CUDA SGEMM to 29 TFLOPS on H100",
// section 3; four 4-byte loads covering the same 1 KiB when A's rows are
// off the 16-byte grid) and each keeps partial dot products for the
// few columns; a butterfly over the 64 lanes, always the same one, finishes
// them.
//
// Work: workgroup w owns row block w / KS and K split w % KS.  It stages its
// split's rows of B (K x N, tiny) in LDS once, k-contiguous per column so
// that the lanes read consecutive 16-byte quads, and then walks its rows of
// A: wave v of 8 takes rows v, v + 8, ... of the block, R at a time (R
// loads of A per k quad share one read of B; R = 1 with 16-byte loads, 4
// with 4-byte ones where the block is tall enough).  Eight waves per workgroup
// (two workgroups per CU by their 64 KiB of LDS) measured 4-28% faster than
// four (16384 x 1 x 16384: 5.3 against 5.1 TB/s; 8192 x 2 x 8192: 4.9
// against 3.8).  With KS > 1 each workgroup writes its
// rows' partial dot products and a second kernel adds the KS partials in
// split order.  A lane's sum over its k, the butterfly and the split order
// are the same whatever R and the grid are: results repeat bit for bit.
#include "gemm_common.h"
#include "kernels.h"
#include "plan.h"

namespace sgemm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// B(k, n) of the product (B stored K x N, or N x K when trans_b).
__device__ __forceinline__ float b_at(const KernelArgs &a, int k, int n) {
    return a.trans_b ? a.B[(int64_t)n * a.ldb + k] : a.B[(int64_t)k * a.ldb + n];
}

// C(m, n) of the product: C stored M x N, or N x M when trans_c (the
// transposed product of a call with few rows and B stored N x K).
__device__ __forceinline__ float *c_at(const KernelArgs &a, int trans_c, int m, int n) {
    return trans_c ? a.C + (int64_t)n * a.ldc + m : a.C + (int64_t)m * a.ldc + n;
}

// Sum over the 64 lanes of a wave by a butterfly of fixed order (every lane
// ends with the same total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// A's row at columns k..k+3: one 16-byte load when the rows lie on 16-byte
// boundaries (VEC) and all four come before k_end, else one float at a
// time (zeros at and after k_end).
template <bool VEC>
__device__ __forceinline__ f32x4 a_quad(const float *row, int k, int k_end) {
    if (VEC && k + 4 <= k_end) return *(const f32x4 *)(row + k);
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
        if (k + t < k_end) v[t] = row[k + t];
    return v;
}

template <int R, int NR, bool VEC>
__global__ __launch_bounds__(kThreads) void sgemm_rowdot_kernel(KernelArgs a, int trans_c) {
    constexpr int KB = kRowdotFloats / NR;   // k of B per column staged
    constexpr int U = R == 1 ? 8 : 4;        // A quads in flight per lane and row
    __shared__ __attribute__((aligned(16))) float bs[kRowdotFloats];   // bs[n * KB + k]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ks_count = a.ipt;
    const int blk = blockIdx.x / ks_count, ks = blockIdx.x - blk * ks_count;
    const int k_per = ((a.K + ks_count - 1) / ks_count + 3) & ~3;   // splits start on 16-byte boundaries
    const int k_begin = ks * k_per;
    const int k_end = k_begin + k_per < a.K ? k_begin + k_per : a.K;
    const int klen = k_end > k_begin ? k_end - k_begin : 0;
    const int rows_per = (a.M + a.tiles_m - 1) / a.tiles_m;
    const int r_begin = blk * rows_per;
    const int r_end = r_begin + rows_per < a.M ? r_begin + rows_per : a.M;

    // B's split, columns n < N, zeros beyond; threads along B's contiguous
    // dimension.
    for (int i = tid; i < NR * KB; i += kThreads) {
        int n, kl;
        if (a.trans_b) { n = i / KB; kl = i - n * KB; }
        else { kl = i / NR; n = i - kl * NR; }
        bs[n * KB + kl] = (n < a.N && kl < klen) ? b_at(a, k_begin + kl, n) : 0.0f;
    }
    __syncthreads();

    for (int m0 = r_begin + wave * R; m0 < r_end; m0 += kWaves * R) {
        const float *row[R];
        bool ok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ok[r] = m0 + r < r_end;
            row[r] = a.A + (int64_t)(ok[r] ? m0 + r : r_begin) * a.lda;
        }
        float acc[R][NR];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int n = 0; n < NR; ++n) acc[r][n] = 0.0f;

        // This lane's quads: k = k_begin + 4 (lane + 64 j), U of them at a time.
        for (int q0 = 4 * lane; q0 < klen; q0 += 256 * U) {
            f32x4 av[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int kl = q0 + 256 * u;
                    av[u][r] = (ok[r] && kl < klen) ? a_quad<VEC>(row[r], k_begin + kl, k_end)
                                                    : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kl = q0 + 256 * u;
                if (kl >= klen) break;   // per lane: the quads past this split add nothing
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    const f32x4 bv = *(const f32x4 *)(bs + n * KB + kl);
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int t = 0; t < 4; ++t) acc[r][n] += av[u][r][t] * bv[t];
                }
            }
        }

#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int n = 0; n < NR; ++n) acc[r][n] = wave_sum(acc[r][n]);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (!ok[r]) continue;
                if (ks_count == 1) {
#pragma unroll
                    for (int n = 0; n < NR; ++n)
                        if (n < a.N) {
                            float *c = c_at(a, trans_c, m0 + r, n);
                            *c = epilogue(a, acc[r][n], c);
                        }
                } else {
                    // Partial dot products: split ks, row m, column n at
                    // partials[(ks * M + m) * 8 + n].
                    float *p = a.partials + ((int64_t)ks * a.M + m0 + r) * 8;
#pragma unroll
                    for (int n = 0; n < NR; ++n) p[n] = acc[r][n];
                }
            }
        }
    }
}

// C(m, n) = the KS partial dot products added in split order, then the
// epilogue: one thread per output.
__global__ __launch_bounds__(256) void sgemm_rowdot_sum_kernel(KernelArgs a, int trans_c) {
    const int64_t total = (int64_t)a.M * a.N;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(t / a.N), n = (int)(t - (int64_t)m * a.N);
        const float *p = a.partials + (int64_t)m * 8 + n;
        float sum = 0.0f;
        for (int s = 0; s < a.ipt; ++s) sum += p[(int64_t)s * a.M * 8];
        float *c = c_at(a, trans_c, m, n);
        *c = epilogue(a, sum, c);
    }
}

template <int R, int NR, bool VEC>
hipError_t launch_shape(const KernelArgs &a, int trans_c, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args, &trans_c};
    hipError_t e = hipLaunchKernel((const void *)sgemm_rowdot_kernel<R, NR, VEC>, dim3(a.grid), dim3(kThreads),
                                   params, 0, s);
    if (e != hipSuccess || a.ipt <= 1) return e;
    const int64_t threads = (int64_t)a.M * a.N;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return hipLaunchKernel((const void *)sgemm_rowdot_sum_kernel, dim3((unsigned)blocks), dim3(256), params, 0, s);
}

template <int R, bool VEC>
hipError_t launch_rows(const KernelArgs &a, int trans_c, hipStream_t s) {
    if (a.N == 1) return launch_shape<R, 1, VEC>(a, trans_c, s);
    if (a.N == 2) return launch_shape<R, 2, VEC>(a, trans_c, s);
    if (a.N <= 4) return launch_shape<R, 4, VEC>(a, trans_c, s);
    return launch_shape<R, 8, VEC>(a, trans_c, s);
}

}  // namespace

hipError_t launch_rowdot(int cfg, const KernelArgs &a, hipStream_t s, int trans_c) {
    if (cfg != SGEMM_CFG_ROWDOT_N8 || a.N < 1 || a.N > 8 || a.trans_a || a.tiles_m < 1 || a.ipt < 1 ||
        (a.ipt > 1 && !a.partials) || rowdot_k_per(a.K, a.ipt) > kRowdotFloats / rowdot_cols(a.N))
        return hipErrorInvalidValue;
    // 16-byte loads when A's rows start on 16-byte boundaries, one row per
    // wave at a time (measured 1-6% faster than four: 16384 x 8 x 16384 in
    // 220 against 225 us, 65536 x 4 x 1024 in 46 against 49).  With 4-byte
    // loads, four rows per wave once a block has at least four per wave
    // (16384 x 1 x 16383: 259 against 268 us with one).
    const bool vec = ((uintptr_t)a.A & 15) == 0 && (a.lda & 3) == 0;
    const int tc = trans_c ? 1 : 0;
    if (vec) return launch_rows<1, true>(a, tc, s);
    const int rows_per = (a.M + a.tiles_m - 1) / a.tiles_m;
    return rows_per >= 4 * kWaves ? launch_rows<4, false>(a, tc, s) : launch_rows<1, false>(a, tc, s);
}

hipError_t occupancy_rowdot(int cfg, int *wg_per_cu) {
    if (cfg != SGEMM_CFG_ROWDOT_N8) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(wg_per_cu, (const void *)sgemm_rowdot_kernel<1, 8, true>,
                                                        kThreads, 0);
}

}  // namespace sgemm
