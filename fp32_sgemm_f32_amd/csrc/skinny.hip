// Products with at most 16 rows (M <= 16), B stored K x N: HBM-bound on B.
// A tile of the matrix-core kernels computes 64 or more rows, so for such
// an M most of its work is empty rows, and streaming B stops at what those
// MFMAs allow (~4.4 TB/s).  This kernel does only the M rows' multiply-adds
// on the vector ALU and spends its registers on loads in flight instead:
// the design the pages use for their FMA kernels (a register-tiled outer
// product fed from shared memory: "2D Block Tiling: Scaling Matrix
// Multiplication on NVIDIA H100", section 3; 16-byte loads: "Vectorized
// Memory Access: Pushing CUDA SGEMM to 29 TFLOPS on H100", section 3), with
// A as the small operand held in LDS and B streamed.
//
// Work: workgroup w of the grid owns column strip w / KS (256 columns) and
// K split w % KS.  K is cut into blocks of 512 k (shorter when K / KS is),
// dealt to the splits in turn, so that at any time all workgroups read B
// within a band of KS blocks rather than in KS bands far apart; inside a
// block the 8 waves take interleaved groups of 16 k, so that together they
// read one window of consecutive rows of B.  Both measured:
// 1 x 16384 x 16384 in 168 us against 181 with contiguous splits and
// per-wave k ranges.  DRAM locality, not loads in flight, was the limit:
// twice the loads in flight per lane ran slower.
//
// Up to 8 rows, each lane holds 4 adjacent columns for MR rows (4 or 8):
// per k one 16-byte B load (when B is off the 16-byte grid: four 4-byte
// loads, the lane's columns 64 apart so that each load of a wave is
// contiguous) and 4 * MR multiply-adds, 16 loads in flight per lane.  A's
// values, the same for every lane, are staged in LDS (k-major, MR floats
// per k) a block at a time and read as broadcasts.  For 9-16 rows the
// multiply-adds go to the matrix cores instead (16 x 16 x 4 steps, all 16
// rows at once, no row of B read twice): 216 against 245 us at 16 x 16384
// x 16384 for two groups of 8 rows on the vector ALU, each group reading
// every B line.  Two waves per SIMD: the LDS of the 16-row kernel (96 KiB)
// admits one workgroup per CU anyway, so each wave may use 256 registers.
// The 8 waves' sums are added through LDS in a fixed tree order; with
// KS > 1 each workgroup writes its strip's partial sum, and a second kernel
// adds the KS partials in split order and writes C.  Every sum is taken in
// a fixed order, so results repeat bit for bit.
#include "gemm_common.h"
#include "kernels.h"
#include "plan.h"

namespace sgemm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 256;            // columns per strip: 64 lanes x 4
constexpr int kBlock = kSkinnyBlock;  // k per A staging block

// C(m, n) of the product: C stored M x N, or N x M when trans_c (the
// transposed product of a call with few columns and A stored K x M).
__device__ __forceinline__ float *c_at(const KernelArgs &a, int trans_c, int m, int n) {
    return trans_c ? a.C + (int64_t)n * a.ldc + m : a.C + (int64_t)m * a.ldc + n;
}

// A(m, k) of the product (A stored M x K, or K x M when trans_a).
__device__ __forceinline__ float a_at(const KernelArgs &a, int m, int k) {
    return a.trans_a ? a.A[(int64_t)k * a.lda + m] : a.A[(int64_t)m * a.lda + k];
}

// acc[m][j] += A(m, k) * B(k, the lane's column j) for one k: A's MR values (a broadcast
// LDS read) times the lane's 4 B values, m and then j ascending.
template <int MR>
__device__ __forceinline__ void fma_k(float (&acc)[MR][4], const float *ap, const f32x4 &b) {
#pragma unroll
    for (int q = 0; q < MR / 4; ++q) {
        const f32x4 av = *(const f32x4 *)(ap + 4 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * q + r][j] += av[r] * b[j];
    }
}

// The lane's 4 columns of its strip: adjacent (n0 .. n0 + 3, one 16-byte
// load) when B's rows and N are on the 16-byte grid (VEC); else 64 apart
// (base + 64 j + lane), so that each of the 4 one-float loads of a wave
// reads 64 consecutive floats.
template <bool VEC>
__device__ __forceinline__ int lane_col(int strip, int lane, int j) {
    return VEC ? strip * kCols + 4 * lane + j : strip * kCols + 64 * j + lane;
}

// B's row k at the lane's 4 columns, zeros at and after N.
template <bool VEC>
__device__ __forceinline__ f32x4 b_quad(const KernelArgs &a, int k, int strip, int lane) {
    const float *p = a.B + (int64_t)k * a.ldb;
    if (VEC) return *(const f32x4 *)(p + lane_col<true>(strip, lane, 0));
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = lane_col<false>(strip, lane, j);
        if (n < a.N) v[j] = p[n];
    }
    return v;
}

template <int MR, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sgemm_skinny_kernel(KernelArgs a, int trans_c) {
    constexpr int kUnroll = 16;   // B loads in flight per lane
    // A block (k-major, MR floats per k), then the waves' sums.
    __shared__ __attribute__((aligned(16))) float as[kBlock * MR];
    __shared__ __attribute__((aligned(16))) float red[(kWaves / 2) * MR * kCols];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ks_count = a.ipt;
    const int strip = blockIdx.x / ks_count, ks = blockIdx.x - strip * ks_count;
    // K is cut into blocks of kb (at most kBlock, at least what puts every
    // split's k in one block when the splits are short), dealt to the
    // splits in turn: split ks takes blocks ks, ks + KS, ...
    const int64_t k_per = ((int64_t)a.K + ks_count - 1) / ks_count;
    const int kb = k_per < kBlock ? (int)(k_per + kUnroll - 1) / kUnroll * kUnroll : kBlock;
    const bool col_ok = lane_col<VEC>(strip, lane, 0) < a.N;   // the lane's first (lowest) column

    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = 0.0f;

    for (int64_t b0 = (int64_t)ks * kb; b0 < a.K; b0 += (int64_t)ks_count * kb) {
        const int blk = (int)b0;
        const int blen = a.K - blk < kb ? a.K - blk : kb;
        __syncthreads();   // the previous block's reads are done
        // Stage A(0..MR-1, blk..blk+blen-1), zeros in rows >= M; threads
        // along A's contiguous dimension.
        for (int i = tid; i < blen * MR; i += kThreads) {
            int m, kl;
            if (a.trans_a) { kl = i / MR; m = i - kl * MR; }
            else { m = i / blen; kl = i - m * blen; }
            as[kl * MR + m] = m < a.M ? a_at(a, m, blk + kl) : 0.0f;
        }
        __syncthreads();
        // This wave's share of the block: groups wave, wave + 8, ... of
        // kUnroll k (all loads first), so that the waves read one window of
        // 8 * kUnroll consecutive rows of B at a time; a last, shorter group
        // one k at a time.
        for (int g0 = wave * kUnroll; g0 < blen; g0 += kWaves * kUnroll) {
            const int k = blk + g0;
            if (g0 + kUnroll <= blen) {
                f32x4 b[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    b[u] = col_ok ? b_quad<VEC>(a, k + u, strip, lane) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) fma_k(acc, as + (k + u - blk) * MR, b[u]);
            } else {
                for (int kk = k; kk < blk + blen; ++kk) {
                    const f32x4 b = col_ok ? b_quad<VEC>(a, kk, strip, lane) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    fma_k(acc, as + (kk - blk) * MR, b);
                }
            }
        }
    }

    // Sum the waves in a fixed tree: (w + 4), (w + 2), then (w + 1).
#pragma unroll
    for (int half = kWaves / 2; half >= 1; half >>= 1) {
        __syncthreads();
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
                *(f32x4 *)(red + ((wave - half) * MR + m) * kCols + 4 * lane) =
                    f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        }
        __syncthreads();
        if (wave < half) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const f32x4 v = *(const f32x4 *)(red + (wave * MR + m) * kCols + 4 * lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][j] += v[j];
            }
        }
    }
    if (wave != 0 || !col_ok) return;

    if (ks_count == 1) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= a.M) break;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = lane_col<VEC>(strip, lane, j);
                if (VEC || n < a.N) {
                    float *c = c_at(a, trans_c, m, n);
                    *c = epilogue(a, acc[m][j], c);
                }
            }
        }
    } else {
        // Partial sums, dense: split ks, row m, column n at
        // partials[(ks * 16 + m) * Np + n], Np = strips * 256.
        const int64_t np = (int64_t)a.tiles_n * kCols;
        float *p = a.partials + (int64_t)ks * 16 * np;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= a.M) break;
            if (VEC) {
                *(f32x4 *)(p + m * np + lane_col<true>(strip, lane, 0)) =
                    f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) p[m * np + lane_col<false>(strip, lane, j)] = acc[m][j];
            }
        }
    }
}

// 16 rows on the matrix cores: v_mfma_f32_16x16x4f32 steps (A operand: lane
// l holds A(l % 16, k0 + l / 16); B operand: B(k0 + l / 16, column l % 16 of
// the step's 16; result: rows 4 (l / 16) + r, r = 0..3, column l % 16).  A
// wave's 256 columns are 16 such 16-column steps: with 16-byte loads of B
// (VEC) step (g, q) takes columns 64 g + 4 c + q, c = 0..15, so that one
// lane's quad B(k, 64 g + 4 c .. + 3) is its operand for the four steps
// (g, 0..3); else step (g, q) takes columns 64 g + 16 q + c, one float each.
// Work, blocks, groups and the waves' sums as in the vector-ALU kernel.
template <bool VEC>
__device__ __forceinline__ int mf_col(int strip, int g, int q, int c) {
    return VEC ? strip * kCols + 64 * g + 4 * c + q : strip * kCols + 64 * g + 16 * q + c;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sgemm_skinny_mfma_kernel(KernelArgs a, int trans_c) {
    constexpr int kGroup = 16;            // k per group: four 4-k steps, 16 B loads in flight per lane
    __shared__ __attribute__((aligned(16))) float as[kBlock * 16];            // [k][16 rows]
    __shared__ __attribute__((aligned(16))) float red[(kWaves / 2) * 16 * 4 * 64];   // [slot][step][r][lane]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = lane & 15, kq = lane >> 4;
    const int ks_count = a.ipt;
    const int strip = blockIdx.x / ks_count, ks = blockIdx.x - strip * ks_count;
    const int64_t k_per = ((int64_t)a.K + ks_count - 1) / ks_count;
    const int kb = k_per < kBlock ? (int)(k_per + kGroup - 1) / kGroup * kGroup : kBlock;

    f32x4 acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t b0 = (int64_t)ks * kb; b0 < a.K; b0 += (int64_t)ks_count * kb) {
        const int blk = (int)b0;
        const int blen = a.K - blk < kb ? a.K - blk : kb;
        const int blen16 = (blen + kGroup - 1) / kGroup * kGroup;   // <= kBlock
        __syncthreads();   // the previous block's reads are done
        // Stage A(0..15, blk..blk+blen16-1), zeros in rows >= M and k >= blen.
        for (int i = tid; i < blen16 * 16; i += kThreads) {
            int m, kl;
            if (a.trans_a) { kl = i >> 4; m = i & 15; }
            else { m = i / blen16; kl = i - m * blen16; }
            as[kl * 16 + m] = (m < a.M && kl < blen) ? a_at(a, m, blk + kl) : 0.0f;
        }
        __syncthreads();
        for (int g0 = wave * kGroup; g0 < blen; g0 += kWaves * kGroup) {
            f32x4 b[4][4];   // [step][column group]
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int kl = g0 + 4 * s + kq;
                const bool k_ok = kl < blen;
                const float *p = a.B + (int64_t)(blk + (k_ok ? kl : 0)) * a.ldb;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    if (VEC) {
                        const int n = mf_col<true>(strip, g, 0, c);
                        b[s][g] = (k_ok && n < a.N) ? *(const f32x4 *)(p + n) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = mf_col<false>(strip, g, q, c);
                            b[s][g][q] = (k_ok && n < a.N) ? p[n] : 0.0f;
                        }
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float av = as[(g0 + 4 * s + kq) * 16 + c];
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[4 * g + q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b[s][g][q], acc[4 * g + q], 0, 0, 0);
            }
        }
    }

    // Sum the 8 waves in a fixed tree: (w + 4), (w + 2), (w + 1).
#pragma unroll
    for (int half = kWaves / 2; half >= 1; half >>= 1) {
        __syncthreads();
        if (wave >= half && wave < 2 * half) {
            float *slot = red + (wave - half) * (16 * 4 * 64);
#pragma unroll
            for (int t = 0; t < 16; ++t) *(f32x4 *)(slot + (t * 64 + lane) * 4) = acc[t];
        }
        __syncthreads();
        if (wave < half) {
            const float *slot = red + wave * (16 * 4 * 64);
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[t] += *(const f32x4 *)(slot + (t * 64 + lane) * 4);
        }
    }
    if (wave != 0) return;

    const int64_t np = (int64_t)a.tiles_n * kCols;
    if (VEC && ks_count > 1) {
        // The four steps (g, 0..3) hold a lane's 4 adjacent columns: one
        // 16-byte store per row.
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = mf_col<true>(strip, g, 0, c);
            if (n >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * kq + r;
                if (m < a.M)
                    *(f32x4 *)(a.partials + ((int64_t)ks * 16 + m) * np + n) =
                        f32x4{acc[4 * g][r], acc[4 * g + 1][r], acc[4 * g + 2][r], acc[4 * g + 3][r]};
            }
        }
        return;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = mf_col<VEC>(strip, g, q, c);
            if (n >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * kq + r;
                if (m >= a.M) continue;
                if (ks_count == 1) {
                    float *cp = c_at(a, trans_c, m, n);
                    *cp = epilogue(a, acc[4 * g + q][r], cp);
                } else {
                    // partials[(ks * 16 + m) * Np + n], Np = strips * 256.
                    a.partials[((int64_t)ks * 16 + m) * np + n] = acc[4 * g + q][r];
                }
            }
        }
}

// C(m, n..n+3) = the KS partial sums added in split order, then the
// epilogue: one thread per 4 outputs (the last quad of a row may end at N),
// up to 8 splits' loads in flight.
__global__ __launch_bounds__(256) void sgemm_skinny_sum_kernel(KernelArgs a, int trans_c) {
    const int quads = (a.N + 3) / 4;
    const int64_t total = (int64_t)a.M * quads;
    const int64_t np = (int64_t)a.tiles_n * kCols;
    const int ks_count = a.ipt;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int m = (int)(t / quads), n = 4 * (int)(t - (int64_t)m * quads);
        const float *p = a.partials + (int64_t)m * np + n;
        f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < ks_count; s0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < ks_count) v[u] = *(const f32x4 *)(p + (int64_t)(s0 + u) * 16 * np);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < ks_count) sum += v[u];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n + j < a.N) {
                float *c = c_at(a, trans_c, m, n + j);
                *c = epilogue(a, sum[j], c);
            }
    }
}

// The KS partial sums are added by a second kernel when K is split.
hipError_t launch_with_sum(const void *f, const KernelArgs &a, int trans_c, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args, &trans_c};
    hipError_t e = hipLaunchKernel(f, dim3(a.grid), dim3(kThreads), params, 0, s);
    if (e != hipSuccess || a.ipt <= 1) return e;
    const int64_t threads = (int64_t)a.M * ((a.N + 3) / 4);
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return hipLaunchKernel((const void *)sgemm_skinny_sum_kernel, dim3((unsigned)blocks), dim3(256), params, 0, s);
}

}  // namespace

hipError_t launch_skinny(int cfg, const KernelArgs &a, hipStream_t s, int trans_c) {
    if (cfg != SGEMM_CFG_SKINNY_16x256 || a.M < 1 || a.M > 16 || a.trans_b ||
        (a.ipt > 1 && !a.partials))
        return hipErrorInvalidValue;
    // 16-byte loads of B when its rows and N are on the 16-byte grid.
    const bool vec = ((uintptr_t)a.B & 15) == 0 && (a.ldb & 3) == 0 && (a.N & 3) == 0;
    const void *f;
    if (a.M <= 4) f = vec ? (const void *)sgemm_skinny_kernel<4, true> : (const void *)sgemm_skinny_kernel<4, false>;
    else if (a.M <= 8) f = vec ? (const void *)sgemm_skinny_kernel<8, true> : (const void *)sgemm_skinny_kernel<8, false>;
    else f = vec ? (const void *)sgemm_skinny_mfma_kernel<true> : (const void *)sgemm_skinny_mfma_kernel<false>;
    return launch_with_sum(f, a, trans_c ? 1 : 0, s);
}

hipError_t occupancy_skinny(int cfg, int *wg_per_cu) {
    if (cfg != SGEMM_CFG_SKINNY_16x256) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(wg_per_cu, (const void *)sgemm_skinny_mfma_kernel<true>, kThreads,
                                                        0);
}

}  // namespace sgemm
