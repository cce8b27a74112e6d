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
// block the waves of a row group take interleaved groups of 16 k, so that
// together they read one window of consecutive rows of B.  Both measured:
// 1 x 16384 x 16384 in 168 us against 181 with contiguous splits and
// per-wave k ranges.  DRAM locality, not loads in flight, was the limit:
// twice the loads in flight per lane ran slower.
//
// Each lane holds 4 adjacent columns for MRW rows (4 or 8): per k one
// 16-byte B load (when B is off the 16-byte grid: four 4-byte loads, the
// lane's columns 64 apart so that each load of a wave is contiguous) and
// 4 * MRW multiply-adds, 16 loads in flight per lane.  For 9-16 rows the
// workgroup's two halves each take 8 of the rows over the same columns and
// K range, four waves each.  Two waves per SIMD: the 16-row kernel's LDS
// (96 KiB) admits one workgroup per CU anyway, so each wave may use 256
// registers.  A's values, the same for every lane, are staged in LDS
// (k-major, MR floats per k) a block at a time and read as broadcasts.  The
// 8 waves' sums are added through LDS in a fixed tree order; with KS > 1
// each workgroup writes its strip's partial sum, and a second kernel adds
// the KS partials in split order and writes C.  Every sum is taken in a
// fixed order, so results repeat bit for bit.
#include "gemm_common.h"
#include "kernels.h"
#include "plan.h"

namespace sgemm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 256;            // columns per strip: 64 lanes x 4
constexpr int kBlock = kSkinnyBlock;  // k per A staging block

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

// MRW rows per wave, H row groups per workgroup (MR = MRW * H rows in all):
// with H = 2 the two halves of the workgroup take rows 0-7 and 8-15 of the
// same columns and K range, each wave keeping the 32 accumulators of the
// 8-row form (the second read of each B line comes from L2).
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

template <int MRW, int H, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sgemm_skinny_kernel(KernelArgs a) {
    constexpr int kUnroll = 16;   // B loads in flight per lane
    constexpr int MR = MRW * H;   // rows staged
    constexpr int WH = kWaves / H;   // waves per row group
    // A block (k-major, MR floats per k), then the waves' sums.
    __shared__ __attribute__((aligned(16))) float as[kBlock * MR];
    __shared__ __attribute__((aligned(16))) float red[H * (WH / 2) * MRW * kCols];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int grp = wave / WH, sub = wave - grp * WH;   // row group, wave within it
    const int ks_count = a.ipt;
    const int strip = blockIdx.x / ks_count, ks = blockIdx.x - strip * ks_count;
    // K is cut into blocks of kb (at most kBlock, at least what puts every
    // split's k in one block when the splits are short), dealt to the
    // splits in turn: split ks takes blocks ks, ks + KS, ...
    const int64_t k_per = ((int64_t)a.K + ks_count - 1) / ks_count;
    const int kb = k_per < kBlock ? (int)(k_per + kUnroll - 1) / kUnroll * kUnroll : kBlock;
    const bool col_ok = lane_col<VEC>(strip, lane, 0) < a.N;   // the lane's first (lowest) column

    float acc[MRW][4];
#pragma unroll
    for (int m = 0; m < MRW; ++m)
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
        // This wave's share of the block: groups sub, sub + WH, ... of
        // kUnroll k (all loads first), so that a row group's waves read one
        // window of WH * kUnroll consecutive rows of B at a time; a last,
        // shorter group one k at a time.
        const float *ag = as + grp * MRW;   // this group's rows of each k
        for (int g0 = sub * kUnroll; g0 < blen; g0 += WH * kUnroll) {
            const int k = blk + g0;
            if (g0 + kUnroll <= blen) {
                f32x4 b[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    b[u] = col_ok ? b_quad<VEC>(a, k + u, strip, lane) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) fma_k(acc, ag + (k + u - blk) * MR, b[u]);
            } else {
                for (int kk = k; kk < blk + blen; ++kk) {
                    const f32x4 b = col_ok ? b_quad<VEC>(a, kk, strip, lane) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    fma_k(acc, ag + (kk - blk) * MR, b);
                }
            }
        }
    }

    // Sum each group's waves in a fixed tree: (w + WH/2), ..., then (w + 1).
    float *const rg = red + grp * (WH / 2) * MRW * kCols;
#pragma unroll
    for (int half = WH / 2; half >= 1; half >>= 1) {
        __syncthreads();
        if (sub >= half && sub < 2 * half) {
#pragma unroll
            for (int m = 0; m < MRW; ++m)
                *(f32x4 *)(rg + ((sub - half) * MRW + m) * kCols + 4 * lane) =
                    f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        }
        __syncthreads();
        if (sub < half) {
#pragma unroll
            for (int m = 0; m < MRW; ++m) {
                const f32x4 v = *(const f32x4 *)(rg + (sub * MRW + m) * kCols + 4 * lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][j] += v[j];
            }
        }
    }
    if (sub != 0 || !col_ok) return;
    const int row0 = grp * MRW;   // this group's first row

    if (ks_count == 1) {
#pragma unroll
        for (int m = 0; m < MRW; ++m) {
            if (row0 + m >= a.M) break;
            float *c = a.C + (int64_t)(row0 + m) * a.ldc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = lane_col<VEC>(strip, lane, j);
                if (VEC || n < a.N) c[n] = epilogue(a, acc[m][j], c + n);
            }
        }
    } else {
        // Partial sums, dense: split ks, row m, column n at
        // partials[(ks * 16 + m) * Np + n], Np = strips * 256.
        const int64_t np = (int64_t)a.tiles_n * kCols;
        float *p = a.partials + ((int64_t)ks * 16 + row0) * np;
#pragma unroll
        for (int m = 0; m < MRW; ++m) {
            if (row0 + m >= a.M) break;
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

// C(m, n..n+3) = the KS partial sums added in split order, then the
// epilogue: one thread per 4 outputs (the last quad of a row may end at N),
// up to 8 splits' loads in flight.
__global__ __launch_bounds__(256) void sgemm_skinny_sum_kernel(KernelArgs a) {
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
        float *c = a.C + (int64_t)m * a.ldc + n;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (n + j < a.N) c[j] = epilogue(a, sum[j], c + j);
    }
}

template <int MRW, int H>
hipError_t launch_rows(const KernelArgs &a, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args};
    // 16-byte loads of B when its rows and N are on the 16-byte grid.
    const bool vec = ((uintptr_t)a.B & 15) == 0 && (a.ldb & 3) == 0 && (a.N & 3) == 0;
    const void *f = vec ? (const void *)sgemm_skinny_kernel<MRW, H, true>
                        : (const void *)sgemm_skinny_kernel<MRW, H, false>;
    hipError_t e = hipLaunchKernel(f, dim3(a.grid), dim3(kThreads), params, 0, s);
    if (e != hipSuccess || a.ipt <= 1) return e;
    const int64_t threads = (int64_t)a.M * ((a.N + 3) / 4);
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return hipLaunchKernel((const void *)sgemm_skinny_sum_kernel, dim3((unsigned)blocks), dim3(256), params, 0, s);
}

}  // namespace

hipError_t launch_skinny(int cfg, const KernelArgs &a, hipStream_t s) {
    if (cfg != SGEMM_CFG_SKINNY_16x256 || a.M < 1 || a.M > 16 || a.trans_b ||
        (a.ipt > 1 && !a.partials))
        return hipErrorInvalidValue;
    if (a.M <= 4) return launch_rows<4, 1>(a, s);
    if (a.M <= 8) return launch_rows<8, 1>(a, s);
    return launch_rows<8, 2>(a, s);
}

hipError_t occupancy_skinny(int cfg, int *wg_per_cu) {
    if (cfg != SGEMM_CFG_SKINNY_16x256) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(wg_per_cu, (const void *)sgemm_skinny_kernel<8, 2, true>, kThreads,
                                                        0);
}

}  // namespace sgemm
