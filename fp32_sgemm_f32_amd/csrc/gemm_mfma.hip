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
//     of A rows and B rows, adjacent lanes on adjacent addresses; the next
//     chunk but one is in flight while the current chunk is multiplied
//     (register prefetch).
//   * registers -> LDS: two LDS stages (ping-pong), one barrier per chunk.
//     Both tiles are kept k-contiguous with rows padded to BK+4 floats: A as
//     loaded (row-major), B transposed on the way in (each lane loads R
//     consecutive k-rows of 4 columns and writes, per column, R consecutive
//     k values).  With a row stride of 4 x odd words, the operand reads
//     below are free of bank conflicts.
//   * LDS -> matrix cores: the waves tile the workgroup tile WAVES_M x
//     WAVES_N; a wave owns FM x FN blocks of 32x32.  Inside a chunk the K
//     index is permuted so that lane half h (lanes 32h .. 32h+31) works on
//     k in [h*BK/2, (h+1)*BK/2): each MFMA step p pairs k = p (half 0) with
//     k = BK/2 + p (half 1).  A sum is a sum, so the product is unchanged,
//     and a lane's operands for four consecutive steps are four consecutive
//     floats of its LDS row: one ds_read_b128 per 32-row block of A and one
//     per 32-column block of B feed four MFMA steps.
//   * epilogue: each lane owns 16 values of each 32x32 block; a lane half
//     writes 32 consecutive floats of a C row per store.
#include "gemm_common.h"
#include "kernels.h"

namespace sgemm {

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WAVES_M, int WAVES_N, int PF_ = 1>
struct MfmaCore {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int PF = PF_;                // chunks of global loads in flight (register sets)
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WTM = BM / WAVES_M;      // wave tile rows
    static constexpr int WTN = BN / WAVES_N;      // wave tile columns
    static constexpr int FM = WTM / 32;           // 32x32 blocks per wave, down
    static constexpr int FN = WTN / 32;           // 32x32 blocks per wave, across
    static constexpr int KH = BK / 2;             // k values per lane half per chunk
    static constexpr int G = KH / 4;              // groups of four MFMA steps per chunk
    static constexpr int LDK = BK + 4;            // LDS row stride of both tiles (floats)
    static constexpr int A_STAGE = BM * LDK;
    static constexpr int B_STAGE = BN * LDK;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_FLOATS = 2 * STAGE;
    static constexpr int A_VEC = BM * BK / 4 / NT;   // float4 loads of A per lane per chunk
    static constexpr int R = BK * BN / 4 / NT;       // k-rows of B per lane per chunk (4 columns each)
    static constexpr int RL = R >= 4 ? 4 : (R == 2 ? 8 : 16);   // lanes along k in the B loader
    static constexpr int A_ROWS_PER_PASS = NT / (BK / 4);
    static constexpr int TILE_FLOATS = BM * BN;

    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BK % 8 == 0, "BK/2 must be a multiple of 4 (one b128 per four steps)");
    static_assert(G % 2 == 0, "operand register sets alternate by group; the parity must carry");
    static_assert(A_VEC >= 1 && A_VEC * NT * 4 == BM * BK, "A tile must split evenly into float4s");
    static_assert((R == 1 || R == 2 || R == 4 || R == 8) && R * NT * 4 == BK * BN,
                  "B tile must split into R x 4 blocks");
    static_assert((LDK / 4) % 2 == 1, "row stride must be 4 x odd words");
    static_assert(PF == 1 || PF == 2, "prefetch depth");
    static_assert((BK / R) % RL == 0 && NT % (RL * (BN / 4)) == 0, "B loader lane map must tile the chunk");
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

    // Per-lane addressing, computed once per tile.
    struct Geo {
        const float *ga, *gb;   // next global A / B chunk of this lane
        int64_t ga_pass;        // A rows handled by the other passes
        int64_t gb_row;         // one k-row of B
        int64_t gb_chunk;       // one chunk of B rows
        int sa, sb;             // LDS store offsets within a stage
        int fa, fb;             // LDS operand offsets within a stage
    };

    // K loop over chunks [k0, k1) of tile (tm, tn).  A chunk is G groups of
    // four MFMA steps.  Schedule of chunk c (two LDS stages, two register
    // sets of operands, PF register sets of global loads, one barrier):
    //
    //   group 0:        read operands of group 1          | MFMAs of group 0
    //                   store chunk c+1 (loaded PF chunks ago) to the other
    //                   stage, issue global loads of chunk c+1+PF into the
    //                   register set just freed
    //   group g < G-1:  read operands of group g+1        | MFMAs of group g
    //   group G-1:      barrier,
    //                   read operands of group 0 of c+1   | MFMAs of group G-1
    //
    // The LDS stores land early in the chunk, so the barrier has nothing to
    // wait for but the other waves; the last group's MFMAs cover the barrier
    // and the next chunk's first LDS reads; the global loads have PF whole
    // chunks to land (two where registers allow: under full load the memory
    // latency exceeds one chunk of 256x256x16).  Stage safety: the stage
    // written in chunk c held chunk c-1, whose reads all finished before the
    // barrier ending chunk c-1; the barrier ending chunk c orders those writes
    // before their reads and every read of chunk c's stage before its next
    // write (in chunk c+1).  Chunks are unrolled in pairs so that stage and
    // register sets are compile-time.
    __device__ __forceinline__ void mainloop(const KernelArgs &a, float *lds, int tm, int tn,
                                             int k0, int k1) {
        const int tid = threadIdx.x;
        Geo g;
        {
            const int a_row = tid / (BK / 4), a_c4 = tid % (BK / 4);
            // B: columns 4*b_c4 .. +3, k rows R*b_kb .. +R-1.  Lanes vary the
            // k block fastest (RL of them), then the column block, so that the
            // lanes the LDS serves together (16 for b128 writes, 32 for b64)
            // land on 4 column blocks x RL k blocks: distinct banks, as the
            // column stride is 4 x LDK = 16 x odd words.  Each global load
            // instruction still covers whole 128-256 B row segments.
            const int b_c4 = (tid / RL) % (BN / 4);
            const int b_kb = tid % RL + RL * (tid / (RL * (BN / 4)));
            g.ga = a.A + ((int64_t)tm * BM + a_row) * a.lda + (int64_t)k0 * BK + a_c4 * 4;
            g.gb = a.B + ((int64_t)k0 * BK + b_kb * R) * a.ldb + (int64_t)tn * BN + b_c4 * 4;
            g.ga_pass = (int64_t)A_ROWS_PER_PASS * a.lda;
            g.gb_row = a.ldb;
            g.gb_chunk = (int64_t)BK * a.ldb;
            g.sa = a_row * LDK + a_c4 * 4;
            g.sb = A_STAGE + (b_c4 * 4) * LDK + b_kb * R;
            const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
            const int lane = tid & 63;
            const int wm = wave / WAVES_N, wn = wave % WAVES_N;
            const int lr = lane & 31, lh = lane >> 5;
            g.fa = (wm * WTM + lr) * LDK + lh * KH;
            g.fb = A_STAGE + (wn * WTN + lr) * LDK + lh * KH;
        }

        f32x4 ra[PF][A_VEC], rb[PF][R];
        f32x4 av[2][FM], bv[2][FN];

        const int nch = k1 - k0;
        // Prologue: chunk 0 into stage 0, chunks 1 .. PF in flight (chunk j in
        // register set j % PF), group 0 operands.
        load_global(g, ra[0], rb[0]);
        if (PF == 2 && nch > 1) {
            g.ga += BK;
            g.gb += g.gb_chunk;
            load_global(g, ra[PF - 1], rb[PF - 1]);
        }
        __syncthreads();                 // LDS may still be read by a previous tile
        store_lds(lds, g, ra[0], rb[0]);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        if (nch > PF) {
            g.ga += BK;
            g.gb += g.gb_chunk;
            load_global(g, ra[0], rb[0]);
            __builtin_amdgcn_sched_barrier(0);
        }
        read_operands(lds, 0, g, av[0], bv[0]);

        // Steady state without branches (every condition of chunks c, c+1
        // holds), so that no control-flow merge forces the compiler to wait
        // for outstanding LDS reads before the MFMAs; then the last chunks
        // with their conditions.
        int c = 0;
        for (; c + PF + 2 < nch; c += 2) {
            chunk<0, true>(c, nch, lds, g, ra, rb, av, bv);
            chunk<1, true>(c + 1, nch, lds, g, ra, rb, av, bv);
        }
        for (; c < nch; c += 2) {
            chunk<0, false>(c, nch, lds, g, ra, rb, av, bv);
            if (c + 1 < nch) chunk<1, false>(c + 1, nch, lds, g, ra, rb, av, bv);
        }
    }

    template <int ST, bool STEADY>
    __device__ __forceinline__ void chunk(int c, int nch, float *lds, Geo &g, f32x4 (&ra)[PF][A_VEC],
                                          f32x4 (&rb)[PF][R], f32x4 (&av)[2][FM], f32x4 (&bv)[2][FN]) {
        const float *cur = lds + ST * STAGE;
        float *nxt = lds + (ST ^ 1) * STAGE;
        constexpr int SET = PF == 2 ? (ST ^ 1) : 0;   // register set holding chunk c+1
        const bool more = STEADY || c + 1 < nch;
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int cb = q & 1;
            if (q + 1 < G) {
                read_operands(cur, (q + 1) * 4, g, av[cb ^ 1], bv[cb ^ 1]);
            } else if (more) {
                __syncthreads();
                read_operands(nxt, 0, g, av[cb ^ 1], bv[cb ^ 1]);
            }
            mfma_group(av[cb], bv[cb]);
            if (q == 0 && more) {
                store_lds(nxt, g, ra[SET], rb[SET]);
                if (STEADY || c + 1 + PF < nch) {
                    g.ga += BK;
                    g.gb += g.gb_chunk;
                    load_global(g, ra[SET], rb[SET]);
                }
                if (STEADY && INTERLEAVE_REFILL) {
                    interleave_refill_group();
                } else {
                    // Keep the loads here: the scheduler would otherwise sink
                    // them next to their use to shorten live ranges.
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if (STEADY) {
                interleave_reads_with_mfmas();
            }
        }
    }

    // Groups of at least 8 MFMAs interleave the refill with them; with fewer
    // (64-wide wave tiles) the refill stays a block of its own, which measured
    // faster there.
    static constexpr bool INTERLEAVE_REFILL = 4 * FM * FN >= 8;

    // Scheduling directive for group 0 of a chunk, which also refills: its
    // operand reads, then the LDS stores of the next chunk, then the global
    // loads of the chunk after, each placed after one MFMA, so that the wave
    // keeps issuing MFMAs throughout (a cluster of stores and loads would
    // stall the MFMA stream while the stores wait for their data), and the
    // loads stay a chunk ahead of their use.
    __device__ __forceinline__ static void interleave_refill_group() {
        constexpr int reads = FM + FN, mfmas = 4 * FM * FN;
        constexpr int writes = A_VEC + (R >= 4 ? R : 4), loads = A_VEC + R;
        constexpr int paired = reads + writes + loads < mfmas ? reads + writes + loads : mfmas;
#pragma unroll
        for (int i = 0; i < reads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
#pragma unroll
        for (int i = 0; i < writes; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // LDS write
        }
#pragma unroll
        for (int i = 0; i < loads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
        }
        if (mfmas > paired) __builtin_amdgcn_sched_group_barrier(0x008, mfmas - paired, 0);
    }

    // Scheduling directive for one group: its operand reads for the next
    // group go out one after each of the first MFMAs, so their latency is
    // covered by the rest of the group.  (Left alone, the scheduler delays
    // the reads to the end of the group to shorten register live ranges, and
    // the next group's first MFMAs then wait on them.)
    __device__ __forceinline__ static void interleave_reads_with_mfmas() {
        constexpr int reads = FM + FN, mfmas = 4 * FM * FN;
        static_assert(mfmas >= reads, "one MFMA per read");
#pragma unroll
        for (int i = 0; i < reads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, mfmas - reads, 0);
    }

    __device__ __forceinline__ static void load_global(const Geo &g, f32x4 (&ra)[A_VEC], f32x4 (&rb)[R]) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) ra[i] = *(const f32x4 *)(g.ga + i * g.ga_pass);
#pragma unroll
        for (int r = 0; r < R; ++r) rb[r] = *(const f32x4 *)(g.gb + r * g.gb_row);
    }

    // A as loaded; B transposed: column 4*b_c4 + i receives the R k-values
    // rb[0][i] .. rb[R-1][i] as one contiguous run.
    __device__ __forceinline__ static void store_lds(float *s, const Geo &g, const f32x4 (&ra)[A_VEC],
                                                     const f32x4 (&rb)[R]) {
#pragma unroll
        for (int i = 0; i < A_VEC; ++i) *(f32x4 *)(s + g.sa + i * A_ROWS_PER_PASS * LDK) = ra[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *d = s + g.sb + i * LDK;
            if constexpr (R == 1) {
                *d = rb[0][i];
            } else if constexpr (R == 2) {
                typedef float f32x2 __attribute__((ext_vector_type(2)));
                *(f32x2 *)d = f32x2{rb[0][i], rb[1][i]};
            } else {
#pragma unroll
                for (int r = 0; r < R; r += 4)
                    *(f32x4 *)(d + r) = f32x4{rb[r][i], rb[r + 1][i], rb[r + 2][i], rb[r + 3][i]};
            }
        }
    }

    // Operands of the four MFMA steps starting at step p.
    __device__ __forceinline__ static void read_operands(const float *s, int p, const Geo &g,
                                                         f32x4 (&av)[FM], f32x4 (&bv)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i) av[i] = *(const f32x4 *)(s + g.fa + i * 32 * LDK + p);
#pragma unroll
        for (int j = 0; j < FN; ++j) bv[j] = *(const f32x4 *)(s + g.fb + j * 32 * LDK + p);
    }

    __device__ __forceinline__ void mfma_group(const f32x4 (&av)[FM], const f32x4 (&bv)[FN]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][q], bv[j][q], acc[i][j], 0, 0, 0);
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
                for (int r = 0; r < 16; ++r) {
                    float *p = c + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * a.ldc + j * 32;
                    *p = epilogue(a, acc[i][j][r], p);
                }
    }

    // The same mapping into a dense row-major BM x BN tile (a split tile's
    // partial sum).
    __device__ __forceinline__ void store_tile(float *p) {
        const int tid = threadIdx.x;
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        const int lr = lane & 31, lh = lane >> 5;
        float *q = p + (wm * WTM + 4 * lh) * BN + wn * WTN + lr;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) q[(i * 32 + 8 * (r >> 2) + (r & 3)) * BN + j * 32] = acc[i][j][r];
    }
};

template <class Core, bool SPLIT>
__global__ __launch_bounds__(Core::NT) void sgemm_mfma_kernel(KernelArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[Core::LDS_FLOATS];
    run_gemm<Core, SPLIT>(a, lds);
}

using Mfma256x256x16 = MfmaCore<256, 256, 16, 4, 2>;
using Mfma128x128x32 = MfmaCore<128, 128, 32, 2, 2>;
using Mfma256x256x32 = MfmaCore<256, 256, 32, 2, 2>;
using Mfma256x128x32 = MfmaCore<256, 128, 32, 2, 2>;
using Mfma256x256x32W8 = MfmaCore<256, 256, 32, 4, 2>;
using Mfma128x128x32W8 = MfmaCore<128, 128, 32, 4, 2>;
using Mfma64x64x32 = MfmaCore<64, 64, 32, 2, 2>;
using Mfma128x64x32 = MfmaCore<128, 64, 32, 2, 2>;
using Mfma64x64x64 = MfmaCore<64, 64, 64, 2, 2>;
using Mfma128x128x64 = MfmaCore<128, 128, 64, 2, 2>;
using Mfma64x64x128 = MfmaCore<64, 64, 128, 2, 2>;

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
    case SGEMM_CFG_MFMA_256x256x32_W8: return launch<Mfma256x256x32W8>(a, s);
    case SGEMM_CFG_MFMA_128x128x32_W8: return launch<Mfma128x128x32W8>(a, s);
    case SGEMM_CFG_MFMA_64x64x32: return launch<Mfma64x64x32>(a, s);
    case SGEMM_CFG_MFMA_128x64x32: return launch<Mfma128x64x32>(a, s);
    case SGEMM_CFG_MFMA_64x64x64: return launch<Mfma64x64x64>(a, s);
    case SGEMM_CFG_MFMA_128x128x64: return launch<Mfma128x128x64>(a, s);
    case SGEMM_CFG_MFMA_64x64x128: return launch<Mfma64x64x128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t occupancy_mfma(int cfg, int *wg_per_cu) {
    switch (cfg) {
    case SGEMM_CFG_MFMA_256x256x16: return occ<Mfma256x256x16>(wg_per_cu);
    case SGEMM_CFG_MFMA_128x128x32: return occ<Mfma128x128x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_256x256x32: return occ<Mfma256x256x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_256x128x32: return occ<Mfma256x128x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_256x256x32_W8: return occ<Mfma256x256x32W8>(wg_per_cu);
    case SGEMM_CFG_MFMA_128x128x32_W8: return occ<Mfma128x128x32W8>(wg_per_cu);
    case SGEMM_CFG_MFMA_64x64x32: return occ<Mfma64x64x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_128x64x32: return occ<Mfma128x64x32>(wg_per_cu);
    case SGEMM_CFG_MFMA_64x64x64: return occ<Mfma64x64x64>(wg_per_cu);
    case SGEMM_CFG_MFMA_128x128x64: return occ<Mfma128x128x64>(wg_per_cu);
    case SGEMM_CFG_MFMA_64x64x128: return occ<Mfma64x64x128>(wg_per_cu);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sgemm
