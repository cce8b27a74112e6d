// Device-side pieces shared by every kernel configuration: the kernel
// argument block, the workgroup -> work mapping (data-parallel tiles first,
// then the Stream-K share), and the deterministic sum of split tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

// Native 4-wide vector (one 128-bit load/store).  Arrays of it are promoted to
// registers, unlike arrays of HIP's float4 struct.
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Passed by value to every GEMM kernel.  Row-major A (M x K), B (K x N),
// C (M x N) with leading dimensions in elements.
struct KernelArgs {
    const float *A;
    const float *B;
    float *C;
    int lda, ldb, ldc;      // leading dimensions in elements (the API takes int)
    int M, N, K;      // the shape (the edge-masking kernels need it)
    int cm, cn;       // rows and columns of C to store (M, N unless the
                      // operands were padded beyond C: then C's own)
    int c_scalar;     // C's layout rules out vector stores (edge kernels)
    int edge;         // the shape is not a multiple of the tile
    int trans_a;      // A stored K x M (op(A) = A^T); else M x K
    int trans_b;      // B stored N x K (op(B) = B^T); else K x N
    int scaled;       // C = alpha * product + beta * C; else C = product
    float alpha, beta;
    int tiles_m, tiles_n;
    int ipt;          // K chunks per tile
    int dp_tiles;     // tiles [0, dp_tiles) are computed whole
    int sk_tiles;     // tiles [dp_tiles, dp_tiles + sk_tiles) are K-split
    int grid;         // workgroups launched
    int sk_grid;      // logical workgroups [0, sk_grid) share the split tiles
    int xcd_remap;    // remap blockIdx so each XCD owns a contiguous run of work
    int group_m;      // tile order: groups of group_m tile rows
    int64_t sk_iters; // sk_tiles * ipt
    float *partials;  // [sk_grid][2][tile rows][tile columns] partial tiles
};

// Value stored to C at p for a product value v: v itself for the plain
// product, else alpha * v + beta * C (C read only when beta != 0, so that C
// need not hold numbers then, as in BLAS).
template <class V>
__device__ __forceinline__ V epilogue(const KernelArgs &a, V v, const float *p) {
    if (!a.scaled) return v;
    V r = a.alpha * v;
    if (a.beta != 0.0f) r += a.beta * *(const V *)p;
    return r;
}

// The launch geometry as a kernel reads it.  RuntimeShape: from the
// argument block.  FixedShape: one dense row-major product C (M x N) =
// A (M x K) B (K x N), known when the kernel is compiled ("Beyond Kernel 7:
// Closing the Gap to cuBLAS on an H100 FP32 GEMM", section "Kernel 13", the
// size-specialised build): leading dimensions K, N, N, whole BM x BN tiles
// of BK-deep chunks, one workgroup per tile (data-parallel), the XCD remap,
// tile groups of GM rows; every field below is then a constant.
struct RuntimeShape {
    static constexpr bool kFixed = false;
    __device__ static int lda(const KernelArgs &a) { return a.lda; }
    __device__ static int ldb(const KernelArgs &a) { return a.ldb; }
    __device__ static int ldc(const KernelArgs &a) { return a.ldc; }
    __device__ static int ipt(const KernelArgs &a) { return a.ipt; }
    __device__ static int tiles_m(const KernelArgs &a) { return a.tiles_m; }
    __device__ static int tiles_n(const KernelArgs &a) { return a.tiles_n; }
    __device__ static int dp_tiles(const KernelArgs &a) { return a.dp_tiles; }
    __device__ static int grid(const KernelArgs &a) { return a.grid; }
    __device__ static int xcd_remap(const KernelArgs &a) { return a.xcd_remap; }
    __device__ static int group_m(const KernelArgs &a) { return a.group_m; }
};

template <int M, int N, int K, int BM, int BN, int BK, int GM>
struct FixedShape {
    static constexpr bool kFixed = true;
    static constexpr int TM = M / BM, TN = N / BN, TILES = TM * TN;
    static_assert(M % BM == 0 && N % BN == 0 && K % BK == 0, "whole tiles");
    static_assert(TILES % 8 == 0 && TM % GM == 0, "XCD remap and whole tile groups");
    __device__ static constexpr int lda(const KernelArgs &) { return K; }
    __device__ static constexpr int ldb(const KernelArgs &) { return N; }
    __device__ static constexpr int ldc(const KernelArgs &) { return N; }
    __device__ static constexpr int ipt(const KernelArgs &) { return K / BK; }
    __device__ static constexpr int tiles_m(const KernelArgs &) { return TM; }
    __device__ static constexpr int tiles_n(const KernelArgs &) { return TN; }
    __device__ static constexpr int dp_tiles(const KernelArgs &) { return TILES; }
    __device__ static constexpr int grid(const KernelArgs &) { return TILES; }
    __device__ static constexpr int xcd_remap(const KernelArgs &) { return 1; }
    __device__ static constexpr int group_m(const KernelArgs &) { return GM; }
};

// Workgroups are handed to the 8 XCDs round-robin by blockIdx.  With the
// remap, XCD x runs logical ids [x*grid/8, (x+1)*grid/8): neighbouring tiles
// (and the K-split pieces of one tile) land on one XCD and share its L2.
template <class SH = RuntimeShape>
__device__ __forceinline__ int logical_wg(const KernelArgs &a) {
    int w = (int)blockIdx.x;
    if (SH::xcd_remap(a)) {
        const int per = SH::grid(a) >> 3;
        w = (w & 7) * per + (w >> 3);
    }
    return w;
}

// Tile id -> (tile row, tile column): groups of group_m tile rows, walked
// down each column of the group before moving right.
template <class SH = RuntimeShape>
__device__ __forceinline__ void tile_coords(const KernelArgs &a, int t, int &tm, int &tn) {
    const int group_m = SH::group_m(a);
    const int gsz = group_m * SH::tiles_n(a);
    const int g = t / gsz;
    const int first = g * group_m;
    int rows = SH::tiles_m(a) - first;
    if (rows > group_m) rows = group_m;
    const int r = t - g * gsz;
    tm = first + r % rows;
    tn = r / rows;
}

// Stream-K partition of the sk_iters (tile, K chunk) steps over sk_grid
// workgroups: workgroup w owns [begin(w), begin(w + 1)).  The planner keeps
// sk_grid <= sk_iters (every owner has at least one step) and
// (sk_iters + 1) * sk_grid < 2^31, so 32-bit arithmetic is exact here.
__device__ __forceinline__ int sk_begin(const KernelArgs &a, int w) {
    return (int)((uint32_t)w * (uint32_t)a.sk_iters / (uint32_t)a.sk_grid);
}

// The workgroup whose range holds step i.
__device__ __forceinline__ int sk_owner(const KernelArgs &a, int i) {
    return (int)(((uint32_t)(i + 1) * (uint32_t)a.sk_grid - 1u) / (uint32_t)a.sk_iters);
}

// Partial slot of workgroup w for split tile tl: 0 if tl is the tile its
// range starts in, else 1 (its range can only leave a partial in its first
// and its last tile).
__device__ __forceinline__ int sk_slot(const KernelArgs &a, int w, int tl) {
    return sk_begin(a, w) / a.ipt == tl ? 0 : 1;
}

template <int TILE_FLOATS>
__device__ __forceinline__ float *partial_ptr(const KernelArgs &a, int w, int slot) {
    return a.partials + ((int64_t)w * 2 + slot) * TILE_FLOATS;
}

// Runs one workgroup's share of the GEMM with the given core.  The core
// provides:
//   zero()                          accumulators := 0
//   mainloop(a, lds, tm, tn, k0, k1) accumulate K chunks [k0, k1) of tile (tm, tn)
//   store_c(a, tm, tn)              write the accumulators to C
//   store_tile(p)                   write them to a dense row-major tile at p
//
// A split tile's contributors each leave their partial sum in the workspace
// and nothing else: sk_fixup (a second kernel on the same stream, which the
// kernel boundary orders after every partial is written) adds them and
// writes C.  No workgroup waits for, or synchronises with, another.
//
// SPLIT = false is the whole-tile-only instance (sk_tiles == 0): it carries
// none of the split bookkeeping, which keeps its register allocation to the
// main loop's needs.
//
// SH supplies the launch geometry (RuntimeShape, or a FixedShape for a
// kernel compiled for one product, which has no split part).
template <class Core, bool SPLIT, class SH = RuntimeShape>
__device__ __forceinline__ void run_gemm(const KernelArgs &a, float *lds) {
    static_assert(!(SPLIT && SH::kFixed), "a compile-time shape runs whole tiles only");
    Core core;
    const int w = logical_wg<SH>(a);

    for (int t = w; t < SH::dp_tiles(a); t += SH::grid(a)) {
        int tm, tn;
        tile_coords<SH>(a, t, tm, tn);
        core.zero();
        core.mainloop(a, lds, tm, tn, 0, SH::ipt(a));
        core.store_c(a, tm, tn);
    }
    if (!SPLIT || w >= a.sk_grid) return;

    int s = sk_begin(a, w);
    const int e = sk_begin(a, w + 1);
    while (s < e) {
        // Uniform bookkeeping first, while the accumulators are not yet live.
        const int tl = __builtin_amdgcn_readfirstlane(s / a.ipt);   // split-tile index
        const int k0 = s - tl * a.ipt;
        const int k1 = k0 + (e - s < a.ipt - k0 ? e - s : a.ipt - k0);
        int tm, tn;
        tile_coords(a, a.dp_tiles + tl, tm, tn);
        core.zero();
        core.mainloop(a, lds, tm, tn, k0, k1);
        if (k0 == 0 && k1 == a.ipt)
            core.store_c(a, tm, tn);   // the whole K range: not split after all
        else
            core.store_tile(partial_ptr<Core::TILE_FLOATS>(a, w, sk_slot(a, w, tl)));
        s += k1 - k0;
    }
}

// The sum of the split tiles: one thread per 4 adjacent outputs of a split
// tile (BM x BN, row-major in the partials).  Contributors are added in
// Stream-K order, first to last, whatever order they finished in, so the
// result is the same on every run.  Loads of up to 8 contributors are in
// flight at once; the sum itself stays in contributor order.  Rows and
// columns outside M x N are dropped; C is written with the epilogue.
template <int BM, int BN>
__device__ __forceinline__ void sk_fixup(const KernelArgs &a) {
    constexpr int QUADS = BM * BN / 4;
    const int64_t total = (int64_t)a.sk_tiles * QUADS;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int tl = (int)(q / QUADS);
        const int e = 4 * (int)(q - (int64_t)tl * QUADS);
        const int first = sk_owner(a, tl * a.ipt), last = sk_owner(a, (tl + 1) * a.ipt - 1);
        if (first == last) continue;   // stored whole by its only owner
        int tm, tn;
        tile_coords(a, a.dp_tiles + tl, tm, tn);
        const int row = tm * BM + e / BN, col = tn * BN + e % BN;
        if (row >= a.cm || col >= a.cn) continue;
        f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int c0 = first; c0 <= last; c0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (c0 + u <= last)
                    v[u] = *(const f32x4 *)(partial_ptr<BM * BN>(a, c0 + u, sk_slot(a, c0 + u, tl)) + e);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (c0 + u <= last) sum += v[u];
        }
        float *p = a.C + (int64_t)row * a.ldc + col;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (col + u < a.cn) p[u] = epilogue(a, sum[u], p + u);
    }
}

}  // namespace sgemm
