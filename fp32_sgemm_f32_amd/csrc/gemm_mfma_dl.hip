// FP32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32) with the
// tiles moved from global memory straight into LDS (global_load_lds_dwordx4).
//
// The register-staged core (gemm_mfma.hip) loads a chunk into VGPRs and
// writes it to LDS a chunk later; a wave whose data has not arrived stalls
// on that write, and with one wave per SIMD (the 64x64 tiles that fill 256
// CUs at 1024 x 1024) the matrix core idles with it.  Here each lane names
// the global address of 16 bytes and the load itself deposits them in LDS,
// in lane order: no staging registers, no LDS write instructions, and the
// loads of a chunk may stay in flight for S-1 chunks of MFMAs (a ring of S
// LDS stages).  This is the role asynchronous global->shared copies play in
// "Beyond Kernel 7: Closing the Gap to cuBLAS on an H100 FP32 GEMM" (kernel
// 8, the multi-stage pipeline).
//
// LDS layout of one stage (a DMA instruction fills 1 KiB in lane order, so
// the layout is chosen through the global address each lane loads).  Each
// operand is kept in LDS the way it is stored in memory:
//   * k-contiguous (A stored M x K, B stored N x K): rows of BK floats, one
//     per m (n), no padding; the 16-byte quad Q of row r is stored at quad
//     position Q ^ swz(r), chosen so that the operand reads below hit
//     distinct banks (measured with the bank-conflict counter).
//   * m/n-contiguous (A stored K x M, B stored K x N): BK rows of BM (BN)
//     floats, one per k, as in memory.
// Operands: as in the register-staged core, lane half h (lanes 32h..32h+31)
// handles k in [h*BK/2, (h+1)*BK/2).  A k-contiguous operand gives four
// consecutive k of one row per ds_read_b128 (four MFMA steps).  An m/n-
// contiguous one is read along m (n): the wave's F fragments are
// interleaved, row (column) F*l + f of the wave tile belonging to fragment f,
// so a lane's F values for one k are adjacent (one b32/b64/b128 read per
// step).  B always uses the interleaved column order (a k-contiguous B gets
// it by loading its rows permuted), so the epilogue writes FN adjacent
// floats per store.
//
// Synchronisation of the ring (chunk c in stage c % S, S >= 3): chunks
// 0 .. S-2 are loaded up front; during chunk c the loads of chunk c+S-1 go
// out, spread over its groups, into the stage of chunk c-1.  Each chunk has
// one barrier, LA groups before its end: before it a wave waits until its
// loads of chunk c+1 have landed (S-3 later chunks and the part of chunk
// c+S-1 issued so far may stay in flight) and its LDS reads of chunk c are
// done; after it the waves read chunk c+1.  A two-stage double buffer (loads
// of chunk c+1 waited for within chunk c) measured 6-17% slower on MI355X:
// one chunk of MFMAs does not cover the load latency.  The compiler does not
// order these loads against LDS reads, so the waits and the barrier are
// explicit (s_waitcnt vmcnt(N)).
#include <utility>

#include "gemm_common.h"
#include "kernels.h"

namespace sgemm {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8; a field at its maximum does not wait.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
    static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
    constexpr int imm = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8);
    __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier that is also a compiler barrier for memory operations.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS byte address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const float *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float *)p;
}

// Operand reads from LDS.  They are issued as instructions of their own and
// waited for explicitly (lgkmcnt), so that reads for two groups ahead may be
// in flight: the compiler's own waits for these loads drain every
// outstanding LDS read.
template <int OFF>
__device__ __forceinline__ f32x4 lds_read4(uint32_t addr) {
    f32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ f32x2 lds_read2(uint32_t addr) {
    f32x2 v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ float lds_read1(uint32_t addr) {
    float v;
    asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// One LDS-DMA load: 16 bytes per lane from base + voff (a uniform 64-bit
// base and a per-lane 32-bit offset, so the address costs no vector ALU
// instruction) into LDS at m0 + 16 * lane.  m0 is set here; nothing else in
// these kernels keeps a value in it (gfx9 LDS instructions do not read it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char *base, uint32_t voff, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0v)
                 : "memory", "m0");
}

// The same from a buffer resource: lanes whose offset is out of the
// resource's range (>= 2^31 here) load nothing and leave zeros in LDS.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void bdma16(i32x4 rsrc, uint32_t voff, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(m0v)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource over [p, p + 2^31): base address, stride 0, 2^31
// records, default data format.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ i32x4 buffer_rsrc(const void *p) {
    const uint64_t a = (uint64_t)p;
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)kOutOfRange, 0x00020000};
}

__device__ __forceinline__ void advance_rsrc(i32x4 &r, int64_t bytes) {
    const uint64_t a = (((uint64_t)(uint32_t)r[1] << 32) | (uint32_t)r[0]) + (uint64_t)bytes;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)(uint32_t)(a >> 32);
}

// 1 if a == b, else 0, in a scalar register (a boolean would be kept in a
// vector register and tested with vector ALU instructions).
__device__ __forceinline__ int scalar_eq(int a, int b) {
    int r;
    asm("s_cmp_eq_u32 %1, %2\n\ts_cselect_b32 %0, 1, 0" : "=s"(r) : "s"(a), "s"(b) : "scc");
    return r;
}

template <int F>
struct FVec;
template <>
struct FVec<1> { typedef float T; };
template <>
struct FVec<2> { typedef f32x2 T; };
template <>
struct FVec<4> { typedef f32x4 T; };

template <int F, int OFF>
__device__ __forceinline__ typename FVec<F>::T lds_read_vec(uint32_t addr) {
    if constexpr (F == 1) return lds_read1<OFF>(addr);
    else if constexpr (F == 2) return lds_read2<OFF>(addr);
    else return lds_read4<OFF>(addr);
}

// One operand's registers for a group of four MFMA steps, F fragments.
// k-contiguous in LDS: a quad of four consecutive k per fragment.
// m/n-contiguous: per step, the F fragments' values at that step's k.
template <bool KC, int F>
struct GroupOps;
template <int F>
struct GroupOps<true, F> {
    f32x4 v[F];
    __device__ __forceinline__ float at(int u, int f) const { return v[f][u]; }
    __device__ __forceinline__ void keep() const {
#pragma unroll
        for (int f = 0; f < F; ++f) asm volatile("" ::"v"(v[f]));
    }
};
template <int F>
struct GroupOps<false, F> {
    typename FVec<F>::T v[4];
    __device__ __forceinline__ float at(int u, int f) const {
        if constexpr (F == 1) return v[u];
        else return v[u][f];
    }
    __device__ __forceinline__ void keep() const {
#pragma unroll
        for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(v[u]));
    }
};

// KSPLIT = 2 splits every chunk's K range between two groups of waves
// (sliced K): with one tile per CU the SIMDs then hold two waves each, one
// issuing MFMAs while the other waits; the groups' sums are added through
// LDS at the end of the tile.
// WS gives every MFMA wave a partner wave that only loads: it issues all of
// a chunk's LDS-DMA loads at the chunk's start and waits for them, and the
// MFMA waves only read LDS and multiply (two waves per SIMD).  Measured on
// the 128x128 tiles: +0.7% at 2048^3 and 2048x4096x2048 (alternating rounds,
// identical results); level on the 64x64 tiles, which keep one wave.
// EDGE: the shape need not be a multiple of the tile (the contiguous extent
// of each operand, and N, multiples of 4): loads through buffer resources
// with rows / columns / k beyond the matrix masked to zeros, stores masked.
// TA: A stored K x M (m-contiguous); TB: B stored N x K (k-contiguous).
// SH: the launch geometry, from the arguments or fixed at compile time for
// one product (gemm_common.h).
template <int BM_, int BN_, int BK_, int WAVES_M, int WAVES_N, int S_, int KSPLIT = 1, int LA_ = 1,
          bool EDGE = false, bool TA = false, bool TB = false, class SH = RuntimeShape, bool WS = false>
struct MfmaDlCore {
    using Shape = SH;
    static constexpr bool kEdge = EDGE;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
    static constexpr int LA = LA_;                  // groups of operand reads ahead of the MFMAs
    static constexpr int NS = LA == 1 ? 2 : 4;      // operand register sets
    static constexpr int NW_MN = WAVES_M * WAVES_N;   // waves per K group
    static constexpr int NW = NW_MN * KSPLIT;           // waves that issue MFMAs
    static constexpr int NT = 64 * NW * (WS ? 2 : 1);   // WS: as many more that only load
    static constexpr int NT_MN = 64 * NW_MN;          // threads holding the result
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KW = BK / KSPLIT;         // k values per wave per chunk
    static constexpr int KH = KW / 2;              // k values per lane half per chunk
    static constexpr int G = KH / 4;               // groups of four MFMA steps per chunk
    static constexpr int QPR = BK / 4;             // quads per k-contiguous row
    static constexpr bool AKC = !TA, BKC = TB;     // operand kept k-contiguous in LDS
    static constexpr int A_STAGE = BM * BK, B_STAGE = BK * BN;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_FLOATS = S * STAGE;
    static constexpr int A_INSTR = A_STAGE / 256, B_INSTR = B_STAGE / 256;   // 1 KiB DMA blocks
    static constexpr int A_PW = A_INSTR / NW, B_PW = B_INSTR / NW;           // per wave
    static constexpr int L = A_PW + B_PW;          // loads per wave per chunk
    static constexpr int TILE_FLOATS = BM * BN;
    typedef GroupOps<AKC, FM> AOps;
    typedef GroupOps<BKC, FN> BOps;

    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && (FM == 1 || FM == 2 || FM == 4) &&
                      (FN == 1 || FN == 2 || FN == 4),
                  "wave tile");
    static_assert(BK == 16 || BK == 32 || BK == 64, "swizzle defined for BK 16/32/64");
    static_assert(KSPLIT == 1 || KSPLIT == 2, "K groups");
    static_assert(LA == 1 || LA == 2, "read-ahead depth");
    static_assert(G > LA && G % NS == 0, "operand register sets rotate by group; the rotation must carry");
    static_assert((AKC || (BM <= 256 && 256 % BM == 0)) && (BKC || (BN <= 256 && 256 % BN == 0)),
                  "DMA block = whole rows of an m/n-contiguous operand");
    static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0 && A_PW >= 1 && B_PW >= 1,
                  "DMA blocks must split evenly over the waves");
    static_assert(S >= 3 && L * (S - 2) < 64, "ring depth (loads run S-2 chunks ahead) / vmcnt range");
    static_assert(LDS_FLOATS * 4 + 16 <= 160 * 1024, "LDS budget");
    static_assert(KSPLIT == 1 || TILE_FLOATS <= LDS_FLOATS, "room to add the K groups' sums");
    static_assert(!SH::kFixed || (!EDGE && !TA && !TB), "a compile-time shape: whole tiles, A M x K, B K x N");
    static_assert(!WS || KSPLIT == 1, "load waves with one K group");
    // Roles of a wave: both (not WS), or, with WS, MFMA waves and load waves.
    static constexpr int kBoth = 0, kMath = 1, kLoad = 2;

    floatx16 acc[FM][FN];
    int tiles_started = 0;   // uniform: tiles (or split ranges) this workgroup has begun

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }

    // Quad position of quad Q of a k-contiguous row r is Q ^ swz(r).  Each
    // was checked on gfx950 with the SQ_LDS_BANK_CONFLICT counter for the
    // operand reads below: none.  (For BK = 16, ((r >> 1) ^ (r >> 3)) & 3,
    // conflict-free in 32-bank and 64-bank models of the LDS, measured 4
    // extra cycles per ds_read_b128 on the hardware; (r >> 2) & 3 measured
    // none.)
    __device__ __forceinline__ static int swz(int r) {
        if constexpr (BK == 16) return (r >> 2) & 3;
        else if constexpr (BK == 32) return (r ^ (r >> 3)) & 7;
        else return r & 15;
    }

    // Tile column held by row r of a k-contiguous B stage: the rows are
    // loaded permuted so that fragment j's 32 columns (FN*l + j of the wave
    // tile, l = 0..31) sit in consecutive rows, read like A's.
    __device__ __forceinline__ static int b_kc_col(int r) {
        const int w = r / WTN, f = (r % WTN) / 32, l = r % 32;
        return w * WTN + FN * l + f;
    }

    // Per-lane addressing, computed once per tile.  The main loop holds no
    // vector ALU instruction: on gfx950 one between two dependent MFMAs
    // stalls the second for most of an MFMA's duration, so every address
    // the loop needs is either a register set up here or a scalar.
    struct Geo {
        const char *ga, *gb;     // uniform: A / B source of the next chunk to load
        i32x4 rsa, rsb;          // EDGE: the same as buffer resources
        int64_t a_step, b_step;  // uniform: bytes per chunk
        uint32_t va[A_PW];       // this lane's byte offset in each of its A DMA blocks
        uint32_t vb[B_PW];
        uint32_t va_t[A_PW];     // EDGE: the same for the tile's last chunk (K tail masked)
        uint32_t vb_t[B_PW];
        // LDS byte addresses of the operand reads, per stage: per fragment
        // and group for a k-contiguous operand (the swizzle moves each
        // quad), one base for an m/n-contiguous one (steps at fixed offsets).
        uint32_t ra[S][AKC ? FM : 1][AKC ? G : 1];
        uint32_t rb[S][BKC ? FN : 1][BKC ? G : 1];
        uint32_t lds;            // uniform: LDS byte address of the ring
        int wave;
        int dwave;               // uniform: this wave's index among the waves that load
    };

    // Source byte offset of this lane's 16 bytes in DMA block blk of an
    // operand (within the tile at chunk 0), whether it lies inside the matrix,
    // and whether it does in the tile's last chunk (k < kt).  KC: LDS row r
    // holds tile row src(r) (length BK); MC: LDS row kr holds k row kr
    // (length BX).  `lim` = valid rows (KC) or columns (MC) from the tile's
    // first.
    template <bool KC, int BX, class Src>
    __device__ __forceinline__ static void dma_lane(int blk, int lane, int64_t ld, int lim, int kt, Src src,
                                                    uint32_t &off, uint32_t &off_t) {
        uint32_t o;
        bool ok, ok_t;
        if constexpr (KC) {
            const int r = blk * (256 / BK) + lane / QPR;
            const int q = (lane % QPR) ^ swz(r);
            const int row = src(r);
            o = (uint32_t)(((int64_t)row * ld + 4 * q) * 4);
            ok = row < lim;
            ok_t = ok && 4 * q < kt;
        } else {
            const int kr = blk * (256 / BX) + lane / (BX / 4), cq = lane % (BX / 4);
            o = (uint32_t)(((int64_t)kr * ld + 4 * cq) * 4);
            ok = 4 * cq < lim;
            ok_t = ok && kr < kt;
        }
        off = !EDGE || ok ? o : kOutOfRange;
        off_t = !EDGE || ok_t ? o : kOutOfRange;
    }

    __device__ __forceinline__ void setup(Geo &g, const KernelArgs &a, float *lds, int tm, int tn, int k0) const {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        g.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        g.dwave = WS ? g.wave % NW : g.wave;
        // EDGE: valid k values in the tile's last chunk (a k-contiguous
        // operand needs K a multiple of 4, so its quads are all in or out).
        const int kt = EDGE ? a.K - (SH::ipt(a) - 1) * BK : BK;
        const int m_lim = a.M - tm * BM, n_lim = a.N - tn * BN;
#pragma unroll
        for (int u = 0; u < A_PW; ++u)
            dma_lane<AKC, BM>(g.dwave + NW * u, lane, SH::lda(a), m_lim, kt, [](int r) { return r; }, g.va[u],
                              g.va_t[u]);
#pragma unroll
        for (int u = 0; u < B_PW; ++u)
            dma_lane<BKC, BN>(g.dwave + NW * u, lane, SH::ldb(a), n_lim, kt, [](int r) { return b_kc_col(r); }, g.vb[u],
                              g.vb_t[u]);
        if constexpr (AKC) {
            g.ga = (const char *)(a.A + (int64_t)tm * BM * SH::lda(a) + (int64_t)k0 * BK);
            g.a_step = (int64_t)BK * 4;
        } else {
            g.ga = (const char *)(a.A + (int64_t)k0 * BK * SH::lda(a) + (int64_t)tm * BM);
            g.a_step = (int64_t)BK * SH::lda(a) * 4;
        }
        if constexpr (BKC) {
            g.gb = (const char *)(a.B + (int64_t)tn * BN * SH::ldb(a) + (int64_t)k0 * BK);
            g.b_step = (int64_t)BK * 4;
        } else {
            g.gb = (const char *)(a.B + (int64_t)k0 * BK * SH::ldb(a) + (int64_t)tn * BN);
            g.b_step = (int64_t)BK * SH::ldb(a) * 4;
        }
        if constexpr (EDGE) {
            g.rsa = buffer_rsrc(g.ga);
            g.rsb = buffer_rsrc(g.gb);
        }
        const int kg = g.wave / NW_MN, wmn = g.wave % NW_MN;
        const int wm = wmn / WAVES_N, wn = wmn % WAVES_N;
        const int lr = lane & 31, lh = lane >> 5;
        const uint32_t base = lds_addr(lds);
        g.lds = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
        for (int st = 0; st < S; ++st) {
            const uint32_t sa = base + 4 * st * STAGE, sb = sa + 4 * A_STAGE;
            if constexpr (AKC) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wm * WTM + i * 32 + lr;
#pragma unroll
                    for (int q = 0; q < G; ++q)
                        g.ra[st][i][q] = sa + 4 * (r * BK + 4 * ((kg * (KW / 4) + lh * G + q) ^ swz(r)));
                }
            } else {
                g.ra[st][0][0] = sa + 4 * ((kg * KW + lh * KH) * BM + wm * WTM + FM * lr);
            }
            if constexpr (BKC) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int r = wn * WTN + j * 32 + lr;
#pragma unroll
                    for (int q = 0; q < G; ++q)
                        g.rb[st][j][q] = sb + 4 * (r * BK + 4 * ((kg * (KW / 4) + lh * G + q) ^ swz(r)));
                }
            } else {
                g.rb[st][0][0] = sb + 4 * ((kg * KW + lh * KH) * BN + wn * WTN + FN * lr);
            }
        }
    }

    // DMA instruction d (A blocks first, then B blocks) of this wave for the
    // chunk at g.ga / g.gb (EDGE: g.rsa / g.rsb) into stage ST.
    template <int ST>
    __device__ __forceinline__ static void issue_one(const Geo &g, int d) {
        const uint32_t m0 = g.lds + 4 * (ST * STAGE + (d < A_PW ? 0 : A_STAGE) +
                                         (g.dwave + NW * (d < A_PW ? d : d - A_PW)) * 256);
        if constexpr (EDGE) {
            if (d < A_PW) bdma16(g.rsa, g.va[d], m0);
            else bdma16(g.rsb, g.vb[d - A_PW], m0);
        } else {
            if (d < A_PW) dma16(g.ga, g.va[d], m0);
            else dma16(g.gb, g.vb[d - A_PW], m0);
        }
    }

    // EDGE: before the loads of the tile's last chunk (its k beyond K
    // masked), which are the last loads of the tile: switch to the tail
    // offsets.  Vector moves, but once per tile.
    // (Volatile asm moves: plain assignments would be turned into selects
    // executed on every chunk.)
    __device__ __forceinline__ static void mask_k_tail(Geo &g) {
#pragma unroll
        for (int u = 0; u < A_PW; ++u) asm volatile("v_mov_b32 %0, %1" : "=v"(g.va[u]) : "v"(g.va_t[u]));
#pragma unroll
        for (int u = 0; u < B_PW; ++u) asm volatile("v_mov_b32 %0, %1" : "=v"(g.vb[u]) : "v"(g.vb_t[u]));
    }

    __device__ __forceinline__ static void advance(Geo &g) {
        if constexpr (EDGE) {
            advance_rsrc(g.rsa, g.a_step);
            advance_rsrc(g.rsb, g.b_step);
        } else {
            g.ga += g.a_step;
            g.gb += g.b_step;
        }
    }

    // Operands of group TQ (four MFMA steps) from stage ST: R read
    // instructions (one per fragment for a k-contiguous operand, one per
    // step for an m/n-contiguous one).
    static constexpr int R = (AKC ? FM : 4) + (BKC ? FN : 4);
    template <bool KC, int F, int BX, int ST, int TQ, int NF, int NQ>
    __device__ __forceinline__ static void read_ops(GroupOps<KC, F> &o, const uint32_t (&addr)[S][NF][NQ]) {
        if constexpr (KC) {
#pragma unroll
            for (int f = 0; f < F; ++f) o.v[f] = lds_read4<0>(addr[ST][f][TQ]);
        } else {
            o.v[0] = lds_read_vec<F, (4 * TQ + 0) * BX * 4>(addr[ST][0][0]);
            o.v[1] = lds_read_vec<F, (4 * TQ + 1) * BX * 4>(addr[ST][0][0]);
            o.v[2] = lds_read_vec<F, (4 * TQ + 2) * BX * 4>(addr[ST][0][0]);
            o.v[3] = lds_read_vec<F, (4 * TQ + 3) * BX * 4>(addr[ST][0][0]);
        }
    }
    template <int ST, int TQ>
    __device__ __forceinline__ static void read_group(const Geo &g, AOps &av, BOps &bv) {
        read_ops<AKC, FM, BM, ST, TQ>(av, g.ra);
        read_ops<BKC, FN, BN, ST, TQ>(bv, g.rb);
    }

    __device__ __forceinline__ void mfma_step(const AOps &av, const BOps &bv, int u) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av.at(u, i), bv.at(u, j), acc[i][j], 0, 0, 0);
    }

    // DMA instructions [dma_lo(q), dma_lo(q+1)) go out in group q: the
    // loads of a chunk are spread over the groups of the chunk before (a
    // wave issues one such load every few dozen cycles; a burst would
    // stall its MFMAs).
    __device__ __forceinline__ static constexpr int dma_lo(int q) { return q * L / G; }
    // Loads that may still be in flight at chunk c's barrier: S-3 whole
    // chunks and what was issued of chunk c+S-1.
    static constexpr int VM_AT_BARRIER = L * (S - 3) + dma_lo(G - LA);

    // 1 while chunk c still loads (c <= nch - S), else 0, in a scalar
    // register; volatile, so that each test gets its own.
    __device__ __forceinline__ static int steady_now(int c, int nch) {
        int r;
        asm volatile("s_cmp_le_i32 %1, %2\n\ts_cselect_b32 %0, 1, 0" : "=s"(r) : "s"(c), "s"(nch - S) : "scc");
        return r;
    }

    // Group Q of chunk c, in stage ST.  Stage ST+1 holds chunk c+1; stage
    // ST-1 (free since the barrier of chunk c-1) receives chunk c+S-1 over
    // the course of the chunk (STEADY only: the last S-1 chunks load
    // nothing).
    //   * The group's operands were read LA groups earlier: wait for them,
    //     then its first MFMA step.
    //   * Group G-LA holds the chunk's barrier: once chunk c+1 has landed
    //     (loads of later chunks may stay in flight: S-3 whole chunks and
    //     what the groups before issued of chunk c+S-1) and this wave's
    //     reads of chunk c are done, the waves may move on to chunk c+1.
    //   * The reads for group Q+LA (of this chunk or the next), then the
    //     other three MFMA steps with the group's DMA instructions spread
    //     after them.  Issuing an LDS-DMA load holds the wave for a few dozen
    //     cycles; behind the operand reads in one MFMA's shadow it delayed
    //     the next dependent MFMA (3% at one wave per SIMD).
    // Loads in flight at a load wave's barrier (WS): S-3 whole chunks and
    // chunk c+S-1, issued whole at the start of chunk c.
    static constexpr int VM_AT_BARRIER_LOAD = L * (S - 2);

    template <int ROLE, int ST, int Q>
    __device__ __forceinline__ void group(Geo &g, int c, int nch, int tail_ch, AOps (&av)[NS], BOps (&bv)[NS]) {
        // Whether this chunk still loads (c <= nch - S), computed afresh in a
        // scalar register at every test: one boolean shared by the group's
        // several tests would be carried across blocks in a vector register,
        // set and tested with vector ALU instructions.
#define SGEMM_DL_STEADY (steady_now(c, nch) != 0)
        constexpr int cs = Q % NS, TQ = Q + LA, ts = TQ % NS;
        constexpr int NXT = (ST + 1) % S, PRV = (ST + S - 1) % S;
        if constexpr (ROLE == kLoad) {
            // A load wave: the whole of chunk c+S-1 at the chunk's start,
            // then, in the group of the chunk's barrier, the wait for chunk
            // c+1 and the barrier, the same one the MFMA waves reach.
            if constexpr (Q == 0) {
                if (SGEMM_DL_STEADY) {
                    if constexpr (EDGE) {
                        if (scalar_eq(c + S - 1, tail_ch)) mask_k_tail(g);
                    }
#pragma unroll
                    for (int d = 0; d < L; ++d) issue_one<PRV>(g, d);
                    advance(g);
                }
            }
            if constexpr (TQ == G) {
                if (SGEMM_DL_STEADY) wait_counts<VM_AT_BARRIER_LOAD, 0>();
                else wait_counts<0, 0>();
                lds_barrier();
            }
            return;
        }
        wait_counts<63, (LA - 1) * R>();
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(av[cs], bv[cs], 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (TQ < G) {
            read_group<ST, TQ>(g, av[ts], bv[ts]);
        } else {
            if constexpr (TQ == G) {
                if (SGEMM_DL_STEADY) wait_counts<VM_AT_BARRIER, 0>();
                else wait_counts<0, 0>();
                lds_barrier();
            }
            read_group<NXT, TQ - G>(g, av[ts], bv[ts]);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(av[cs], bv[cs], 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ROLE == kBoth) {
            if (SGEMM_DL_STEADY) {
                if constexpr (EDGE && Q == 0) {
                    if (scalar_eq(c + S - 1, tail_ch)) mask_k_tail(g);
                }
                dma_slot<PRV, Q, 0>(g);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(av[cs], bv[cs], 2);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ROLE == kBoth && dma_lo(Q + 1) - dma_lo(Q) > 1) {
            if (SGEMM_DL_STEADY) dma_slot<PRV, Q, 1>(g);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(av[cs], bv[cs], 3);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ROLE == kBoth) {
            if (SGEMM_DL_STEADY) {
                if constexpr (dma_lo(Q + 1) - dma_lo(Q) > 2) dma_slot<PRV, Q, 2>(g);
                if constexpr (Q == G - 1) advance(g);
            }
        }
#undef SGEMM_DL_STEADY
        __builtin_amdgcn_sched_barrier(0);
    }

    // The group's DMA instructions d with (d - dma_lo(Q)) % 3 == SLOT: each
    // slot follows its own MFMA step, so that no step waits behind more
    // than a third of the group's loads.
    template <int PRV, int Q, int SLOT>
    __device__ __forceinline__ static void dma_slot(const Geo &g) {
#pragma unroll
        for (int d = dma_lo(Q); d < dma_lo(Q + 1); ++d)
            if ((d - dma_lo(Q)) % 3 == SLOT) issue_one<PRV>(g, d);
    }

    template <int ROLE, int ST, int... Qs>
    __device__ __forceinline__ void chunk_groups(std::integer_sequence<int, Qs...>, Geo &g, int c, int nch,
                                                 int tail_ch, AOps (&av)[NS], BOps (&bv)[NS]) {
        (group<ROLE, ST, Qs>(g, c, nch, tail_ch, av, bv), ...);
    }

    // Chunks ST, ST+1, ... of the ring from chunk c on; true once chunk
    // nch-1 is done.  Chunk c loads chunk c+S-1 while c <= nch-S.
    template <int ROLE, int ST>
    __device__ __forceinline__ bool chunks_from(int &c, int nch, int tail_ch, Geo &g, AOps (&av)[NS],
                                                BOps (&bv)[NS]) {
        chunk_groups<ROLE, ST>(std::make_integer_sequence<int, G>{}, g, c, nch, tail_ch, av, bv);
        if (++c >= nch) return true;
        if constexpr (ST + 1 < S) return chunks_from<ROLE, ST + 1>(c, nch, tail_ch, g, av, bv);
        else return false;
    }

    template <int ST>
    __device__ __forceinline__ static void issue_prologue(Geo &g, int nch, int tail_ch) {
        if constexpr (ST < S - 1) {
            if (ST < nch) {
                if constexpr (EDGE) {
                    if (ST == tail_ch) mask_k_tail(g);
                }
#pragma unroll
                for (int d = 0; d < L; ++d) issue_one<ST>(g, d);
                advance(g);
                issue_prologue<ST + 1>(g, nch, tail_ch);
            }
        }
    }

    __device__ __forceinline__ void mainloop(const KernelArgs &a, float *lds, int tm, int tn, int k0, int k1) {
        if constexpr (WS) {
            if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= NW) mainloop_role<kLoad>(a, lds, tm, tn, k0, k1);
            else mainloop_role<kMath>(a, lds, tm, tn, k0, k1);
        } else {
            mainloop_role<kBoth>(a, lds, tm, tn, k0, k1);
        }
    }

    // One role's part of the tile's K range.  Every barrier of it is in code
    // the roles share (the ring's start, one per chunk, one per later tile),
    // so the waves of a workgroup meet the same barriers in the same order.
    template <int ROLE>
    __device__ __forceinline__ void mainloop_role(const KernelArgs &a, float *lds, int tm, int tn, int k0, int k1) {
        Geo g;
        setup(g, a, lds, tm, tn, k0);
        int nch = k1 - k0;
        if constexpr (SH::kFixed) {
            // A compile-time shape makes the chunk count a constant; kept
            // opaque, so that the compiler keeps the loop over the ring as
            // written instead of unrolling or re-peeling it (which moved the
            // operand registers of the in-flight LDS reads).
            asm volatile("" : "+s"(nch));
        }
        // EDGE: the range's last chunk is the tile's last, with k beyond K,
        // when it reaches the end of a K not a multiple of BK.
        const int tail_ch =
            __builtin_amdgcn_readfirstlane(EDGE && k1 == SH::ipt(a) && a.K % BK != 0 ? nch - 1 : -1);

        // A previous tile of this workgroup may still read the ring (not
        // before the workgroup's first tile: its waves start on an idle
        // ring).
        if (tiles_started++ > 0) {
            wait_counts<0, 0>();
            lds_barrier();
        }
        // Chunks 0 .. S-2 up front (stage = chunk); chunk c+S-1 is loaded
        // during chunk c.
        if constexpr (ROLE != kMath) issue_prologue<0>(g, nch, tail_ch);
        if (nch >= S - 1) wait_counts<L * (S - 2), 0>();
        else wait_counts<0, 0>();
        lds_barrier();

        AOps av[NS];
        BOps bv[NS];
        if constexpr (ROLE != kLoad) {
            read_group<0, 0>(g, av[0], bv[0]);
            if constexpr (LA == 2) read_group<0, 1>(g, av[1], bv[1]);
        }

        int c = 0;
        while (!chunks_from<ROLE, 0>(c, nch, tail_ch, g, av, bv)) {
        }
        // The last groups read operands of a chunk that does not exist; the
        // registers must not be reused before those reads have returned.
        wait_counts<0, 0>();
        if constexpr (ROLE != kLoad) {
#pragma unroll
            for (int v = 0; v < NS; ++v) {
                av[v].keep();
                bv[v].keep();
            }
        }

        if constexpr (KSPLIT == 2) {
            // Group 1 hands its sums to group 0 through the (now idle) ring.
            const int tid = threadIdx.x;
            const int t = tid % NT_MN;
            wait_counts<0, 0>();
            lds_barrier();
            if (tid >= NT_MN) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) lds[((i * FN + j) * 16 + r) * NT_MN + t] = acc[i][j][r];
            }
            wait_counts<0, 0>();
            lds_barrier();
            if (tid < NT_MN) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[i][j][r] += lds[((i * FN + j) * 16 + r) * NT_MN + t];
            }
        }
    }

    // C element of block (i, j), register r, for this lane, with
    // rho = 8 (r / 4) + 4 (lane / 32) + r % 4 the MFMA's output row:
    //   row = 32 i + rho (A k-contiguous) or FM rho + i (A m-contiguous,
    //   fragments interleaved), col = FN (lane % 32) + j.
    // Only the first K group holds the result.  EDGE: rows beyond M and
    // columns beyond N are not written (N is a multiple of 4, so a lane's FN
    // adjacent columns are all in or all out).
    __device__ __forceinline__ void store_c(const KernelArgs &a, int tm, int tn) {
        const int tid = threadIdx.x;
        if ((KSPLIT > 1 || WS) && tid >= NT_MN) return;
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        const int lr = lane & 31, lh = lane >> 5;
        const int row0 = tm * BM + wm * WTM + (AKC ? 4 : 4 * FM) * lh, col0 = tn * BN + wn * WTN + FN * lr;
        if (EDGE && col0 >= a.cn) return;
        const int ldc = SH::ldc(a);
        float *c = a.C + (int64_t)row0 * ldc + col0;
        if (EDGE && a.c_scalar) {
            // C with a leading dimension or base off the vector grid, or
            // columns that end inside a lane's group: one float at a time.
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rho = 8 * (r >> 2) + (r & 3);
                    const int dr = AKC ? i * 32 + rho : FM * rho + i;
                    if (row0 + dr >= a.cm) continue;
                    float *p = c + (int64_t)dr * ldc;
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        if (col0 + j < a.cn) p[j] = epilogue(a, acc[i][j][r], p + j);
                }
            return;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rho = 8 * (r >> 2) + (r & 3);
                const int dr = AKC ? i * 32 + rho : FM * rho + i;
                if (EDGE && row0 + dr >= a.cm) continue;
                float *p = c + (int64_t)dr * ldc;
                // Non-temporal stores: nothing in this kernel reads C back
                // (measured +0.8-1% at 2048^3 and 1024^3, level at 4096^3).
                if constexpr (FN == 1) {
                    __builtin_nontemporal_store(epilogue(a, acc[i][0][r], p), p);
                } else if constexpr (FN == 2) {
                    __builtin_nontemporal_store(epilogue(a, f32x2{acc[i][0][r], acc[i][1][r]}, p), (f32x2 *)p);
                } else {
                    __builtin_nontemporal_store(
                        epilogue(a, f32x4{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]}, p), (f32x4 *)p);
                }
            }
    }

    // The same mapping into a dense row-major BM x BN tile (a split tile's
    // partial sum; whole tile, no masking, no epilogue).
    __device__ __forceinline__ void store_tile(float *p) {
        const int tid = threadIdx.x;
        if ((KSPLIT > 1 || WS) && tid >= NT_MN) return;
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / WAVES_N, wn = wave % WAVES_N;
        const int lr = lane & 31, lh = lane >> 5;
        float *q = p + (wm * WTM + (AKC ? 4 : 4 * FM) * lh) * BN + wn * WTN + FN * lr;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rho = 8 * (r >> 2) + (r & 3);
                float *d = q + (AKC ? i * 32 + rho : FM * rho + i) * BN;
                if constexpr (FN == 1) {
                    *d = acc[i][0][r];
                } else if constexpr (FN == 2) {
                    *(f32x2 *)d = f32x2{acc[i][0][r], acc[i][1][r]};
                } else {
                    *(f32x4 *)d = f32x4{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]};
                }
            }
    }
};

template <class Core, bool SPLIT>
__global__ __launch_bounds__(Core::NT) void sgemm_mfma_dl_kernel(KernelArgs a) {
    __shared__ __attribute__((aligned(1024))) float lds[Core::LDS_FLOATS];
    // Every argument the first tile needs, in scalar registers before
    // anything else: the compiler would otherwise load the tile-order fields,
    // branch on them, and only then load the operand pointers, two dependent
    // round trips to the argument memory before the first global load.
    using SH = typename Core::Shape;
    asm volatile("" ::"s"(a.A), "s"(a.B), "s"(a.C), "s"(SH::lda(a)), "s"(SH::ldb(a)), "s"(SH::ldc(a)),
                 "s"(SH::ipt(a)), "s"(SH::grid(a)), "s"(SH::dp_tiles(a)), "s"(SH::tiles_m(a)), "s"(SH::tiles_n(a)),
                 "s"(SH::group_m(a)), "s"(SH::xcd_remap(a)), "s"(a.scaled), "s"(a.alpha), "s"(a.beta));
    if constexpr (Core::kEdge)
        asm volatile("" ::"s"(a.M), "s"(a.N), "s"(a.K), "s"(a.cm), "s"(a.cn), "s"(a.c_scalar));
    run_gemm<Core, SPLIT, SH>(a, lds);
    // No load may still write this workgroup's LDS once its waves are gone.
    wait_counts<0, 0>();
}

using Dl64x64x32 = MfmaDlCore<64, 64, 32, 2, 2, 4, 1, 2>;
using Dl64x64x64K2 = MfmaDlCore<64, 64, 64, 2, 2, 3, 2, 2>;
using Dl128x128x32 = MfmaDlCore<128, 128, 32, 2, 2, 3, 1, 2, false, false, false, RuntimeShape, true>;
using Dl256x256x16 = MfmaDlCore<256, 256, 16, 4, 2, 3>;
using Dl64x64x32K2 = MfmaDlCore<64, 64, 32, 2, 2, 4, 2>;
using Dl128x128x32K2 = MfmaDlCore<128, 128, 32, 2, 2, 3, 2>;
using Dl64x64x64 = MfmaDlCore<64, 64, 64, 2, 2, 3, 1, 2>;
using Dl128x256x16 = MfmaDlCore<128, 256, 16, 2, 2, 3>;
using Dl256x128x16 = MfmaDlCore<256, 128, 16, 2, 2, 3>;
// The configurations the automatic choice uses, for each storage order of A
// and B (NN, TN, NT, TT): whole-tile variants (the NN one is defined above)
// and edge-masking ones.
#define SGEMM_DL_LAYOUT_CORES(name, BM, BN, BK, WM, WN, S, KS, LA, WS)                                  \
    using name##TN = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, false, true, false, RuntimeShape, WS>;  \
    using name##NT = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, false, false, true, RuntimeShape, WS>;  \
    using name##TT = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, false, true, true, RuntimeShape, WS>;   \
    using name##E = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, true, false, false, RuntimeShape, WS>;   \
    using name##ETN = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, true, true, false, RuntimeShape, WS>;  \
    using name##ENT = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, true, false, true, RuntimeShape, WS>;  \
    using name##ETT = MfmaDlCore<BM, BN, BK, WM, WN, S, KS, LA, true, true, true, RuntimeShape, WS>;
SGEMM_DL_LAYOUT_CORES(Dl64x64x32, 64, 64, 32, 2, 2, 4, 1, 2, false)
SGEMM_DL_LAYOUT_CORES(Dl64x64x64, 64, 64, 64, 2, 2, 3, 1, 2, false)
SGEMM_DL_LAYOUT_CORES(Dl128x128x32, 128, 128, 32, 2, 2, 3, 1, 2, true)
SGEMM_DL_LAYOUT_CORES(Dl256x256x16, 256, 256, 16, 4, 2, 3, 1, 1, false)
#undef SGEMM_DL_LAYOUT_CORES

// Kernels compiled for one product each (SGEMM_SCHED_FIXED): the automatic
// choice's configuration and tile order for the measured square and long-K
// products, in the order of kFixedShapes (plan.cpp).
using DlFixed4096 = MfmaDlCore<256, 256, 16, 4, 2, 3, 1, 1, false, false, false,
                               FixedShape<4096, 4096, 4096, 256, 256, 16, 4>>;
using DlFixed2048 = MfmaDlCore<128, 128, 32, 2, 2, 3, 1, 2, false, false, false,
                               FixedShape<2048, 2048, 2048, 128, 128, 32, 4>, true>;
using DlFixed1024 = MfmaDlCore<64, 64, 64, 2, 2, 3, 1, 2, false, false, false,
                               FixedShape<1024, 1024, 1024, 64, 64, 64, 4>>;
using DlFixed1024x16384 = MfmaDlCore<64, 64, 64, 2, 2, 3, 1, 2, false, false, false,
                                     FixedShape<1024, 1024, 16384, 64, 64, 64, 4>>;

template <class Core>
static hipError_t launch(const KernelArgs &a, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args};
    const void *f = a.sk_tiles > 0 ? (const void *)sgemm_mfma_dl_kernel<Core, true>
                                   : (const void *)sgemm_mfma_dl_kernel<Core, false>;
    return hipLaunchKernel(f, dim3(a.grid), dim3(Core::NT), params, 0, s);
}

template <class Core>
static hipError_t occ(int *n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, (const void *)sgemm_mfma_dl_kernel<Core, true>,
                                                        Core::NT, 0);
}

#define SGEMM_DL_CONFIGS(X)                         \
    X(SGEMM_CFG_DL_64x64x32, Dl64x64x32)            \
    X(SGEMM_CFG_DL_64x64x64_K2, Dl64x64x64K2)       \
    X(SGEMM_CFG_DL_128x128x32, Dl128x128x32)        \
    X(SGEMM_CFG_DL_256x256x16, Dl256x256x16)        \
    X(SGEMM_CFG_DL_64x64x32_K2, Dl64x64x32K2)       \
    X(SGEMM_CFG_DL_128x128x32_K2, Dl128x128x32K2)   \
    X(SGEMM_CFG_DL_64x64x64, Dl64x64x64)            \
    X(SGEMM_CFG_DL_128x256x16, Dl128x256x16)        \
    X(SGEMM_CFG_DL_256x128x16, Dl256x128x16)

#define SGEMM_DL_LAYOUT_CONFIGS(X)                \
    X(SGEMM_CFG_DL_64x64x32, Dl64x64x32)          \
    X(SGEMM_CFG_DL_64x64x64, Dl64x64x64)          \
    X(SGEMM_CFG_DL_128x128x32, Dl128x128x32)     \
    X(SGEMM_CFG_DL_256x256x16, Dl256x256x16)

hipError_t launch_mfma_dl(int cfg, const KernelArgs &a, hipStream_t s) {
    const int layout = (a.trans_a ? 1 : 0) | (a.trans_b ? 2 : 0);
    switch (cfg) {
#define X(id, core)                                                   \
    case id:                                                          \
        switch (layout | (a.edge ? 4 : 0)) {                          \
        case 0: return launch<core>(a, s);                            \
        case 1: return launch<core##TN>(a, s);                        \
        case 2: return launch<core##NT>(a, s);                        \
        case 3: return launch<core##TT>(a, s);                        \
        case 4: return launch<core##E>(a, s);                         \
        case 5: return launch<core##ETN>(a, s);                       \
        case 6: return launch<core##ENT>(a, s);                       \
        default: return launch<core##ETT>(a, s);                      \
        }
        SGEMM_DL_LAYOUT_CONFIGS(X)
#undef X
    default: break;
    }
    // The other configurations: whole tiles, A M x K and B K x N only.
    if (a.edge || layout) return hipErrorInvalidValue;
    switch (cfg) {
#define X(id, core) \
    case id: return launch<core>(a, s);
        SGEMM_DL_CONFIGS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

// A compile-time-shape kernel: whole tiles only, its own grid.
template <class Core>
static hipError_t launch_whole(const KernelArgs &a, hipStream_t s) {
    KernelArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel((const void *)sgemm_mfma_dl_kernel<Core, false>,
                           dim3(Core::Shape::TILES), dim3(Core::NT), params, 0, s);
}

// The compile-time-shape kernel kFixedShapes[idx]; the plan has checked
// that the call is that product (dense, whole tiles, data-parallel).
hipError_t launch_mfma_dl_fixed(int idx, const KernelArgs &a, hipStream_t s) {
    if (a.sk_tiles != 0) return hipErrorInvalidValue;
    switch (idx) {
    case 0: return launch_whole<DlFixed4096>(a, s);
    case 1: return launch_whole<DlFixed2048>(a, s);
    case 2: return launch_whole<DlFixed1024>(a, s);
    case 3: return launch_whole<DlFixed1024x16384>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t occupancy_mfma_dl(int cfg, int *wg_per_cu) {
    switch (cfg) {
#define X(id, core) \
    case id: return occ<core>(wg_per_cu);
        SGEMM_DL_CONFIGS(X)
#undef X
    default: return hipErrorInvalidValue;
    }
}

}  // namespace sgemm
