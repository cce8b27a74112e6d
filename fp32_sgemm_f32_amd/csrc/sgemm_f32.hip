// C-ABI entry points of libsgemm_f32 (declared in include/sgemm_f32.h):
// argument checks, launch planning, the per-(device, stream) Stream-K
// workspace, and the kernel launch on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <utility>

#include "gemm_common.h"
#include "kernels.h"
#include "plan.h"
#include "sgemm_f32.h"

#define SGEMM_API extern "C" __attribute__((visibility("default")))

namespace sgemm {
namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return SGEMM_ERR_HIP;
}

struct DeviceInfo {
    bool ready = false;
    int num_cus = 0;
    int occupancy[SGEMM_NUM_CFGS] = {};
};

struct Workspace {
    float *partials = nullptr;
    int64_t partial_bytes = 0;
    float *pack = nullptr;         // repacked operands (see run_packed)
    int64_t pack_bytes = 0;
};

// Recursive: a repacked call holds it across its nested call of run().
std::recursive_mutex g_mu;
std::map<int, DeviceInfo> g_devices;
std::map<std::pair<int, hipStream_t>, Workspace> g_workspaces;

// Scratch memory of the no-allocation entry point (sgemm_f32_gemm_noalloc):
// the Stream-K partial tiles and the repacked copies of its calls, in a
// file-scope device array that every device running the library holds from
// module load to process exit.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): each device's
// copy is looked up once with hipGetSymbolAddress and kept in g_scratch.
constexpr int64_t kScratchBytes = SGEMM_F32_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
std::map<int, char *> g_scratch;   // device -> address of its copy of `scratch`

hipError_t launch_cfg(int cfg, const KernelArgs &a, hipStream_t s, int trans_c = 0) {
    switch (kCfgs[cfg].kind) {
    case kKindMfma: return launch_mfma(cfg, a, s);
    case kKindMfmaDl: return launch_mfma_dl(cfg, a, s);
    case kKindGeneric: return launch_generic(cfg, a, s);
    case kKindSkinny: return launch_skinny(cfg, a, s, trans_c);
    case kKindRowdot: return launch_rowdot(cfg, a, s, trans_c);
    default: return launch_valu(cfg, a, s);
    }
}

hipError_t occupancy_of(int cfg, int *n) {
    switch (kCfgs[cfg].kind) {
    case kKindMfma: return occupancy_mfma(cfg, n);
    case kKindMfmaDl: return occupancy_mfma_dl(cfg, n);
    case kKindGeneric: return occupancy_generic(cfg, n);
    case kKindSkinny: return occupancy_skinny(cfg, n);
    case kKindRowdot: return occupancy_rowdot(cfg, n);
    default: return occupancy_valu(cfg, n);
    }
}

int env_int(const char *name, int dflt) {
    const char *v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

// Compute-unit count and per-configuration occupancy of the current device
// (queried once per device).
int device_info(int dev, DeviceInfo *out) {
    std::lock_guard<std::recursive_mutex> lock(g_mu);
    DeviceInfo &d = g_devices[dev];
    if (!d.ready) {
        int cus = 0;
        hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e);
        d.num_cus = cus;
        for (int c = 1; c < SGEMM_NUM_CFGS; ++c) {
            int n = 0;
            e = occupancy_of(c, &n);
            if (e != hipSuccess) return hip_fail(e);
            d.occupancy[c] = n > 0 ? n : 1;
        }
        d.ready = true;
    }
    *out = d;
    return SGEMM_OK;
}

// Device address of the scratch array on device dev (current), looked up on
// the first call for that device.
int scratch_of(int dev, char **out) {
    std::lock_guard<std::recursive_mutex> lock(g_mu);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!ptr) return hip_fail(hipErrorInvalidSymbol);
        it = g_scratch.emplace(dev, (char *)ptr).first;
    }
    *out = it->second;
    return SGEMM_OK;
}

// A device pointer of the current device whose allocation holds `bytes`
// bytes from p on.
int check_device_range(const void *p, int64_t bytes, int dev) {
    if (bytes <= 0) return SGEMM_OK;
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // not HIP-known memory: do not leave a sticky error behind
        return SGEMM_ERR_POINTER;
    }
    if (attr.type != hipMemoryTypeDevice || attr.device != dev) return SGEMM_ERR_POINTER;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    e = hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return SGEMM_ERR_POINTER;
    }
    const uintptr_t lo = (uintptr_t)base, hi = lo + size, q = (uintptr_t)p;
    if (q < lo || q + (uint64_t)bytes > hi) return SGEMM_ERR_POINTER;
    return SGEMM_OK;
}

// Bytes spanned by a row-major rows x cols matrix with leading dimension ld.
int64_t extent_bytes(int rows, int cols, int ld) {
    if (rows <= 0 || cols <= 0) return 0;
    return ((int64_t)(rows - 1) * ld + cols) * 4;
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb) {
    if (na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uint64_t)nb && b0 < a0 + (uint64_t)na;
}

// One call: C = op(A) op(B) (plain), or alpha op(A) op(B) + beta C (scaled).
struct Call {
    int M, N, K;
    int ta, tb;                    // A stored K x M / B stored N x K
    const float *A, *B;
    float *C;
    int lda, ldb, ldc;
    int scaled;
    float alpha, beta;
    hipStream_t stream;
    int config, sched;
    int repacked = 0;              // already laid out for the vector kernels by run_packed
    int cm = 0, cn = 0;            // C's rows and columns when the operands were padded
                                   // beyond them (run_packed); 0: M and N
    int tc = 0;                    // C stored N x M: the transposed product of a thin
                                   // call (transposed_route)
    char *scratch = nullptr;       // set: take the Stream-K partials and the repacked
    int64_t scratch_bytes = 0;     // copies from here (the device address of the
                                   // no-allocation scratch array), allocate nothing

    // Rows and columns of C, and of A and B as stored.
    int c_rows() const { return tc ? N : cm ? cm : M; }
    int c_cols() const { return tc ? M : cn ? cn : N; }
    int a_rows() const { return ta ? K : M; }
    int a_cols() const { return ta ? M : K; }
    int b_rows() const { return tb ? N : K; }
    int b_cols() const { return tb ? K : N; }
    // A and B are read only when the product contributes.
    bool reads_ab() const { return K > 0 && !(scaled && alpha == 0.0f); }
};

// Host-only checks (no HIP call).  Order: shape, ld, null, alignment, alias.
int check_args(const Call &c) {
    if (c.M < 0 || c.N < 0 || c.K < 0) return SGEMM_ERR_SHAPE;
    if (c.M == 0 || c.N == 0) return SGEMM_OK;
    const bool ab = c.reads_ab();
    // A and B (and their leading dimensions) are not read when the product
    // does not contribute.
    if (c.ldc < c.c_cols() || (ab && (c.lda < c.a_cols() || c.ldb < c.b_cols()))) return SGEMM_ERR_LD;
    if (!c.C || (ab && (!c.A || !c.B))) return SGEMM_ERR_NULL;
    if (((uintptr_t)c.C & 3) || (ab && (((uintptr_t)c.A & 3) || ((uintptr_t)c.B & 3)))) return SGEMM_ERR_ALIGN;
    const int64_t nc = extent_bytes(c.c_rows(), c.c_cols(), c.ldc);
    if (ab && (overlap(c.C, nc, c.A, extent_bytes(c.a_rows(), c.a_cols(), c.lda)) ||
               overlap(c.C, nc, c.B, extent_bytes(c.b_rows(), c.b_cols(), c.ldb))))
        return SGEMM_ERR_ALIAS;
    return SGEMM_OK;
}

// The layout the vector (16-byte) kernels need: the contiguous extent and
// the leading dimension of every operand a multiple of 4, and 16-byte
// aligned operands; anything else runs on the general kernel.  Loads (A, B
// and N, the column count the tiles cover) and C stores separately.
bool vector_ab(const Call &c) {
    return (c.a_cols() & 3) == 0 && (c.b_cols() & 3) == 0 && (c.N & 3) == 0 && (c.lda & 3) == 0 &&
           (c.ldb & 3) == 0 && ((uintptr_t)c.A & 15) == 0 && ((uintptr_t)c.B & 15) == 0;
}

bool vector_c(const Call &c) {
    return (c.c_cols() & 3) == 0 && (c.ldc & 3) == 0 && ((uintptr_t)c.C & 15) == 0;
}

bool vector_layout(const Call &c) { return vector_ab(c) && vector_c(c); }

// Kernels that read A or B and write C one float at a time where needed, so
// that no layout calls for repacking them.
bool any_layout(int cfg) { return kCfgs[cfg].kind == kKindSkinny || kCfgs[cfg].kind == kKindRowdot; }

// Thin products whose stored layout the thin kernels cannot read, run as
// the transposed product C^T = op(B)^T op(A)^T with C written transposed:
// - few rows (M <= 8) with B stored N x K, as in x W^T with W row-major (the
//   tiled kernels spend a 64-row tile on them, the skinny kernel reads B
//   along N): on the row-dot kernel, B's rows streamed, where that kernel's
//   own rule would take the shape (at most 2 rows, B of 2^26 elements or
//   more, or a layout the tiled kernels cannot load);
// - few columns (N <= 16) with A stored K x M, as in X^T v (the row-dot
//   kernel reads A along K): on the skinny kernel, A's rows streamed, where
//   its own rule would take the shape (at most 8 columns, A above 2^22
//   elements, or a layout the tiled kernels cannot load).
// Returns the configuration of the transposed product, or SGEMM_CFG_AUTO
// for none.
int transposed_route(const Call &c) {
    if (c.config != SGEMM_CFG_AUTO || c.tc || c.repacked || c.cm || c.cn || c.K < 256 || !c.reads_ab())
        return SGEMM_CFG_AUTO;
    if (c.tb && c.M <= 8 && c.N >= 256 &&
        (c.M <= 2 || (int64_t)c.N * c.K >= ((int64_t)1 << 26) || !vector_layout(c)) &&
        (c.sched != SGEMM_SCHED_DP || c.K <= kRowdotFloats / rowdot_cols(c.M)))   // DP: B's K range in LDS
        return SGEMM_CFG_ROWDOT_N8;
    if (c.ta && c.N <= 16 && c.M >= 256 &&
        (c.N <= 8 || (int64_t)c.M * c.K > ((int64_t)1 << 22) || !vector_layout(c)))
        return SGEMM_CFG_SKINNY_16x256;
    return SGEMM_CFG_AUTO;
}

// That transposed call on configuration cfg: A' = op(B)^T, stored as B is
// (B stored N x K is A' stored M' x K; B stored K x N is A' stored K x M'),
// B' = op(A)^T likewise, C' = C^T.
Call transposed(const Call &c, int cfg) {
    Call q = c;
    q.M = c.N; q.N = c.M;
    q.A = c.B; q.lda = c.ldb; q.ta = c.tb ? 0 : 1;
    q.B = c.A; q.ldb = c.lda; q.tb = c.ta ? 0 : 1;
    q.tc = 1;
    q.config = cfg;
    return q;
}

// Stream-K workspace of (dev, stream), grown to hold `plan`'s partial
// tiles.  Caller holds g_mu.
int workspace_for(int dev, hipStream_t s, const Plan &p, Workspace *out) {
    Workspace &w = g_workspaces[{dev, s}];
    const int64_t need_part = p.workspace_bytes;
    if (w.partial_bytes < need_part) {
        hipError_t e = hipStreamSynchronize(s);   // the old buffer may still be in use
        if (e != hipSuccess) return hip_fail(e);
        if (w.partials) (void)hipFree(w.partials);
        w.partials = nullptr;
        w.partial_bytes = 0;
        e = hipMalloc((void **)&w.partials, (size_t)need_part);
        if (e != hipSuccess) return hip_fail(e);
        w.partial_bytes = need_part;
    }
    *out = w;
    return SGEMM_OK;
}

// Repacking buffer of (dev, stream) holding at least `bytes`.  Takes g_mu.
int pack_space_for(int dev, hipStream_t s, int64_t bytes, float **out) {
    std::lock_guard<std::recursive_mutex> lock(g_mu);
    Workspace &w = g_workspaces[{dev, s}];
    if (w.pack_bytes < bytes) {
        hipError_t e = hipStreamSynchronize(s);   // the old buffer may still be in use
        if (e != hipSuccess) return hip_fail(e);
        if (w.pack) (void)hipFree(w.pack);
        w.pack = nullptr;
        w.pack_bytes = 0;
        e = hipMalloc((void **)&w.pack, (size_t)bytes);
        if (e != hipSuccess) return hip_fail(e);
        w.pack_bytes = bytes;
    }
    *out = w.pack;
    return SGEMM_OK;
}

int run(const Call &c);

inline int up4(int x) { return (x + 3) & ~3; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Products of at least this many multiply-adds whose layout the vector
// kernels cannot load are repacked rather than run on the general kernel.
// Measured on MI355X (N odd, M = K = N - 1): the general kernel is faster at
// 256^3 (17 vs 20 us, the copies' launches dominate), the repacked product
// from 384^3 on (20 vs 25 us) and 3.3x faster at 2048^3; 2^25 ~ 322^3 lies
// between.
constexpr int64_t kRepackMinMacs = (int64_t)1 << 25;

bool worth_repacking(const Call &c) {
    const char *v = std::getenv("SGEMM_F32_REPACK_MIN_MACS");
    const int64_t lim = v && *v ? std::atoll(v) : kRepackMinMacs;
    // Any side length: where a thin kernel takes the product (any layout)
    // the plan has chosen it and nothing is repacked; elsewhere the general
    // kernel is the alternative (16384 x 9 x 16384 with B's rows of 9
    // floats: 1204 us there, about 274 for a 12-column padded copy on the
    // tiled kernel).
    return lim >= 0 && (int64_t)c.M * c.N * c.K >= lim;
}

// The same product on copies laid out for the vector kernels: every stored
// row length of A and B (and N, and M when A is stored K x M) padded to a
// multiple of 4 with zeros, 16-byte aligned rows; the padded k terms are
// 0 * 0.  A, B are copied only when their own layout does not already
// qualify.  C is written in place: the kernels store only its own rows and
// columns (one float at a time when its layout rules out vector stores), so
// it is neither copied in nor back.  All on the caller's stream, in the
// library's per-stream repacking buffer.
//
// The lock is held from taking the buffer to the last launch of the product:
// another thread's call on the same stream could otherwise enqueue its own
// copies into the same buffer between this call's copy and its GEMM, or
// grow the buffer (free it) before this call's copy is enqueued.
int run_packed(const Call &c, int dev) {
    std::lock_guard<std::recursive_mutex> lock(g_mu);
    const int Mp = c.ta ? up4(c.M) : c.M, Np = up4(c.N), Kp = up4(c.K);
    const int ar = c.ta ? Kp : Mp, ac = c.ta ? Mp : Kp;     // A as stored, padded
    const int br = c.tb ? Np : Kp, bc = c.tb ? Kp : Np;
    const bool pa = !(aligned16(c.A) && (c.lda & 3) == 0 && c.a_rows() == ar && c.a_cols() == ac);
    const bool pb = !(aligned16(c.B) && (c.ldb & 3) == 0 && c.b_rows() == br && c.b_cols() == bc);
    auto round256 = [](int64_t b) { return (b + 255) / 256 * 256; };
    const int64_t a_bytes = pa ? round256((int64_t)ar * ac * 4) : 0;
    const int64_t b_bytes = pb ? round256((int64_t)br * bc * 4) : 0;
    float *buf = nullptr;
    int st = SGEMM_OK;
    if (c.scratch) {
        // No allocation: the copies at the start of the scratch array.
        if (a_bytes + b_bytes > c.scratch_bytes) return SGEMM_ERR_SCRATCH;
        buf = (float *)c.scratch;
    } else if (a_bytes + b_bytes > 0 &&
               (st = pack_space_for(dev, c.stream, a_bytes + b_bytes, &buf)) != SGEMM_OK) {
        return st;
    }
    float *Ap = buf, *Bp = (float *)((char *)buf + a_bytes);
    PackJob jobs[2];
    int njobs = 0;
    if (pa) jobs[njobs++] = PackJob{c.A, c.lda, c.a_rows(), c.a_cols(), Ap, ac, ar, ac};
    if (pb) jobs[njobs++] = PackJob{c.B, c.ldb, c.b_rows(), c.b_cols(), Bp, bc, br, bc};
    const hipError_t e = launch_pack(jobs, njobs, c.stream);
    if (e != hipSuccess) return hip_fail(e);

    Call q = c;
    q.M = Mp; q.N = Np; q.K = Kp;
    if (pa) { q.A = Ap; q.lda = ac; }
    if (pb) { q.B = Bp; q.ldb = bc; }
    if (Mp != c.M || Np != c.N || !vector_c(c)) { q.cm = c.M; q.cn = c.N; }
    q.repacked = 1;
    if (c.scratch) {   // the rest of the array for the product's partial tiles
        q.scratch = c.scratch + a_bytes + b_bytes;
        q.scratch_bytes = c.scratch_bytes - (a_bytes + b_bytes);
    }
    return run(q);
}

int run(const Call &c) {
    int st = check_args(c);
    if (st != SGEMM_OK) return st;
    if (c.config < 0 || c.config >= SGEMM_NUM_CFGS) return SGEMM_ERR_CONFIG;
    if (c.sched < SGEMM_SCHED_AUTO || c.sched > SGEMM_SCHED_FIXED) return SGEMM_ERR_CONFIG;
    if (c.M == 0 || c.N == 0) return SGEMM_OK;
    // The compile-time-shape kernels know the leading dimensions and run
    // the plain product only: anything else is refused before any work.
    if (c.sched == SGEMM_SCHED_FIXED &&
        (c.ta || c.tb || c.tc || c.repacked || c.cm || c.cn || !c.reads_ab() || c.lda != c.K || c.ldb != c.N ||
         c.ldc != c.N || !vector_layout(c) || (c.scaled && !(c.alpha == 1.0f && c.beta == 0.0f))))
        return SGEMM_ERR_CONFIG;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if ((st = check_device_range(c.C, extent_bytes(c.c_rows(), c.c_cols(), c.ldc), dev)) != SGEMM_OK) return st;
    // Repacked operands are the library's own copies, the caller's were
    // checked before they were copied.
    if (c.reads_ab() && !c.repacked) {
        if ((st = check_device_range(c.A, extent_bytes(c.a_rows(), c.a_cols(), c.lda), dev)) != SGEMM_OK) return st;
        if ((st = check_device_range(c.B, extent_bytes(c.b_rows(), c.b_cols(), c.ldb), dev)) != SGEMM_OK) return st;
    }

    const int tcfg = transposed_route(c);
    if (tcfg != SGEMM_CFG_AUTO) return run(transposed(c, tcfg));

    // C written in place beyond padded operands (run_packed): the edge
    // variants store only C's own rows and columns.
    const bool c_own = c.cm != 0 || c.cn != 0;
    DeviceInfo info;
    if ((st = device_info(dev, &info)) != SGEMM_OK) return st;
    PlanRequest req{c.M, c.N, c.K, c.config, c.sched, info.num_cus, info.occupancy,
                    env_int("SGEMM_F32_SK_WG_PER_CU", 0), vector_ab(c) && (c_own || vector_c(c)) ? 1 : 0,
                    c.ta, c.tb};
    Plan p;
    if ((st = make_plan(req, &p)) != SGEMM_OK) return st;
    // An automatic choice other than the kernels that take any layout of
    // their small operands, on a layout the vector kernels cannot load:
    // large products run on repacked copies.
    if (!c.repacked && c.config == SGEMM_CFG_AUTO && c.reads_ab() && !any_layout(p.config) && !vector_layout(c) &&
        worth_repacking(c))
        return run_packed(c, dev);
    if (c_own) p.edge = 1;
    if (c.K > 0 && !dl_offsets_fit(p.config, p.edge != 0, c.lda, c.ldb, c.ta != 0, c.tb != 0)) {
        // Leading dimensions too large for the 32-bit source offsets of the
        // direct-to-LDS kernels: an automatic choice falls back to the
        // register-staged kernel of the same tile (the general one when the
        // tile does not divide the shape or an operand is transposed, which
        // the staged kernels do not load); a forced one is refused.
        if (c.config != SGEMM_CFG_AUTO) return SGEMM_ERR_CONFIG;
        req.config = p.edge || c.ta || c.tb ? SGEMM_CFG_GENERIC_64x64x16 : staged_equivalent(p.config);
        if ((st = make_plan(req, &p)) != SGEMM_OK) return st;
    }
    if (c.scratch && p.workspace_bytes > c.scratch_bytes) {
        // No allocation, and the split tiles' partials do not fit the
        // scratch array: the same configuration with whole tiles only.
        req.config = p.config;
        req.sched = SGEMM_SCHED_DP;
        if (make_plan(req, &p) != SGEMM_OK || p.workspace_bytes > c.scratch_bytes) return SGEMM_ERR_SCRATCH;
        if (c_own) p.edge = 1;
    }

    if (!c.reads_ab()) {
        // No product: C = beta * C (zeros for the plain product, K == 0).
        e = launch_scale_c(c.C, c.M, c.N, c.ldc, c.scaled ? c.beta : 0.0f, c.stream);
        return e == hipSuccess ? SGEMM_OK : hip_fail(e);
    }

    KernelArgs a{};
    a.A = c.A; a.B = c.B; a.C = c.C;
    a.lda = c.lda; a.ldb = c.ldb; a.ldc = c.ldc;
    a.M = c.M; a.N = c.N; a.K = c.K;
    a.cm = c.c_rows(); a.cn = c.c_cols();
    a.c_scalar = c_own && !vector_c(c) ? 1 : 0;
    a.edge = p.edge;
    a.trans_a = c.ta; a.trans_b = c.tb;
    a.scaled = c.scaled && !(c.alpha == 1.0f && c.beta == 0.0f);
    a.alpha = c.alpha; a.beta = c.beta;
    a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n; a.ipt = p.ipt;
    a.dp_tiles = p.dp_tiles; a.sk_tiles = p.sk_tiles;
    a.grid = p.grid; a.sk_grid = p.sk_grid;
    a.xcd_remap = env_int("SGEMM_F32_XCD_REMAP", 1) ? p.xcd_remap : 0;
    a.group_m = env_int("SGEMM_F32_GROUP_M", 0) > 0 ? env_int("SGEMM_F32_GROUP_M", 0) : p.group_m;
    a.sk_iters = p.sk_iters;

    if (p.sk_tiles > 0) {
        // Workspace acquisition and launch under the lock, so that a
        // concurrent call on the same stream cannot replace the buffers
        // between the two.
        // (The no-allocation path shares one array per device: under the
        // lock, two threads' calls on one stream cannot interleave their
        // GEMM and sum kernels either.)
        std::lock_guard<std::recursive_mutex> lock(g_mu);
        if (c.scratch) {
            a.partials = (float *)c.scratch;
        } else {
            Workspace w;
            if ((st = workspace_for(dev, c.stream, p, &w)) != SGEMM_OK) return st;
            a.partials = w.partials;
        }
        e = launch_cfg(p.config, a, c.stream, c.tc);   // the skinny and row-dot kernels add their own splits
        if (e == hipSuccess && !any_layout(p.config)) e = launch_sk_fixup(a, p.bm, p.bn, c.stream);
    } else if (p.fixed) {
        e = launch_mfma_dl_fixed(p.fixed - 1, a, c.stream);
    } else {
        e = launch_cfg(p.config, a, c.stream, c.tc);
    }
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

Call plain(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C, int ldc,
           hipStream_t stream, int config, int sched) {
    return Call{M, N, K, 0, 0, A, B, C, lda, ldb, ldc, 0, 1.0f, 0.0f, stream, config, sched, 0};
}

Call blas(int ta, int tb, int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, hipStream_t stream, int config, int sched) {
    return Call{M, N, K, ta != 0, tb != 0, A, B, C, lda, ldb, ldc, 1, alpha, beta, stream, config, sched, 0};
}

}  // namespace
}  // namespace sgemm

SGEMM_API int sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                        float *C, int ldc, hipStream_t stream) {
    return sgemm::run(sgemm::plain(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_CFG_AUTO, SGEMM_SCHED_AUTO));
}

SGEMM_API int sgemm_f32_ex(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                           float *C, int ldc, hipStream_t stream, int config, int sched) {
    return sgemm::run(sgemm::plain(M, N, K, A, lda, B, ldb, C, ldc, stream, config, sched));
}

SGEMM_API int sgemm_f32_gemm(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                             int lda, const float *B, int ldb, float beta, float *C, int ldc,
                             hipStream_t stream) {
    if (trans_a < 0 || trans_a > 1 || trans_b < 0 || trans_b > 1) return SGEMM_ERR_CONFIG;
    return sgemm::run(sgemm::blas(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                                  SGEMM_CFG_AUTO, SGEMM_SCHED_AUTO));
}

SGEMM_API int sgemm_f32_gemm_ex(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                                int lda, const float *B, int ldb, float beta, float *C, int ldc,
                                hipStream_t stream, int config, int sched) {
    if (trans_a < 0 || trans_a > 1 || trans_b < 0 || trans_b > 1) return SGEMM_ERR_CONFIG;
    return sgemm::run(sgemm::blas(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                                  config, sched));
}

SGEMM_API int sgemm_f32_gemm_noalloc(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                                     int lda, const float *B, int ldb, float beta, float *C, int ldc,
                                     hipStream_t stream) {
    if (trans_a < 0 || trans_a > 1 || trans_b < 0 || trans_b > 1) return SGEMM_ERR_CONFIG;
    sgemm::Call c = sgemm::blas(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                                SGEMM_CFG_AUTO, SGEMM_SCHED_AUTO);
    int st = sgemm::check_args(c);
    if (st != SGEMM_OK || M == 0 || N == 0) return st;
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return sgemm::hip_fail(e);
    if ((st = sgemm::scratch_of(dev, &c.scratch)) != SGEMM_OK) return st;
    c.scratch_bytes = sgemm::kScratchBytes;
    return sgemm::run(c);
}

SGEMM_API void sgemm_f32_granule(int *gm, int *gn, int *gk) {
    if (gm) *gm = sgemm::kGranM;
    if (gn) *gn = sgemm::kGranN;
    if (gk) *gk = sgemm::kGranK;
}

SGEMM_API const char *sgemm_f32_status_string(int status) {
    switch (status) {
    case SGEMM_OK: return "ok";
    case SGEMM_ERR_SHAPE: return "shape: negative or not a multiple of the granule";
    case SGEMM_ERR_LD: return "leading dimension smaller than the row length";
    case SGEMM_ERR_ALIGN: return "pointer not aligned to a float (4 bytes)";
    case SGEMM_ERR_NULL: return "null pointer";
    case SGEMM_ERR_ALIAS: return "C overlaps A or B";
    case SGEMM_ERR_HIP: return "HIP runtime error";
    case SGEMM_ERR_POINTER: return "not device memory of the current device, or extent past its allocation";
    case SGEMM_ERR_CONFIG: return "unknown or inapplicable kernel configuration or schedule";
    case SGEMM_ERR_SCRATCH: return "the no-allocation call needs more scratch memory than its fixed maximum";
    default: return "unknown status";
    }
}

SGEMM_API int sgemm_f32_last_hip_error(void) { return sgemm::g_last_hip_error; }

static int plan_for(int ta, int tb, int M, int N, int K, int config, int sched, int num_cus,
                    const int *occupancy, int sk_wg_per_cu, sgemm_f32_plan_t *out) {
    if (!out) return SGEMM_ERR_NULL;
    if ((ta != 0 && ta != 1) || (tb != 0 && tb != 1)) return SGEMM_ERR_CONFIG;
    // Dense operands on 16-byte boundaries: the vector layout holds when
    // the stored row lengths of A and B, and N, are multiples of 4.  Else
    // the call itself may repack (see run_packed), and the plan is that of
    // the padded product.
    const int a_cols = ta ? M : K, b_cols = tb ? K : N;
    const bool aligned = a_cols % 4 == 0 && b_cols % 4 == 0 && N % 4 == 0;

    sgemm::Call c = sgemm::plain(M, N, K, nullptr, a_cols, nullptr, b_cols, nullptr, N, nullptr, config, sched);
    c.ta = ta;
    c.tb = tb;
    sgemm::PlanRequest req{M, N, K, config, sched, num_cus, occupancy, sk_wg_per_cu, aligned ? 1 : 0, ta, tb};
    const int tcfg = M > 0 && N > 0 ? sgemm::transposed_route(c) : SGEMM_CFG_AUTO;
    const bool swap = tcfg != SGEMM_CFG_AUTO;
    if (swap) {
        const sgemm::Call q = sgemm::transposed(c, tcfg);
        req = sgemm::PlanRequest{q.M, q.N, q.K, q.config, sched, num_cus, occupancy, sk_wg_per_cu,
                                 aligned ? 1 : 0, q.ta, q.tb};
    }
    out->transposed = swap ? 1 : 0;
    sgemm::Plan p;
    int st = sgemm::make_plan(req, &p);
    if (st != SGEMM_OK) return st;
    const bool repack = !aligned && config == SGEMM_CFG_AUTO && K > 0 && M > 0 && N > 0 &&
                        !sgemm::any_layout(p.config) && sgemm::worth_repacking(c);
    if (repack) {
        req.M = ta ? sgemm::up4(M) : M;
        req.N = sgemm::up4(N);
        req.K = sgemm::up4(K);
        req.aligned = 1;
        if ((st = sgemm::make_plan(req, &p)) != SGEMM_OK) return st;
    }
    out->repacked = repack ? 1 : 0;
    out->config = p.config;
    out->sched = p.sched;
    out->tile_m = p.bm;
    out->tile_n = p.bn;
    out->tile_k = p.bk;
    out->threads = p.threads;
    out->tiles_m = p.tiles_m;
    out->tiles_n = p.tiles_n;
    out->iters_per_tile = p.ipt;
    out->dp_tiles = p.dp_tiles;
    out->sk_tiles = p.sk_tiles;
    out->grid = p.grid;
    out->sk_grid = p.sk_grid;
    out->xcd_remap = p.xcd_remap;
    out->group_m = p.group_m;
    out->sk_iters = p.sk_iters;
    out->workspace_bytes = p.workspace_bytes;
    out->fixed_shape = p.fixed ? 1 : 0;
    const int occ = occupancy ? occupancy[p.config] : sgemm::kCfgs[p.config].default_occ;   // as make_plan reads it
    out->model_us = sgemm::plan_cost(p, req.M, req.N, num_cus > 0 ? num_cus : 1, occ);
    return SGEMM_OK;
}

SGEMM_API int sgemm_f32_plan(int M, int N, int K, int config, int sched, int num_cus,
                             const int *occupancy, int sk_wg_per_cu, sgemm_f32_plan_t *out) {
    return plan_for(0, 0, M, N, K, config, sched, num_cus, occupancy, sk_wg_per_cu, out);
}

SGEMM_API int sgemm_f32_gemm_plan(int trans_a, int trans_b, int M, int N, int K, int config, int sched,
                                  int num_cus, const int *occupancy, int sk_wg_per_cu, sgemm_f32_plan_t *out) {
    return plan_for(trans_a, trans_b, M, N, K, config, sched, num_cus, occupancy, sk_wg_per_cu, out);
}

SGEMM_API int sgemm_f32_release(void) {
    std::lock_guard<std::recursive_mutex> lock(sgemm::g_mu);
    int st = SGEMM_OK;
    for (auto &kv : sgemm::g_workspaces) {
        if (kv.second.partials && hipFree(kv.second.partials) != hipSuccess) st = SGEMM_ERR_HIP;
        if (kv.second.pack && hipFree(kv.second.pack) != hipSuccess) st = SGEMM_ERR_HIP;
    }
    sgemm::g_workspaces.clear();
    return st;
}
