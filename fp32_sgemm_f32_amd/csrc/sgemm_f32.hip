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
    int *counters = nullptr;
    int64_t ncounters = 0;
    float *partials = nullptr;
    int64_t partial_bytes = 0;
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_devices;
std::map<std::pair<int, hipStream_t>, Workspace> g_workspaces;

hipError_t launch_cfg(int cfg, const KernelArgs &a, hipStream_t s) {
    switch (kCfgs[cfg].kind) {
    case kKindMfma: return launch_mfma(cfg, a, s);
    case kKindMfmaDl: return launch_mfma_dl(cfg, a, s);
    case kKindGeneric: return launch_generic(cfg, a, s);
    default: return launch_valu(cfg, a, s);
    }
}

hipError_t occupancy_of(int cfg, int *n) {
    switch (kCfgs[cfg].kind) {
    case kKindMfma: return occupancy_mfma(cfg, n);
    case kKindMfmaDl: return occupancy_mfma_dl(cfg, n);
    case kKindGeneric: return occupancy_generic(cfg, n);
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
    std::lock_guard<std::mutex> lock(g_mu);
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

// Host-only checks (no HIP call).  Order: shape, ld, null, alignment, alias.
int check_args(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
               const float *C, int ldc) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_SHAPE;
    if (M == 0 || N == 0) return SGEMM_OK;
    // A and B (and their leading dimensions) are not read when K == 0.
    if (ldc < N || (K > 0 && (lda < K || ldb < N))) return SGEMM_ERR_LD;
    if (!C || (K > 0 && (!A || !B))) return SGEMM_ERR_NULL;
    if (((uintptr_t)C & 3) || (K > 0 && (((uintptr_t)A & 3) || ((uintptr_t)B & 3)))) return SGEMM_ERR_ALIGN;
    const int64_t nc = extent_bytes(M, N, ldc);
    if (K > 0 && (overlap(C, nc, A, extent_bytes(M, K, lda)) ||
                  overlap(C, nc, B, extent_bytes(K, N, ldb))))
        return SGEMM_ERR_ALIAS;
    return SGEMM_OK;
}

// The layout the vector (16-byte) kernels need; anything else runs on the
// general kernel.
bool vector_layout(int N, int K, const float *A, int lda, const float *B, int ldb, const float *C, int ldc) {
    return (N & 3) == 0 && (K & 3) == 0 && (lda & 3) == 0 && (ldb & 3) == 0 && (ldc & 3) == 0 &&
           ((uintptr_t)A & 15) == 0 && ((uintptr_t)B & 15) == 0 && ((uintptr_t)C & 15) == 0;
}

// Stream-K workspace of (dev, stream), grown to hold `plan`.  Counters are
// zeroed when allocated and left at zero by every call.  Caller holds g_mu.
int workspace_for(int dev, hipStream_t s, const Plan &p, Workspace *out) {
    Workspace &w = g_workspaces[{dev, s}];
    const int64_t need_part = (int64_t)p.sk_grid * 2 * p.bm * p.bn * 4;
    if (w.ncounters < p.sk_tiles || w.partial_bytes < need_part) {
        hipError_t e = hipStreamSynchronize(s);   // old buffers may still be in use
        if (e != hipSuccess) return hip_fail(e);
        if (w.ncounters < p.sk_tiles) {
            if (w.counters) (void)hipFree(w.counters);
            w.counters = nullptr;
            w.ncounters = 0;
            int64_t n = p.sk_tiles < 4096 ? 4096 : p.sk_tiles;
            e = hipMalloc((void **)&w.counters, (size_t)n * 4);
            if (e != hipSuccess) return hip_fail(e);
            e = hipMemsetAsync(w.counters, 0, (size_t)n * 4, s);
            if (e != hipSuccess) return hip_fail(e);
            w.ncounters = n;
        }
        if (w.partial_bytes < need_part) {
            if (w.partials) (void)hipFree(w.partials);
            w.partials = nullptr;
            w.partial_bytes = 0;
            e = hipMalloc((void **)&w.partials, (size_t)need_part);
            if (e != hipSuccess) return hip_fail(e);
            w.partial_bytes = need_part;
        }
    }
    *out = w;
    return SGEMM_OK;
}

int run(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float *C,
        int ldc, hipStream_t stream, int config, int sched) {
    int st = check_args(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_OK) return st;
    if (config < 0 || config >= SGEMM_NUM_CFGS) return SGEMM_ERR_CONFIG;
    if (sched < SGEMM_SCHED_AUTO || sched > SGEMM_SCHED_STREAMK) return SGEMM_ERR_CONFIG;
    if (M == 0 || N == 0) return SGEMM_OK;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if ((st = check_device_range(C, extent_bytes(M, N, ldc), dev)) != SGEMM_OK) return st;
    if (K > 0) {
        if ((st = check_device_range(A, extent_bytes(M, K, lda), dev)) != SGEMM_OK) return st;
        if ((st = check_device_range(B, extent_bytes(K, N, ldb), dev)) != SGEMM_OK) return st;
    }

    DeviceInfo info;
    if ((st = device_info(dev, &info)) != SGEMM_OK) return st;
    PlanRequest req{M, N, K, config, sched, info.num_cus, info.occupancy,
                    env_int("SGEMM_F32_SK_WG_PER_CU", 0),
                    vector_layout(N, K, A, lda, B, ldb, C, ldc) ? 1 : 0};
    Plan p;
    if ((st = make_plan(req, &p)) != SGEMM_OK) return st;
    if (K > 0 && !dl_offsets_fit(p.config, p.edge != 0, lda, ldb)) {
        // Leading dimensions too large for the 32-bit source offsets of the
        // direct-to-LDS kernels: an automatic choice falls back to the
        // register-staged kernel of the same tile (the general one when the
        // tile does not divide the shape); a forced one is refused.
        if (config != SGEMM_CFG_AUTO) return SGEMM_ERR_CONFIG;
        req.config = p.edge ? SGEMM_CFG_GENERIC_64x64x16 : staged_equivalent(p.config);
        if ((st = make_plan(req, &p)) != SGEMM_OK) return st;
    }

    if (K == 0) {
        e = launch_fill_zero(C, M, N, ldc, stream);
        return e == hipSuccess ? SGEMM_OK : hip_fail(e);
    }

    KernelArgs a{};
    a.A = A; a.B = B; a.C = C;
    a.lda = lda; a.ldb = ldb; a.ldc = ldc;
    a.M = M; a.N = N; a.K = K;
    a.edge = p.edge;
    a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n; a.ipt = p.ipt;
    a.dp_tiles = p.dp_tiles; a.sk_tiles = p.sk_tiles;
    a.grid = p.grid; a.sk_grid = p.sk_grid;
    a.xcd_remap = env_int("SGEMM_F32_XCD_REMAP", 1) ? p.xcd_remap : 0;
    a.group_m = p.group_m;
    a.sk_iters = p.sk_iters;

    if (p.sk_tiles > 0) {
        // Workspace acquisition and launch under the lock, so that a
        // concurrent call on the same stream cannot replace the buffers
        // between the two.
        std::lock_guard<std::mutex> lock(g_mu);
        Workspace w;
        if ((st = workspace_for(dev, stream, p, &w)) != SGEMM_OK) return st;
        a.counters = w.counters;
        a.partials = w.partials;
        e = launch_cfg(p.config, a, stream);
    } else {
        e = launch_cfg(p.config, a, stream);
    }
    return e == hipSuccess ? SGEMM_OK : hip_fail(e);
}

}  // namespace
}  // namespace sgemm

SGEMM_API int sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                        float *C, int ldc, hipStream_t stream) {
    return sgemm::run(M, N, K, A, lda, B, ldb, C, ldc, stream, SGEMM_CFG_AUTO, SGEMM_SCHED_AUTO);
}

SGEMM_API int sgemm_f32_ex(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                           float *C, int ldc, hipStream_t stream, int config, int sched) {
    return sgemm::run(M, N, K, A, lda, B, ldb, C, ldc, stream, config, sched);
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
    default: return "unknown status";
    }
}

SGEMM_API int sgemm_f32_last_hip_error(void) { return sgemm::g_last_hip_error; }

SGEMM_API int sgemm_f32_plan(int M, int N, int K, int config, int sched, int num_cus,
                             const int *occupancy, int sk_wg_per_cu, sgemm_f32_plan_t *out) {
    if (!out) return SGEMM_ERR_NULL;
    // Planned for dense operands (lda = K, ldb = ldc = N) on 16-byte boundaries.
    sgemm::PlanRequest req{M, N, K, config, sched, num_cus, occupancy, sk_wg_per_cu,
                           (N % 4 == 0 && K % 4 == 0) ? 1 : 0};
    sgemm::Plan p;
    int st = sgemm::make_plan(req, &p);
    if (st != SGEMM_OK) return st;
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
    return SGEMM_OK;
}

SGEMM_API int sgemm_f32_release(void) {
    std::lock_guard<std::mutex> lock(sgemm::g_mu);
    int st = SGEMM_OK;
    for (auto &kv : sgemm::g_workspaces) {
        if (kv.second.counters && hipFree(kv.second.counters) != hipSuccess) st = SGEMM_ERR_HIP;
        if (kv.second.partials && hipFree(kv.second.partials) != hipSuccess) st = SGEMM_ERR_HIP;
    }
    sgemm::g_workspaces.clear();
    return st;
}
