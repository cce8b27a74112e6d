"""Python binding of libsgemm_f32 (include/sgemm_f32.h): FP32 GEMM C = A @ B.

Argument marshalling only: every step of the product runs in the HIP
library.  If the library has not been built, importing succeeds but every
call raises (there is no fallback of any kind).  PyTorch is used only to
hold device memory and to name the current HIP stream.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; SGEMM_F32_LIBRARY may name another build of the same sources.
LIB_PATH = os.environ.get("SGEMM_F32_LIBRARY") or os.path.join(_HERE, "libsgemm_f32.so")

# Status codes (SGEMM_*).
OK = 0
ERR_SHAPE = 1
ERR_LD = 2
ERR_ALIGN = 3
ERR_NULL = 4
ERR_ALIAS = 5
ERR_HIP = 6
ERR_POINTER = 7
ERR_CONFIG = 8
ERR_SCRATCH = 9
# Scratch memory of gemm_noalloc per device (SGEMM_F32_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20

# Kernel configurations (SGEMM_CFG_*).
CFG_AUTO = 0
CFG_MFMA_256x256x16 = 1
CFG_MFMA_128x128x32 = 2
CFG_MFMA_256x256x32 = 3
CFG_MFMA_256x128x32 = 4
CFG_VALU_128x128x8 = 5
CFG_MFMA_256x256x32_W8 = 6
CFG_MFMA_128x128x32_W8 = 7
CFG_MFMA_64x64x32 = 8
CFG_MFMA_128x64x32 = 9
CFG_MFMA_64x64x64 = 10
CFG_MFMA_128x128x64 = 11
CFG_MFMA_64x64x128 = 12
CFG_DL_64x64x32 = 13
CFG_DL_64x64x64_K2 = 14
CFG_DL_128x128x32 = 15
CFG_DL_256x256x16 = 16
CFG_DL_64x64x32_K2 = 17
CFG_DL_128x128x32_K2 = 18
CFG_DL_64x64x64 = 19
CFG_DL_128x256x16 = 20
CFG_DL_256x128x16 = 21
CFG_GENERIC_64x64x16 = 22
CFG_SKINNY_16x256 = 23
CFG_ROWDOT_N8 = 24
CFG_VALU_256x128x8 = 25
NUM_CFGS = 26
CFG_NAMES = {
    CFG_AUTO: "auto",
    CFG_MFMA_256x256x16: "mfma_256x256x16",
    CFG_MFMA_128x128x32: "mfma_128x128x32",
    CFG_MFMA_256x256x32: "mfma_256x256x32",
    CFG_MFMA_256x128x32: "mfma_256x128x32",
    CFG_VALU_128x128x8: "valu_128x128x8",
    CFG_MFMA_256x256x32_W8: "mfma_256x256x32_w8",
    CFG_MFMA_128x128x32_W8: "mfma_128x128x32_w8",
    CFG_MFMA_64x64x32: "mfma_64x64x32",
    CFG_MFMA_128x64x32: "mfma_128x64x32",
    CFG_MFMA_64x64x64: "mfma_64x64x64",
    CFG_MFMA_128x128x64: "mfma_128x128x64",
    CFG_MFMA_64x64x128: "mfma_64x64x128",
    CFG_DL_64x64x32: "dl_64x64x32",
    CFG_DL_64x64x64_K2: "dl_64x64x64_k2",
    CFG_DL_128x128x32: "dl_128x128x32",
    CFG_DL_256x256x16: "dl_256x256x16",
    CFG_DL_64x64x32_K2: "dl_64x64x32_k2",
    CFG_DL_128x128x32_K2: "dl_128x128x32_k2",
    CFG_DL_64x64x64: "dl_64x64x64",
    CFG_DL_128x256x16: "dl_128x256x16",
    CFG_DL_256x128x16: "dl_256x128x16",
    CFG_GENERIC_64x64x16: "generic_64x64x16",
    CFG_SKINNY_16x256: "skinny_16x256",
    CFG_ROWDOT_N8: "rowdot_n8",
    CFG_VALU_256x128x8: "valu_256x128x8",
}
# (tile_m, tile_n, tile_k) of each configuration.
CFG_TILES = {
    CFG_MFMA_256x256x16: (256, 256, 16), CFG_MFMA_128x128x32: (128, 128, 32),
    CFG_MFMA_256x256x32: (256, 256, 32), CFG_MFMA_256x128x32: (256, 128, 32),
    CFG_VALU_128x128x8: (128, 128, 8), CFG_MFMA_256x256x32_W8: (256, 256, 32),
    CFG_MFMA_128x128x32_W8: (128, 128, 32), CFG_MFMA_64x64x32: (64, 64, 32),
    CFG_MFMA_128x64x32: (128, 64, 32), CFG_MFMA_64x64x64: (64, 64, 64),
    CFG_MFMA_128x128x64: (128, 128, 64), CFG_MFMA_64x64x128: (64, 64, 128),
    CFG_DL_64x64x32: (64, 64, 32), CFG_DL_64x64x64_K2: (64, 64, 64),
    CFG_DL_128x128x32: (128, 128, 32), CFG_DL_256x256x16: (256, 256, 16),
    CFG_DL_64x64x32_K2: (64, 64, 32), CFG_DL_128x128x32_K2: (128, 128, 32),
    CFG_DL_64x64x64: (64, 64, 64), CFG_DL_128x256x16: (128, 256, 16),
    CFG_DL_256x128x16: (256, 128, 16), CFG_GENERIC_64x64x16: (64, 64, 16),
    CFG_VALU_256x128x8: (256, 128, 8),
}

# Schedules (SGEMM_SCHED_*).
SCHED_AUTO = 0
SCHED_DP = 1
SCHED_STREAMK = 2
SCHED_FIXED = 3
SCHED_NAMES = {SCHED_AUTO: "auto", SCHED_DP: "dp", SCHED_STREAMK: "streamk", SCHED_FIXED: "fixed"}


class SgemmError(RuntimeError):
    def __init__(self, status, where="sgemm_f32"):
        self.status = status
        hip = last_hip_error() if status == ERR_HIP else 0
        msg = f"{where}: status {status} ({status_string(status)})"
        if hip:
            msg += f", hipError {hip}"
        super().__init__(msg)


class _Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "config", "sched", "tile_m", "tile_n", "tile_k", "threads", "tiles_m", "tiles_n",
        "iters_per_tile", "dp_tiles", "sk_tiles", "grid", "sk_grid", "xcd_remap", "group_m")] + [
        ("sk_iters", ctypes.c_longlong), ("workspace_bytes", ctypes.c_longlong), ("repacked", ctypes.c_int),
        ("transposed", ctypes.c_int), ("fixed_shape", ctypes.c_int), ("model_us", ctypes.c_double)]


_lib = None


def library():
    """The loaded ctypes library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python fp32_sgemm_f32_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i, p, vp = ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    lib.sgemm_f32.restype = i
    lib.sgemm_f32.argtypes = [i, i, i, p, i, p, i, p, i, vp]
    lib.sgemm_f32_ex.restype = i
    lib.sgemm_f32_ex.argtypes = [i, i, i, p, i, p, i, p, i, vp, i, i]
    f = ctypes.c_float
    lib.sgemm_f32_gemm.restype = i
    lib.sgemm_f32_gemm.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, vp]
    lib.sgemm_f32_gemm_ex.restype = i
    lib.sgemm_f32_gemm_ex.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, vp, i, i]
    lib.sgemm_f32_gemm_noalloc.restype = i
    lib.sgemm_f32_gemm_noalloc.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, vp]
    lib.sgemm_f32_granule.restype = None
    lib.sgemm_f32_granule.argtypes = [ctypes.POINTER(i)] * 3
    lib.sgemm_f32_status_string.restype = ctypes.c_char_p
    lib.sgemm_f32_status_string.argtypes = [i]
    lib.sgemm_f32_last_hip_error.restype = i
    lib.sgemm_f32_last_hip_error.argtypes = []
    lib.sgemm_f32_plan.restype = i
    lib.sgemm_f32_plan.argtypes = [i, i, i, i, i, i, ctypes.POINTER(i), i, ctypes.POINTER(_Plan)]
    lib.sgemm_f32_gemm_plan.restype = i
    lib.sgemm_f32_gemm_plan.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(i), i, ctypes.POINTER(_Plan)]
    lib.sgemm_f32_release.restype = i
    lib.sgemm_f32_release.argtypes = []
    _lib = lib
    return lib


def granule():
    """(gm, gn, gk): M, N, K must be multiples of these (1, 1, 1: any shape)."""
    g = [ctypes.c_int() for _ in range(3)]
    library().sgemm_f32_granule(*[ctypes.byref(x) for x in g])
    return tuple(x.value for x in g)


def status_string(status: int) -> str:
    return library().sgemm_f32_status_string(int(status)).decode()


def last_hip_error() -> int:
    return library().sgemm_f32_last_hip_error()


def release() -> None:
    st = library().sgemm_f32_release()
    if st != OK:
        raise SgemmError(st, "sgemm_f32_release")


def plan(M, N, K, config=CFG_AUTO, sched=SCHED_AUTO, num_cus=256, occupancy=None,
         sk_wg_per_cu=0, trans_a=0, trans_b=0) -> dict:
    """The launch plan for a shape (host computation only, no GPU needed);
    trans_a / trans_b: the storage orders of the BLAS form (gemm)."""
    occ = None
    if occupancy is not None:
        if len(occupancy) != NUM_CFGS:
            raise ValueError(f"occupancy needs {NUM_CFGS} entries")
        occ = (ctypes.c_int * NUM_CFGS)(*occupancy)
    out = _Plan()
    st = library().sgemm_f32_gemm_plan(trans_a, trans_b, M, N, K, config, sched, num_cus, occ, sk_wg_per_cu,
                                       ctypes.byref(out))
    if st != OK:
        raise SgemmError(st, "sgemm_f32_gemm_plan")
    return {name: getattr(out, name) for name, _ in _Plan._fields_}


def sgemm_raw(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, stream=0,
              config=CFG_AUTO, sched=SCHED_AUTO) -> int:
    """Direct call with integer device addresses; returns the status code."""
    lib = library()
    if config == CFG_AUTO and sched == SCHED_AUTO:
        return lib.sgemm_f32(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, stream)
    return lib.sgemm_f32_ex(M, N, K, A_ptr, lda, B_ptr, ldb, C_ptr, ldc, stream, config, sched)


def gemm_raw(trans_a, trans_b, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, stream=0,
             config=CFG_AUTO, sched=SCHED_AUTO) -> int:
    """C = alpha op(A) op(B) + beta C with integer device addresses; returns the status."""
    lib = library()
    if config == CFG_AUTO and sched == SCHED_AUTO:
        return lib.sgemm_f32_gemm(trans_a, trans_b, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc,
                                  stream)
    return lib.sgemm_f32_gemm_ex(trans_a, trans_b, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc,
                                 stream, config, sched)


def gemm_noalloc_raw(trans_a, trans_b, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta, C_ptr, ldc, stream=0) -> int:
    """sgemm_f32_gemm_noalloc with integer device addresses (no device memory
    allocated: scratch from the library's fixed per-device array); returns
    the status."""
    return library().sgemm_f32_gemm_noalloc(trans_a, trans_b, M, N, K, alpha, A_ptr, lda, B_ptr, ldb, beta,
                                            C_ptr, ldc, stream)


def gemm(A, B, C=None, alpha=1.0, beta=0.0, trans_a=False, trans_b=False, config=CFG_AUTO,
         sched=SCHED_AUTO, stream=None):
    """C = alpha * op(A) @ op(B) + beta * C for float32 HIP tensors.

    A is the stored matrix: (M, K), or (K, M) with trans_a (op(A) = A^T);
    B: (K, N), or (N, K) with trans_b.  Row-major (unit column stride; padded
    rows allowed); a column-major view (X.t() of a row-major X) is taken as
    the other storage order, without a copy.  C (M, N) must be row-major and
    is allocated if None (then beta must be 0).  Returns C.
    """
    import torch

    for t, n in ((A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{n} must be a float32 tensor on a HIP device")
    M, K = (A.shape[1], A.shape[0]) if trans_a else tuple(A.shape)
    K2, N = (B.shape[1], B.shape[0]) if trans_b else tuple(B.shape)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif C.dtype != torch.float32 or tuple(C.shape) != (M, N) or C.device != A.device:
        raise ValueError("C must be float32 (M, N) on A's device")
    As, ta, lda = _stored(A, "A", trans_a)
    Bs, tb, ldb = _stored(B, "B", trans_b)
    ldc = _row_major_ld(C, "C")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        st = gemm_raw(ta, tb, M, N, K, float(alpha), As.data_ptr(), lda, Bs.data_ptr(), ldb, float(beta),
                      C.data_ptr(), ldc, stream.cuda_stream, config, sched)
    if st != OK:
        raise SgemmError(st, "sgemm_f32_gemm")
    return C


def _stored(t, name, trans):
    """(row-major tensor, transpose flag, leading dimension) for operand t as
    given with flag `trans`: a column-major view (t.t() of a row-major
    matrix) is the same memory stored the other way, so the flag flips and
    nothing is copied."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1 and t.stride(0) == 1:
        s = t.t()
        return s, int(not trans), _row_major_ld(s, name)
    return t, int(bool(trans)), _row_major_ld(t, name)


def _row_major_ld(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.numel() == 0:          # nothing is read or written through it
        return (t.shape[1] + 3) // 4 * 4
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must be row-major (unit column stride)")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def matmul(A, B, out=None, config=CFG_AUTO, sched=SCHED_AUTO, stream=None):
    """C = A @ B for float32 CUDA (HIP) tensors, on the current (or given) stream.

    A: (M, K), B: (K, N), each row-major (unit column stride; padded rows
    allowed) or column-major (a transposed view such as X.t(), run as the
    other storage order without a copy).  `out` must be row-major.  Returns
    `out` (allocated if None).  Raises SgemmError on a library error.
    """
    import torch

    for t, n in ((A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{n} must be a float32 tensor on a HIP device")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, N) or out.device != A.device:
        raise ValueError("out must be float32 (M, N) on A's device")
    As, ta, lda = _stored(A, "A", False)
    Bs, tb, ldb = _stored(B, "B", False)
    ldc = _row_major_ld(out, "out")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    with torch.cuda.device(A.device):
        if ta or tb:
            st = gemm_raw(ta, tb, M, N, K, 1.0, As.data_ptr(), lda, Bs.data_ptr(), ldb, 0.0, out.data_ptr(), ldc,
                          stream.cuda_stream, config, sched)
        else:
            st = sgemm_raw(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc,
                           stream.cuda_stream, config, sched)
    if st != OK:
        raise SgemmError(st)
    return out
