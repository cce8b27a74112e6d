"""FP64 CPU oracle for FP32 GEMM, C = A @ B (AB only).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import this package.  It shares
no code with the GPU library and imports nothing from it.

The arithmetic lives in oracle_f64.c (a plain triple loop that forms each
product exactly in FP64 and adds in ascending k); this module only marshals
numpy arrays through ctypes.  The operation is the one defined on the page
"Beyond Kernel 7: Closing the Gap to cuBLAS on an H100 FP32 GEMM", section
"The operation: GEMM and the precision of the comparison":
C[m, n] = sum_k A[m, k] * B[k, n], computed for AB only.

Each call also returns S[m, n] = sum_k |A[m, k] * B[k, n]|, the scale of the
per-element error bound |C_gpu - C_ref| <= 1e-5 * S.

gemm_blas is the BLAS form the pages' kernels carry (alpha and beta in the
scaled stores of "Vectorized Memory Access: Pushing CUDA SGEMM to 29 TFLOPS
on H100" and "2D Block Tiling: Scaling Matrix Multiplication on NVIDIA
H100", sections 5), with either storage order of A and B:
C = alpha * op(A) op(B) + beta * C0, the product from the same triple loop.

Parity pins: see tests/test_oracle_pins.py (identity, all-ones, integer
exactness, rank-1 closed form, transpose invariance, exact rational brute
force, planted-mistake detection).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    f = lib.oracle_gemm_f64
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_long,
                  ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_long,
                  ctypes.c_int]
    g = lib.oracle_gemm_points_f64
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_long,
                  ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    d = lib.oracle_dot_f64
    d.restype = None
    d.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long,
                  ctypes.c_void_p, ctypes.c_void_p]
    _LIB = lib
    return lib


def default_threads() -> int:
    """Host cores this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _as_f32_2d(x, name):
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.strides[1] != 4 or x.strides[0] % 4 != 0:
        x = np.ascontiguousarray(x)
    return x


def gemm(A, B, threads=None):
    """Return (C_ref, S) as float64 arrays of shape (M, N)."""
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_f64(
        M, N, K, A.ctypes.data, A.strides[0] // 4, B.ctypes.data, B.strides[0] // 4,
        C.ctypes.data, N, S.ctypes.data, N, int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_gemm_f64 failed")
    return C, S


def gemm_blas(A, B, C0=None, alpha=1.0, beta=0.0, trans_a=False, trans_b=False, threads=None):
    """Return (C_ref, S) for C = alpha * op(A) op(B) + beta * C0, in FP64.

    op(A) = A^T when trans_a (A stored K x M), else A; likewise B.  C0 is
    read only when beta != 0 (BLAS convention).  S = |alpha| * sum_k
    |op(A)[m,k] op(B)[k,n]| + |beta| * |C0[m,n]| scales the error bound.
    alpha and beta are taken as the float32 values a GPU call receives."""
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    opA = np.ascontiguousarray(A.T) if trans_a else A
    opB = np.ascontiguousarray(B.T) if trans_b else B
    P, S = gemm(opA, opB, threads)
    a = float(np.float32(alpha))
    b = float(np.float32(beta))
    C = a * P
    S = abs(a) * S
    if b != 0.0:
        C0 = np.asarray(C0, dtype=np.float64)
        if C0.shape != C.shape:
            raise ValueError("C0 shape")
        C = C + b * C0
        S = S + abs(b) * np.abs(C0)
    return C, S


def gemm_points(A, B, rows, cols):
    """Return (C_ref, S) at positions (rows[i], cols[i]) only, float64 1-D."""
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D of equal length")
    c = np.empty(rows.shape[0], dtype=np.float64)
    s = np.empty(rows.shape[0], dtype=np.float64)
    rc = _load().oracle_gemm_points_f64(
        M, N, K, A.ctypes.data, A.strides[0] // 4, B.ctypes.data, B.strides[0] // 4,
        rows.shape[0], rows.ctypes.data, cols.ctypes.data, c.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_gemm_points_f64 failed (index out of range?)")
    return c, s


def dot(a_row, b_col):
    """One element: sum_k a_row[k] * b_col[k] in FP64, ascending k; returns (c, s)."""
    a = np.ascontiguousarray(a_row, dtype=np.float32).ravel()
    b = np.ascontiguousarray(b_col, dtype=np.float32).ravel()
    if a.shape != b.shape:
        raise ValueError("length mismatch")
    c = ctypes.c_double()
    s = ctypes.c_double()
    _load().oracle_dot_f64(a.shape[0], a.ctypes.data, b.ctypes.data, 1,
                           ctypes.byref(c), ctypes.byref(s))
    return c.value, s.value


def within_bound(C_gpu, C_ref, S, rel=1e-5):
    """Per-element acceptance: every element finite and |C_gpu - C_ref| <= rel*S.

    Returns (ok, worst) where worst = max |C_gpu - C_ref| / S over elements
    with S > 0 (elements with S == 0 must match exactly)."""
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    if not np.all(np.isfinite(C_gpu)):
        return False, float("inf")
    err = np.abs(C_gpu - C_ref)
    ok = bool(np.all(err <= rel * S))
    pos = S > 0
    worst = float(np.max(err[pos] / S[pos])) if np.any(pos) else 0.0
    if np.any(err[~pos] > 0):
        worst = float("inf")
    return ok, worst
