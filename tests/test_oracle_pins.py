"""Pins of the FP64 CPU oracle against facts that do not come from the oracle.

The operation is the one defined on "Beyond Kernel 7: Closing the Gap to
cuBLAS on an H100 FP32 GEMM", section "The operation: GEMM and the precision
of the comparison": C[m, n] = sum_k A[m, k] * B[k, n], AB only.  The pages
print no output values for a worked example, so every pin below is a closed
form, an exact integer computation, an exact rational computation, or an
invariant of the definition.  Each pin is written as a check function taking
any candidate implementation; the last test plants plausible mistakes in a
copy of the oracle (on the CPU) and shows that every one of them fails at
least one pin.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import workloads

U53 = 2.0 ** -53  # unit roundoff of FP64


def _fp64_sum_bound(K, S):
    """Recursive-summation bound for K exact terms added in FP64: gamma_{K-1}*S."""
    n = max(K - 1, 0)
    return (n * U53 / (1.0 - n * U53)) * S


# ----------------------------------------------------------------------------
# Pin checks.  Each takes gemm_fn(A, B) -> (C, S) and returns True if it holds.
# ----------------------------------------------------------------------------

def pin_identity(gemm_fn):
    """B = I (K = N): each C[m, n] has exactly one nonzero term, A[m, n] * 1,
    so C must equal A exactly; likewise I @ B = B."""
    A, _ = workloads.generate(13, 9, 9, "uniform", 11)
    C, S = gemm_fn(A, np.eye(9, dtype=np.float32))
    ok = np.array_equal(C, A.astype(np.float64)) and np.array_equal(S, np.abs(A).astype(np.float64))
    _, B = workloads.generate(6, 11, 6, "normal", 12)
    C2, _ = gemm_fn(np.eye(6, dtype=np.float32), B)
    return ok and np.array_equal(C2, B.astype(np.float64))


def pin_all_ones(gemm_fn):
    """A = all ones: C[m, n] is the column sum of B, which math.fsum computes
    correctly rounded; the FP64 ascending sum must lie within the recursive
    summation bound of it.  With integer B the column sum is exact."""
    M, K, N = 3, 37, 10
    _, B = workloads.generate(M, N, K, "normal", 21)
    C, _ = gemm_fn(np.ones((M, K), dtype=np.float32), B)
    ok = True
    for n in range(N):
        col = [float(v) for v in B[:, n]]
        ref = math.fsum(col)
        bound = _fp64_sum_bound(K, math.fsum(abs(v) for v in col))
        ok &= all(abs(C[m, n] - ref) <= bound for m in range(M))
    _, Bi = workloads.generate(M, N, K, "int4", 22)
    Ci, _ = gemm_fn(np.ones((M, K), dtype=np.float32), Bi)
    ok &= np.array_equal(Ci, np.tile(Bi.astype(np.int64).sum(axis=0), (M, 1)).astype(np.float64))
    return bool(ok)


def pin_integer_exact(gemm_fn):
    """Entries in {-4..4}: every product and partial sum is an integer far
    below 2^53, so C must equal numpy's int64 matrix product exactly, and S
    must equal |A| @ |B| in int64 exactly."""
    A, B = workloads.generate(23, 17, 301, "int4", 31)
    C, S = gemm_fn(A, B)
    Ai, Bi = A.astype(np.int64), B.astype(np.int64)
    return np.array_equal(C, (Ai @ Bi).astype(np.float64)) and \
        np.array_equal(S, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def pin_rank1(gemm_fn):
    """A[m, k] = u[m] and B[k, n] = v[n]: every term equals u[m] v[n], so
    C = K u[m] v[n] (closed form) and S = K |u[m] v[n]|."""
    M, N, K = 5, 4, 33
    u = np.array([1, -2, 3, 0, -4], dtype=np.float32)
    v = np.array([2, -1, 4, -3], dtype=np.float32)
    A = np.repeat(u[:, None], K, axis=1)
    B = np.repeat(v[None, :], K, axis=0)
    C, S = gemm_fn(A, B)
    ref = K * np.outer(u.astype(np.float64), v.astype(np.float64))
    return np.array_equal(C, ref) and np.array_equal(S, np.abs(ref))


def pin_transpose(gemm_fn):
    """(A B)^T = B^T A^T with the same terms in the same k order, and each
    product exact in FP64, so the two must agree bit for bit."""
    A, B = workloads.generate(7, 5, 19, "uniform", 41)
    C, S = gemm_fn(A, B)
    Ct, St = gemm_fn(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    return np.array_equal(C, Ct.T) and np.array_equal(S, St.T)


def _exact(A, B):
    """Exact rational C and S by brute force (fractions.Fraction)."""
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(A[m, k])) for k in range(K)] for m in range(M)]
    Bf = [[Fraction(float(B[k, n])) for n in range(N)] for k in range(K)]
    C = [[sum((Af[m][k] * Bf[k][n] for k in range(K)), Fraction(0)) for n in range(N)]
         for m in range(M)]
    S = [[sum((abs(Af[m][k] * Bf[k][n]) for k in range(K)), Fraction(0)) for n in range(N)]
         for m in range(M)]
    return C, S


def pin_bruteforce(gemm_fn):
    """Tiny shapes, random FP32: the exact rational result by brute force must
    lie within the FP64 recursive-summation bound of the oracle's result,
    both for C and for S."""
    ok = True
    for i, (M, N, K) in enumerate([(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 7),
                                   (5, 7, 8), (2, 8, 16), (1, 3, 33)]):
        A, B = workloads.generate(M, N, K, "normal", 100 + i)
        C, S = gemm_fn(A, B)
        Ce, Se = _exact(A, B)
        for m in range(M):
            for n in range(N):
                bound = _fp64_sum_bound(K, float(Se[m][n]))
                ok &= abs(Fraction(float(C[m, n])) - Ce[m][n]) <= Fraction(bound)
                ok &= abs(Fraction(float(S[m, n])) - Se[m][n]) <= Fraction(bound)
    return bool(ok)


def pin_empty_k(gemm_fn):
    """K = 0: the empty sum, C = 0 and S = 0."""
    C, S = gemm_fn(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32))
    return C.shape == (3, 4) and not np.any(C) and not np.any(S)


PINS = [pin_identity, pin_all_ones, pin_integer_exact, pin_rank1,
        pin_transpose, pin_bruteforce, pin_empty_k]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_satisfies_pin(pin):
    assert pin(oracle.gemm)


# ----------------------------------------------------------------------------
# Further properties of the oracle's own interface.
# ----------------------------------------------------------------------------

def test_thread_count_independent():
    A, B = workloads.generate(67, 45, 129, "normal", 5)
    C1, S1 = oracle.gemm(A, B, threads=1)
    C7, S7 = oracle.gemm(A, B, threads=7)
    assert np.array_equal(C1, C7) and np.array_equal(S1, S7)


def test_points_match_full_product():
    A, B = workloads.generate(40, 50, 77, "uniform", 6)
    C, S = oracle.gemm(A, B)
    rng = np.random.default_rng(0)
    r = rng.integers(0, 40, 200)
    c = rng.integers(0, 50, 200)
    cp, sp = oracle.gemm_points(A, B, r, c)
    assert np.array_equal(cp, C[r, c]) and np.array_equal(sp, S[r, c])


def test_dot_matches_full_product():
    A, B = workloads.generate(3, 4, 64, "normal", 7)
    C, S = oracle.gemm(A, B)
    c, s = oracle.dot(A[2], B[:, 1])
    assert c == C[2, 1] and s == S[2, 1]


def test_strided_views():
    """Leading dimensions larger than the row length give the same result."""
    A, B = workloads.generate(8, 12, 20, "uniform", 8)
    Apad = np.zeros((8, 27), np.float32)
    Apad[:, :20] = A
    Bpad = np.zeros((20, 16), np.float32)
    Bpad[:, :12] = B
    C, S = oracle.gemm(A, B)
    Cv, Sv = oracle.gemm(Apad[:, :20], Bpad[:, :12])
    assert np.array_equal(C, Cv) and np.array_equal(S, Sv)


def test_points_reject_out_of_range():
    A, B = workloads.generate(4, 4, 4, "uniform", 9)
    with pytest.raises(RuntimeError):
        oracle.gemm_points(A, B, [4], [0])


def test_within_bound_helper():
    C_ref = np.array([[1.0, 0.0]])
    S = np.array([[2.0, 0.0]])
    assert oracle.within_bound(np.array([[1.0 + 1e-5, 0.0]]), C_ref, S)[0]
    assert not oracle.within_bound(np.array([[1.0 + 3e-5, 0.0]]), C_ref, S)[0]
    assert not oracle.within_bound(np.array([[1.0, 1e-30]]), C_ref, S)[0]
    assert not oracle.within_bound(np.array([[np.nan, 0.0]]), C_ref, S)[0]


# ----------------------------------------------------------------------------
# Planted mistakes: copies of the oracle's loop with one plausible error each.
# Every one must be caught by at least one pin.
# ----------------------------------------------------------------------------

def _loop_oracle(A, B, mistake=None):
    A = np.asarray(A, np.float32)
    B = np.asarray(B, np.float32)
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N))
    S = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            c = np.float32(0) if mistake == "fp32_accumulate" else 0.0
            s = 0.0
            ks = range(K - 1) if mistake == "drop_last_term" else range(K)
            for k in ks:
                if mistake == "transposed_b":
                    b = float(B[n % K, k % N])
                elif mistake == "shifted_k":
                    b = float(B[min(k + 1, K - 1), n])
                else:
                    b = float(B[k, n])
                a = float(A[m, k])
                if mistake == "fp32_accumulate":
                    p = np.float32(np.float32(a) * np.float32(b))
                    c = np.float32(c + p)
                    s += abs(float(p))
                    continue
                p = a * b
                if mistake == "sign_flip" and k == K // 2:
                    p = -p
                c += p
                s += p if mistake == "signed_s" else abs(p)
            C[m, n] = float(c) + (1.0 if mistake == "init_one" else 0.0)
            S[m, n] = s
    return C, S


MISTAKES = ["drop_last_term", "transposed_b", "shifted_k", "sign_flip",
            "fp32_accumulate", "signed_s", "init_one"]


def test_loop_copy_without_mistake_passes_pins():
    fn = lambda A, B: _loop_oracle(A, B)  # noqa: E731
    assert all(p(fn) for p in PINS)


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_is_caught(mistake):
    fn = lambda A, B: _loop_oracle(A, B, mistake)  # noqa: E731
    failed = [p.__name__ for p in PINS if not p(fn)]
    assert failed, f"planted mistake {mistake!r} passed every pin"


# ----------------------------------------------------------------------------
# The BLAS form, C = alpha op(A) op(B) + beta C0 (oracle.gemm_blas).  Pins
# take blas_fn(A, B, C0, alpha, beta, trans_a, trans_b) -> (C, S).
# ----------------------------------------------------------------------------

def _stored(X, trans):
    """The array to pass for op(...) = X: X itself, or X^T stored."""
    return np.ascontiguousarray(X.T) if trans else X


def pin_blas_integer_exact(blas_fn):
    """Integer entries, alpha = 3, beta = -2, integer C0, every storage order:
    C = 3 (A @ B) - 2 C0 exactly (numpy int64), S = 3 |A| @ |B| + 2 |C0|."""
    A, B = workloads.generate(9, 11, 45, "int4", 51)
    C0 = workloads.generate(9, 11, 1, "int4", 52)[0][:, :1] * np.ones((1, 11), np.float32)
    Ai, Bi, C0i = A.astype(np.int64), B.astype(np.int64), C0.astype(np.int64)
    ref = 3 * (Ai @ Bi) - 2 * C0i
    sref = 3 * (np.abs(Ai) @ np.abs(Bi)) + 2 * np.abs(C0i)
    ok = True
    for ta in (False, True):
        for tb in (False, True):
            C, S = blas_fn(_stored(A, ta), _stored(B, tb), C0, 3.0, -2.0, ta, tb)
            ok &= np.array_equal(C, ref.astype(np.float64)) and np.array_equal(S, sref.astype(np.float64))
    return bool(ok)


def pin_blas_beta_zero_leaves_c0_unread(blas_fn):
    """beta = 0: C0 is not read, so NaNs in it do not reach C = alpha A B."""
    A, B = workloads.generate(6, 5, 13, "int4", 53)
    C0 = np.full((6, 5), np.nan, np.float32)
    C, _ = blas_fn(A, B, C0, 2.0, 0.0, False, False)
    return np.array_equal(C, 2.0 * (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))


def pin_blas_alpha_zero(blas_fn):
    """alpha = 0: C = beta C0 exactly (here beta = 0.5, exact in binary)."""
    A, B = workloads.generate(4, 7, 9, "normal", 54)
    C0 = workloads.generate(4, 7, 1, "normal", 55)[0][:, :1] * np.ones((1, 7), np.float32)
    C, _ = blas_fn(A, B, C0, 0.0, 0.5, False, False)
    return np.array_equal(C, 0.5 * C0.astype(np.float64))


def pin_blas_rank1_transposed(blas_fn):
    """op(A)[m, k] = u[m] stored as A^T (K x M), op(B)[k, n] = v[n] stored as
    B^T (N x K): C = alpha K u[m] v[n] (closed form)."""
    M, N, K = 4, 3, 21
    u = np.array([1, -3, 2, 5], dtype=np.float32)
    v = np.array([-2, 1, 3], dtype=np.float32)
    A_stored = np.repeat(u[None, :], K, axis=0)     # K x M: row k holds u
    B_stored = np.repeat(v[:, None], K, axis=1)     # N x K: row n holds v[n]
    C, _ = blas_fn(A_stored, B_stored, None, 2.0, 0.0, True, True)
    return np.array_equal(C, 2.0 * K * np.outer(u.astype(np.float64), v.astype(np.float64)))


BLAS_PINS = [pin_blas_integer_exact, pin_blas_beta_zero_leaves_c0_unread, pin_blas_alpha_zero,
             pin_blas_rank1_transposed]


def _blas_oracle(A, B, C0, alpha, beta, ta, tb):
    return oracle.gemm_blas(A, B, C0, alpha, beta, ta, tb)


@pytest.mark.parametrize("pin", BLAS_PINS, ids=[p.__name__ for p in BLAS_PINS])
def test_oracle_blas_form_satisfies_pin(pin):
    assert pin(_blas_oracle)


def _blas_with_mistake(mistake):
    """oracle.gemm_blas with one plausible bookkeeping error planted."""
    def fn(A, B, C0, alpha, beta, ta, tb):
        if mistake == "ignore_trans_a":
            ta = False
            A = np.ascontiguousarray(A.T) if A.shape[1] != B.shape[0] and not tb else A
        if mistake == "ignore_trans_b":
            tb = False
        if mistake == "swap_alpha_beta":
            alpha, beta = beta, alpha
        if mistake == "read_c0_always":
            C, S = oracle.gemm_blas(A, B, None, alpha, 0.0, ta, tb)
            return C + float(np.float32(beta)) * np.asarray(C0, np.float64), S
        if mistake == "beta_unscaled" and beta != 0.0:
            C, S = oracle.gemm_blas(A, B, C0, alpha, beta, ta, tb)
            return C - float(np.float32(beta)) * np.asarray(C0, np.float64) + np.asarray(C0, np.float64), S
        try:
            return oracle.gemm_blas(A, B, C0, alpha, beta, ta, tb)
        except ValueError:
            return np.full((1, 1), np.nan), np.full((1, 1), np.nan)
    return fn


BLAS_MISTAKES = ["ignore_trans_a", "ignore_trans_b", "swap_alpha_beta", "read_c0_always", "beta_unscaled"]


@pytest.mark.parametrize("mistake", BLAS_MISTAKES)
def test_planted_blas_mistake_is_caught(mistake):
    fn = _blas_with_mistake(mistake)
    failed = []
    for p in BLAS_PINS:
        try:
            if not p(fn):
                failed.append(p.__name__)
        except (ValueError, TypeError):
            failed.append(p.__name__)
    assert failed, f"planted mistake {mistake!r} passed every BLAS pin"
