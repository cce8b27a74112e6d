"""Seeded synthetic inputs for the FP32 GEMM workloads.

This module only draws random matrices; it holds none of the product's
arithmetic, so both the GPU library's tests/benchmark and the CPU oracle's
tests can take their inputs from it without sharing any GEMM code.

Generator (the pages name no generator; this is the reading adopted):
numpy.random.default_rng(seed) (PCG64), drawing A first and then B from the
same generator, in float64, then rounding to float32 (round to nearest):
  * "uniform": uniform(-1.0, 1.0)
  * "normal":  standard_normal()
  * "int4":    integers(-4, 5), i.e. small integers in {-4, ..., 4}, which are
               exact in FP32 and keep every partial sum exact for K <= 1024.

All matrices are row-major and dense: lda = K, ldb = N, ldc = N.
"""
from dataclasses import dataclass
import hashlib

import numpy as np

DISTRIBUTIONS = ("uniform", "normal", "int4")


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist: str
    seed: int

    @property
    def flops(self) -> int:
        """Floating-point operations counted as 2*M*N*K (one multiply-add = 2)."""
        return 2 * self.M * self.N * self.K

    @property
    def shape(self):
        return (self.M, self.N, self.K)


# The square and long-K workloads the GEMM is measured and checked on.
WORKLOADS = {
    w.name: w for w in (
        Workload("sgemm_256", 256, 256, 256, "uniform", 0),
        Workload("sgemm_1024", 1024, 1024, 1024, "uniform", 1),
        Workload("sgemm_1024_int", 1024, 1024, 1024, "int4", 1),
        Workload("sgemm_2048", 2048, 2048, 2048, "normal", 2),
        Workload("sgemm_4096", 4096, 4096, 4096, "uniform", 3),
        Workload("sgemm_1024x1024x16384", 1024, 1024, 16384, "normal", 4),
    )
}

HEADLINE = "sgemm_4096"


def draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """One float32 matrix of the given distribution (drawn in float64, rounded)."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "int4":
        x = rng.integers(-4, 5, size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return np.ascontiguousarray(x, dtype=np.float32)


def generate(M: int, N: int, K: int, dist: str, seed: int):
    """Return (A, B): A is M x K, B is K x N, float32, row-major, A drawn first."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), dist)
    B = draw(rng, (K, N), dist)
    return A, B


def generate_workload(w: Workload):
    return generate(w.M, w.N, w.K, w.dist, w.seed)


def sha256(x: np.ndarray) -> str:
    """Digest of a matrix's bytes, recorded with results."""
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    """Throughput in TFLOP/s, counting 2*M*N*K operations (multiply-add = 2)."""
    return 2.0 * M * N * K / seconds / 1e12
