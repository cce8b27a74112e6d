"""The seeded input generator: determinism, distributions, recorded digests."""
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_sha256.txt")


def test_deterministic():
    A1, B1 = workloads.generate(64, 32, 48, "normal", 7)
    A2, B2 = workloads.generate(64, 32, 48, "normal", 7)
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2)
    A3, _ = workloads.generate(64, 32, 48, "normal", 8)
    assert not np.array_equal(A1, A3)


def test_a_drawn_before_b():
    rng = np.random.default_rng(3)
    a = rng.uniform(-1.0, 1.0, (16, 8)).astype(np.float32)
    b = rng.uniform(-1.0, 1.0, (8, 4)).astype(np.float32)
    A, B = workloads.generate(16, 4, 8, "uniform", 3)
    assert np.array_equal(A, a) and np.array_equal(B, b)


@pytest.mark.parametrize("dist", workloads.DISTRIBUTIONS)
def test_layout_and_dtype(dist):
    A, B = workloads.generate(33, 17, 9, dist, 0)
    assert A.shape == (33, 9) and B.shape == (9, 17)
    assert A.dtype == np.float32 and B.dtype == np.float32
    assert A.flags.c_contiguous and B.flags.c_contiguous


def test_distribution_ranges():
    A, B = workloads.generate(256, 256, 256, "uniform", 0)
    assert A.min() >= -1.0 and A.max() <= 1.0
    assert abs(float(A.mean())) < 0.01 and abs(float(A.var()) - 1 / 3) < 0.01
    A, B = workloads.generate(256, 256, 256, "normal", 0)
    assert abs(float(A.mean())) < 0.01 and abs(float(A.var()) - 1.0) < 0.02
    A, B = workloads.generate(256, 256, 256, "int4", 0)
    vals = set(np.unique(np.concatenate([A.ravel(), B.ravel()])).tolist())
    assert vals == set(float(v) for v in range(-4, 5))


def test_workload_table():
    w = workloads.WORKLOADS
    assert w["sgemm_4096"].shape == (4096, 4096, 4096)
    assert w["sgemm_1024x1024x16384"].shape == (1024, 1024, 16384)
    assert w["sgemm_1024_int"].dist == "int4" and w["sgemm_1024_int"].seed == 1
    for v in w.values():
        assert v.flops == 2 * v.M * v.N * v.K
        assert v.M % 256 == 0 and v.N % 256 == 0 and v.K % 256 == 0


def test_hashes_match_golden():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert {r[0] for r in rows} == set(workloads.WORKLOADS)
    for name, M, N, K, dist, seed, ha, hb in rows:
        w = workloads.WORKLOADS[name]
        assert (w.M, w.N, w.K, w.dist, w.seed) == (int(M), int(N), int(K), dist, int(seed))
        A, B = workloads.generate_workload(w)
        assert workloads.sha256(A) == ha and workloads.sha256(B) == hb, name
