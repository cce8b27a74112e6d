"""GPU parity: the HIP library (through its C-ABI) against the FP64 CPU oracle.

Acceptance per element: finite and |C_gpu - C_ref| <= 1e-5 * S with
S = sum_k |A[m,k] B[k,n]| (tolerance of the GEMM's accuracy target); on
integer-valued inputs, bit-exact.  The pages' own looser check (finite, and
max |err| / max |ref| < 1e-4; "Beyond Kernel 7", section "What the result
establishes") is reported alongside.
"""
import sys

import numpy as np
import pytest

import fp32_sgemm_f32_amd as sg
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-5


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sg.library()
    return torch.device("cuda:0")


def to_dev(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def gpu_matmul(A, B, dev, config=sg.CFG_AUTO, sched=sg.SCHED_AUTO):
    import torch
    C = sg.matmul(to_dev(A, dev), to_dev(B, dev), config=config, sched=sched)
    torch.cuda.synchronize()
    return C.cpu().numpy()


# Configurations that run shapes their tile does not divide (the vector ones
# when N and K are multiples of 4; the general one always).
EDGE_CFGS = [sg.CFG_DL_64x64x32, sg.CFG_DL_64x64x64, sg.CFG_DL_128x128x32, sg.CFG_DL_256x256x16,
             sg.CFG_GENERIC_64x64x16]


def fits(config, M, N, K, vector=None):
    """Whether a forced configuration runs this shape (dense operands: the
    vector layout holds when N and K are multiples of 4)."""
    if config in (sg.CFG_AUTO, sg.CFG_GENERIC_64x64x16):
        return True
    if config == sg.CFG_SKINNY_16x256:   # at most 16 rows, any layout
        return M <= 16
    if config == sg.CFG_ROWDOT_N8:       # at most 8 columns, any layout
        return N <= 8
    if vector is None:
        vector = N % 4 == 0 and K % 4 == 0
    if not vector:
        return False
    bm, bn, bk = sg.CFG_TILES[config]
    return config in EDGE_CFGS or (M % bm == 0 and N % bn == 0 and K % bk == 0)


def check(C, C_ref, S, label):
    ok, worst = oracle.within_bound(C, C_ref, S, TOL)
    pages = float(np.max(np.abs(C - C_ref)) / max(np.max(np.abs(C_ref)), 1e-300))
    log(f"  {label}: max|err|/S = {worst:.3e}, pages' max|err|/max|ref| = {pages:.3e}")
    assert ok, f"{label}: per-element bound violated (worst {worst:.3e})"
    assert pages < 1e-4


CONFIGS = list(range(sg.NUM_CFGS))
SCHEDS = [sg.SCHED_AUTO, sg.SCHED_DP, sg.SCHED_STREAMK]
# Several tiles each way, uneven Stream-K splits (K chunks not divisible by
# the grid), non-square shapes, and the smallest accepted shape.
SHAPES = [(512, 512, 512), (768, 512, 416), (256, 1280, 1152), (1536, 256, 2080), (128, 128, 32)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("sched", SCHEDS, ids=lambda s: sg.SCHED_NAMES[s])
@pytest.mark.parametrize("config", CONFIGS, ids=lambda c: sg.CFG_NAMES[c])
def test_parity_random(dev, config, sched, shape):
    M, N, K = shape
    log(f"case config={sg.CFG_NAMES[config]} sched={sg.SCHED_NAMES[sched]} shape={shape}")
    A, B = workloads.generate(M, N, K, "uniform", 1000 + M + N + K)
    if not fits(config, M, N, K):
        import torch
        with pytest.raises(sg.SgemmError) as e:
            sg.matmul(to_dev(A, dev), to_dev(B, dev), config=config, sched=sched)
        torch.cuda.synchronize()
        assert e.value.status == sg.ERR_CONFIG
        return
    C = gpu_matmul(A, B, dev, config, sched)
    C_ref, S = oracle.gemm(A, B)
    check(C, C_ref, S, f"{sg.CFG_NAMES[config]}/{sg.SCHED_NAMES[sched]}")


@pytest.mark.parametrize("sched", SCHEDS, ids=lambda s: sg.SCHED_NAMES[s])
@pytest.mark.parametrize("config", CONFIGS, ids=lambda c: sg.CFG_NAMES[c])
def test_integer_inputs_bit_exact(dev, config, sched):
    """Entries in {-4..4} with K <= 1024: every partial sum is an integer below
    2^24, exact in FP32 in any order, so every variant must match exactly
    (16 rows for the skinny kernel, which runs at most that many)."""
    M, N, K = (16 if config == sg.CFG_SKINNY_16x256 else 512), (8 if config == sg.CFG_ROWDOT_N8 else 768), 1024
    log(f"case int4 config={sg.CFG_NAMES[config]} sched={sg.SCHED_NAMES[sched]}")
    A, B = workloads.generate(M, N, K, "int4", 77)
    C = gpu_matmul(A, B, dev, config, sched)
    C_ref, _ = oracle.gemm(A, B)
    assert np.array_equal(C.astype(np.float64), C_ref)


@pytest.mark.parametrize("config", CONFIGS, ids=lambda c: sg.CFG_NAMES[c])
def test_identity_b_gives_a(dev, config):
    M, K = (16 if config == sg.CFG_SKINNY_16x256 else 512), (8 if config == sg.CFG_ROWDOT_N8 else 256)
    log(f"case identity config={sg.CFG_NAMES[config]}")
    A, _ = workloads.generate(M, K, K, "normal", 5)
    C = gpu_matmul(A, np.eye(K, dtype=np.float32), dev, config, sg.SCHED_STREAMK)
    assert np.array_equal(C, A)


def test_all_ones_a_gives_column_sums(dev):
    M, N, K = 256, 384, 1024
    log("case all-ones A")
    _, B = workloads.generate(M, N, K, "int4", 6)
    C = gpu_matmul(np.ones((M, K), np.float32), B, dev)
    assert np.array_equal(C, np.tile(B.astype(np.int64).sum(axis=0), (M, 1)).astype(np.float32))


def test_k_zero_writes_zeros(dev):
    import torch
    log("case K=0")
    A = torch.empty((256, 0), dtype=torch.float32, device=dev)
    B = torch.empty((0, 384), dtype=torch.float32, device=dev)
    C = torch.full((256, 384), float("nan"), dtype=torch.float32, device=dev)
    sg.matmul(A, B, out=C)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C).item() == 0


def test_empty_m_is_a_no_op(dev):
    import torch
    log("case M=0")
    A = torch.zeros((0, 64), dtype=torch.float32, device=dev)
    B = torch.zeros((64, 128), dtype=torch.float32, device=dev)
    C = sg.matmul(A, B)
    torch.cuda.synchronize()
    assert C.shape == (0, 128)


# ---------------------------------------------------------------------------
# Arbitrary shapes: ragged edges in M, N and K (the edge-masking vector
# kernels when N and K are multiples of 4, else the general kernel), odd
# leading dimensions and pointers that are only float-aligned.
# ---------------------------------------------------------------------------

RAGGED = [(1, 1, 1), (7, 13, 5), (33, 68, 20), (100, 196, 36), (129, 260, 100), (300, 68, 1004),
          (517, 384, 772), (257, 511, 129), (1000, 1000, 1000)]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("sched", SCHEDS, ids=lambda s: sg.SCHED_NAMES[s])
@pytest.mark.parametrize("config", [sg.CFG_AUTO] + EDGE_CFGS, ids=lambda c: sg.CFG_NAMES[c])
def test_parity_ragged(dev, config, sched, shape):
    M, N, K = shape
    log(f"case ragged config={sg.CFG_NAMES[config]} sched={sg.SCHED_NAMES[sched]} shape={shape}")
    A, B = workloads.generate(M, N, K, "normal", 2000 + M + 3 * N + 7 * K)
    if not fits(config, M, N, K):
        import torch
        with pytest.raises(sg.SgemmError) as e:
            sg.matmul(to_dev(A, dev), to_dev(B, dev), config=config, sched=sched)
        torch.cuda.synchronize()
        assert e.value.status == sg.ERR_CONFIG
        return
    C = gpu_matmul(A, B, dev, config, sched)
    C_ref, S = oracle.gemm(A, B)
    check(C, C_ref, S, f"{sg.CFG_NAMES[config]}/{sg.SCHED_NAMES[sched]}")


@pytest.mark.parametrize("config", [sg.CFG_AUTO] + EDGE_CFGS, ids=lambda c: sg.CFG_NAMES[c])
def test_ragged_integer_inputs_bit_exact(dev, config):
    M, N, K = 517, 772, 1004
    log(f"case ragged int4 config={sg.CFG_NAMES[config]}")
    A, B = workloads.generate(M, N, K, "int4", 78)
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        C = gpu_matmul(A, B, dev, config, sched)
        C_ref, _ = oracle.gemm(A, B)
        assert np.array_equal(C.astype(np.float64), C_ref)


@pytest.mark.parametrize("case", ["a_offset", "b_offset", "c_offset", "odd_ld"])
def test_float_aligned_layouts_run_on_the_general_kernel(dev, case):
    """Operands that start 4 bytes past a 16-byte boundary, and leading
    dimensions that are not multiples of 4: correct results (the general
    kernel), C's padding untouched; a forced vector kernel is refused."""
    import torch
    M, N, K = 130, 196, 72
    log(f"case layout {case}")
    A, B = workloads.generate(M, N, K, "normal", 13)
    extra = {"a_offset": (1, 0, 0), "b_offset": (0, 1, 0), "c_offset": (0, 0, 1)}.get(case, (0, 0, 0))
    pad = 3 if case == "odd_ld" else 0
    Abuf = torch.full((M * (K + pad) + 4,), float("nan"), device=dev)
    Bbuf = torch.full((K * (N + pad) + 4,), float("nan"), device=dev)
    Cbuf = torch.full((M * (N + pad) + 4,), float("nan"), device=dev)
    Av = Abuf[extra[0]:extra[0] + M * (K + pad)].view(M, K + pad)[:, :K]
    Bv = Bbuf[extra[1]:extra[1] + K * (N + pad)].view(K, N + pad)[:, :N]
    Cv = Cbuf[extra[2]:extra[2] + M * (N + pad)].view(M, N + pad)[:, :N]
    Av.copy_(to_dev(A, dev))
    Bv.copy_(to_dev(B, dev))
    with pytest.raises(sg.SgemmError) as e:
        sg.matmul(Av, Bv, out=Cv, config=sg.CFG_DL_64x64x32)
    assert e.value.status == sg.ERR_CONFIG
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        sg.matmul(Av, Bv, out=Cv, sched=sched)
        torch.cuda.synchronize()
        C_ref, S = oracle.gemm(A, B)
        check(Cv.cpu().numpy(), C_ref, S, f"{case}/{sg.SCHED_NAMES[sched]}")
    if pad:
        full = Cbuf[:M * (N + pad)].view(M, N + pad).cpu().numpy()
        assert np.all(np.isnan(full[:, N:])), "ldc padding was written"


# ---------------------------------------------------------------------------
# The BLAS form: C = alpha op(A) op(B) + beta C, either storage order of A
# and B (sgemm_f32_gemm).
# ---------------------------------------------------------------------------

LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]
SCALINGS = [(1.0, 0.0), (2.5, 0.0), (1.5, -0.75), (0.0, 2.0), (-1.0, 1.0)]


def stored(X, trans):
    return np.ascontiguousarray(X.T) if trans else X


def c0_of(M, N, seed):
    return workloads.generate(M, 1, N, "normal", seed)[0]      # M x N


@pytest.mark.parametrize("shape", [(200, 136, 100), (517, 384, 772), (256, 256, 256)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("scaling", SCALINGS, ids=lambda ab: f"a{ab[0]}_b{ab[1]}")
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{l[0]}tb{l[1]}")
def test_blas_form(dev, layout, scaling, shape):
    import torch
    (ta, tb), (alpha, beta), (M, N, K) = layout, scaling, shape
    log(f"case blas ta={ta} tb={tb} alpha={alpha} beta={beta} shape={shape}")
    A, B = workloads.generate(M, N, K, "normal", 3000 + M + N + K)
    As, Bs = stored(A, ta), stored(B, tb)
    C0 = c0_of(M, N, 3100 + M)
    C_ref, S = oracle.gemm_blas(As, Bs, C0, alpha, beta, ta, tb)
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        C = to_dev(C0, dev).clone()
        sg.gemm(to_dev(As, dev), to_dev(Bs, dev), C, alpha, beta, ta, tb, sched=sched)
        torch.cuda.synchronize()
        check(C.cpu().numpy(), C_ref, S, f"blas/{sg.SCHED_NAMES[sched]}")


# The direct-to-LDS kernels load each operand in its storage order (A
# stored K x M, B stored N x K); they need the stored row lengths of A and B,
# and N, to be multiples of 4.  Shapes: tile multiples, ragged in every
# dimension, K not a multiple of 4 (only A K x M with B K x N qualifies), M
# not a multiple of 4 (only A stored M x K qualifies).
DL_LAYOUT_CFGS = [sg.CFG_DL_64x64x32, sg.CFG_DL_64x64x64, sg.CFG_DL_128x128x32, sg.CFG_DL_256x256x16]
LAYOUT_SHAPES = [(512, 512, 512), (260, 196, 100), (516, 388, 772), (132, 68, 1004), (64, 1028, 36),
                 (130, 196, 100), (128, 196, 102)]


def vector_layout(M, N, K, ta, tb):
    return (M if ta else K) % 4 == 0 and (K if tb else N) % 4 == 0 and N % 4 == 0


@pytest.mark.parametrize("shape", LAYOUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"ta{l[0]}tb{l[1]}")
@pytest.mark.parametrize("config", [sg.CFG_AUTO] + DL_LAYOUT_CFGS, ids=lambda c: sg.CFG_NAMES[c])
def test_storage_orders_on_direct_to_lds_kernels(dev, config, layout, shape):
    import torch
    (ta, tb), (M, N, K) = layout, shape
    alpha, beta = 1.5, -0.5
    log(f"case layout config={sg.CFG_NAMES[config]} ta={ta} tb={tb} shape={shape}")
    A, B = workloads.generate(M, N, K, "normal", 4000 + M + 3 * N + 7 * K)
    As, Bs = stored(A, ta), stored(B, tb)
    C0 = c0_of(M, N, 4100 + K)
    if config != sg.CFG_AUTO and not vector_layout(M, N, K, ta, tb):
        with pytest.raises(sg.SgemmError) as e:
            sg.gemm(to_dev(As, dev), to_dev(Bs, dev), to_dev(C0, dev), alpha, beta, ta, tb, config=config)
        torch.cuda.synchronize()
        assert e.value.status == sg.ERR_CONFIG
        return
    C_ref, S = oracle.gemm_blas(As, Bs, C0, alpha, beta, ta, tb)
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        C = to_dev(C0, dev).clone()
        sg.gemm(to_dev(As, dev), to_dev(Bs, dev), C, alpha, beta, ta, tb, config=config, sched=sched)
        torch.cuda.synchronize()
        check(C.cpu().numpy(), C_ref, S, f"{sg.CFG_NAMES[config]}/ta{ta}tb{tb}/{sg.SCHED_NAMES[sched]}")


@pytest.mark.parametrize("layout", LAYOUTS[1:], ids=lambda l: f"ta{l[0]}tb{l[1]}")
@pytest.mark.parametrize("config", DL_LAYOUT_CFGS, ids=lambda c: sg.CFG_NAMES[c])
def test_storage_orders_integer_inputs_bit_exact(dev, config, layout):
    import torch
    ta, tb = layout
    M, N, K = 516, 772, 1004
    log(f"case layout int4 config={sg.CFG_NAMES[config]} ta={ta} tb={tb}")
    A, B = workloads.generate(M, N, K, "int4", 79)
    As, Bs = stored(A, ta), stored(B, tb)
    C_ref, _ = oracle.gemm_blas(As, Bs, None, 1.0, 0.0, ta, tb)
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        sg.gemm(to_dev(As, dev), to_dev(Bs, dev), C, 1.0, 0.0, ta, tb, config=config, sched=sched)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)


@pytest.mark.parametrize("config", [sg.CFG_MFMA_256x256x16, sg.CFG_MFMA_128x128x32, sg.CFG_VALU_128x128x8,
                                    sg.CFG_VALU_256x128x8, sg.CFG_DL_64x64x64, sg.CFG_DL_128x128x32_K2, sg.CFG_GENERIC_64x64x16,
                                    sg.CFG_SKINNY_16x256, sg.CFG_ROWDOT_N8],
                         ids=lambda c: sg.CFG_NAMES[c])
def test_blas_scaling_on_every_kernel_family(dev, config):
    """alpha / beta in the epilogue of each kernel family, whole tiles and
    Stream-K (the scaling is applied once, after the partial sums)."""
    import torch
    M, N, K = (13 if config == sg.CFG_SKINNY_16x256 else 512), (5 if config == sg.CFG_ROWDOT_N8 else 512), 768
    log(f"case blas scaling config={sg.CFG_NAMES[config]}")
    A, B = workloads.generate(M, N, K, "int4", 61)
    C0 = workloads.generate(M, 1, N, "int4", 62)[0]
    C_ref, _ = oracle.gemm_blas(A, B, C0, 2.0, -3.0)
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        C = to_dev(C0, dev).clone()
        sg.gemm(to_dev(A, dev), to_dev(B, dev), C, 2.0, -3.0, config=config, sched=sched)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)   # integers: exact


def test_blas_beta_zero_does_not_read_c(dev):
    import torch
    M, N, K = 300, 260, 200
    log("case blas beta=0 with NaN C")
    A, B = workloads.generate(M, N, K, "normal", 63)
    C = torch.full((M, N), float("nan"), device=dev)
    sg.gemm(to_dev(A, dev), to_dev(B, dev), C, 1.25, 0.0)
    torch.cuda.synchronize()
    C_ref, S = oracle.gemm_blas(A, B, None, 1.25, 0.0)
    check(C.cpu().numpy(), C_ref, S, "beta=0")


def test_blas_alpha_zero_and_empty_k_scale_c(dev):
    """alpha = 0 or K = 0: C = beta C, and A, B are not read (null here)."""
    import torch
    M, N = 130, 70
    log("case blas alpha=0 / K=0")
    C0 = c0_of(M, N, 64)
    for K, alpha in ((50, 0.0), (0, 3.0)):
        C = to_dev(C0, dev).clone()
        st = sg.gemm_raw(0, 0, M, N, K, alpha, 0, max(K, 1), 0, N, -0.5, C.data_ptr(), N,
                         torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == sg.OK
        assert np.array_equal(C.cpu().numpy(), (np.float32(-0.5) * C0).astype(np.float32))
    C = to_dev(C0, dev).clone()
    st = sg.gemm_raw(0, 0, M, N, 0, 1.0, 0, 1, 0, N, 0.0, C.data_ptr(), N,
                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == sg.OK and torch.count_nonzero(C).item() == 0


def test_blas_rejects_bad_transpose_flag(dev):
    assert sg.gemm_raw(2, 0, 64, 64, 64, 1.0, 0, 64, 0, 64, 0.0, 0, 64) == sg.ERR_CONFIG


@pytest.mark.parametrize("config", [sg.CFG_AUTO, sg.CFG_MFMA_128x128x32, sg.CFG_VALU_128x128x8],
                         ids=lambda c: sg.CFG_NAMES[c])
def test_padded_leading_dimensions_and_untouched_gap(dev, config):
    """lda > K, ldb > N, ldc > N: results use only the logical region, and C's
    padding columns (NaN sentinels) are never written."""
    import torch
    M, N, K = 384, 256, 320
    log(f"case padded ld config={sg.CFG_NAMES[config]}")
    A, B = workloads.generate(M, N, K, "normal", 9)
    Ap = torch.full((M, K + 12), float("nan"), device=dev)
    Bp = torch.full((K, N + 36), float("nan"), device=dev)
    Cp = torch.full((M, N + 20), float("nan"), device=dev)
    Ap[:, :K] = to_dev(A, dev)
    Bp[:, :N] = to_dev(B, dev)
    sg.matmul(Ap[:, :K], Bp[:, :N], out=Cp[:, :N], config=config, sched=sg.SCHED_STREAMK)
    torch.cuda.synchronize()
    Cn = Cp.cpu().numpy()
    assert np.all(np.isnan(Cn[:, N:])), "ldc padding was written"
    C_ref, S = oracle.gemm(A, B)
    check(Cn[:, :N], C_ref, S, "padded")


@pytest.mark.parametrize("config", [sg.CFG_MFMA_128x128x32, sg.CFG_MFMA_256x256x16, sg.CFG_VALU_128x128x8,
                                    sg.CFG_VALU_256x128x8],
                         ids=lambda c: sg.CFG_NAMES[c])
def test_repeatable_and_fully_written(dev, config):
    """C pre-filled with NaN is fully overwritten; repeated split runs are
    bit-identical (the partial sums are combined in a fixed order)."""
    import torch
    M, N, K = 512, 512, 2048
    log(f"case repeatability config={sg.CFG_NAMES[config]}")
    A, B = workloads.generate(M, N, K, "normal", 10)
    Ad, Bd = to_dev(A, dev), to_dev(B, dev)
    outs = []
    for _ in range(3):
        C = torch.full((M, N), float("nan"), device=dev)
        sg.matmul(Ad, Bd, out=C, config=config, sched=sg.SCHED_STREAMK)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_non_default_stream(dev):
    import torch
    M, N, K = 512, 256, 1024
    log("case non-default stream")
    A, B = workloads.generate(M, N, K, "uniform", 11)
    s = torch.cuda.Stream(device=dev)
    Ad, Bd = to_dev(A, dev), to_dev(B, dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = sg.matmul(Ad, Bd)
    s.synchronize()
    C_ref, S = oracle.gemm(A, B)
    check(C.cpu().numpy(), C_ref, S, "side stream")


def test_repacked_calls_from_two_threads_on_one_stream(dev):
    """Two host threads make repacked calls (odd N: A and B copied into the
    library's per-stream buffer, then the product) on ONE stream, with no
    host synchronisation, starting from no buffer so that the first calls
    grow it.  Each call's copies and product must run back to back on the
    stream; another thread's copy in between would hand the product the
    wrong operands.  Integer inputs: every result exact."""
    import threading
    import torch
    log("case two threads, one stream, repacked")
    shapes = [(515, 771, 1021), (1031, 517, 770)]
    assert all(sg.plan(*s)["repacked"] == 1 for s in shapes)
    s = torch.cuda.Stream(device=dev)
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = workloads.generate(M, N, K, "int4", 120 + i)
        outs = [torch.full((M, N), float("nan"), dtype=torch.float32, device=dev) for _ in range(12)]
        data.append((A, B, to_dev(A, dev), to_dev(B, dev), outs))
    torch.cuda.synchronize()
    sg.release()   # start with no repacking buffer: the first calls grow it
    errors = []
    go = threading.Barrier(2)

    def worker(i):
        try:
            _, _, Ad, Bd, outs = data[i]
            go.wait()
            for C in outs:
                sg.matmul(Ad, Bd, out=C, stream=s)
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for A, B, _, _, outs in data:
        C_ref, _ = oracle.gemm(A, B)
        for C in outs:
            assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)


def test_concurrent_streams_with_split_tiles(dev):
    """Stream-K calls on two streams with no host synchronisation between
    them: each stream has its own workspace, so the partial tiles of one
    never meet the other's (integer inputs: every
    result exact, every repeat identical)."""
    import torch
    log("case two streams, Stream-K")
    shapes = [(512, 512, 4096), (384, 640, 2048)]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = workloads.generate(M, N, K, "int4", 95 + i)
        data.append((A, B, to_dev(A, dev), to_dev(B, dev)))
    torch.cuda.synchronize()
    outs = [[], []]
    for rep in range(4):
        for i, s in enumerate(streams):
            _, _, Ad, Bd = data[i]
            with torch.cuda.stream(s):
                outs[i].append(sg.matmul(Ad, Bd, sched=sg.SCHED_STREAMK))
    torch.cuda.synchronize()
    for i in range(2):
        A, B, _, _ = data[i]
        C_ref, _ = oracle.gemm(A, B)
        for C in outs[i]:
            assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)


@pytest.mark.parametrize("sched", [sg.SCHED_DP, sg.SCHED_STREAMK], ids=lambda s: sg.SCHED_NAMES[s])
def test_graph_capture_and_replay(dev, sched):
    """Calls captured into a HIP graph (after one eager call has set up the
    Stream-K workspace) replay correctly: new inputs are written between the
    replays, with eager work and synchronisations in between, and every
    replay matches the oracle and the eager result exactly (integer inputs)."""
    import torch
    M, N, K = 768, 512, 1024
    log(f"case graph capture sched={sg.SCHED_NAMES[sched]}")
    s = torch.cuda.Stream(device=dev)
    A0, B = workloads.generate(M, N, K, "int4", 96)
    Ad, Bd = to_dev(A0, dev), to_dev(B, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    with torch.cuda.stream(s):
        sg.gemm(Ad, Bd, C, 1.0, 0.0, sched=sched)          # eager: workspace ready
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sg.gemm(Ad, Bd, C, 1.0, 0.0, sched=sched)
    torch.cuda.synchronize()
    for r in range(3):
        A_r = workloads.generate(M, N, K, "int4", 200 + r)[0]
        Ad.copy_(to_dev(A_r, dev))
        E = sg.matmul(Ad, Bd, sched=sched)                 # eager reference on the device
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm(A_r, B)
        got = C.cpu().numpy()
        assert np.array_equal(got.astype(np.float64), C_ref), f"replay {r}"
        assert np.array_equal(got, E.cpu().numpy()), f"replay {r} vs eager"


def test_rejects_bad_memory_and_leaves_c_untouched(dev):
    import ctypes

    import torch
    log("case pointer checks")
    M, N, K = 256, 256, 256
    Ad = torch.zeros((M, K), device=dev)
    Bd = torch.zeros((K, N), device=dev)
    C = torch.full((M, N), 7.0, device=dev)
    host = np.zeros((M, K), np.float32)
    st = sg.sgemm_raw(M, N, K, host.ctypes.data, K, Bd.data_ptr(), N, C.data_ptr(), N)
    assert st == sg.ERR_POINTER
    with pytest.raises(sg.SgemmError) as e:
        sg.matmul(Ad[:128], Bd[:, :128], config=sg.CFG_MFMA_256x256x16)
    assert e.value.status == sg.ERR_CONFIG
    torch.cuda.synchronize()
    assert torch.all(C == 7.0).item()
    assert sg.last_hip_error() == 0

    # A matrix whose extent runs past its own allocation (hipMalloc of 128 rows,
    # used as 256): refused unless the runtime reports a larger allocation, in
    # which case the access stays inside mapped memory.
    hip = ctypes.CDLL("libamdhip64.so")
    ptr = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(ptr), ctypes.c_size_t(128 * K * 4)) == 0
    try:
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        assert hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), ptr) == 0
        C2 = torch.empty((M, N), device=dev)
        st = sg.sgemm_raw(M, N, K, ptr.value, K, Bd.data_ptr(), N, C2.data_ptr(), N)
        torch.cuda.synchronize()
        if size.value < M * K * 4:
            assert st == sg.ERR_POINTER
        else:
            assert st == sg.OK
    finally:
        hip.hipFree(ptr)


def test_release_then_reuse(dev):
    log("case release")
    M, N, K = 256, 256, 512
    A, B = workloads.generate(M, N, K, "int4", 12)
    C1 = gpu_matmul(A, B, dev, sg.CFG_MFMA_128x128x32, sg.SCHED_STREAMK)
    sg.release()
    C2 = gpu_matmul(A, B, dev, sg.CFG_MFMA_128x128x32, sg.SCHED_STREAMK)
    assert np.array_equal(C1, C2)


# ---------------------------------------------------------------------------
# The measured workloads at full size, in the launch configuration the
# benchmark times (automatic choice).
# ---------------------------------------------------------------------------

# The oracle's full product of each workload, computed once per module (the
# storage-order cases reuse the plain ones' operands).
_FULL_REF = {}


def full_reference(w):
    if w.name not in _FULL_REF:
        A, B = workloads.generate_workload(w)
        C_ref, S = oracle.gemm(A, B)
        _FULL_REF.clear()   # one workload's reference held at a time
        _FULL_REF[w.name] = (A, B, C_ref, S)
    return _FULL_REF[w.name]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(dev, name):
    """Every element of every measured workload against the FP64 oracle's
    full product (4096^3: 16.7 M elements), in the launch configuration the
    benchmark times; the integer-valued one bit-exact."""
    w = workloads.WORKLOADS[name]
    log(f"case workload {name} {w.shape} {w.dist} seed {w.seed}")
    A, B, C_ref, S = full_reference(w)
    C = gpu_matmul(A, B, dev)
    assert np.all(np.isfinite(C))
    if w.dist == "int4":
        assert np.array_equal(C.astype(np.float64), C_ref)
        return
    check(C, C_ref, S, name)


@pytest.mark.parametrize("layout", LAYOUTS[1:], ids=lambda l: f"ta{l[0]}tb{l[1]}")
@pytest.mark.parametrize("name", ["sgemm_4096", "sgemm_2048", "sgemm_1024x1024x16384"])
def test_workload_full_size_storage_orders(dev, name, layout):
    """The measured workloads with A stored K x M and / or B stored N x K, at
    full size, in the automatic choice (the direct-to-LDS kernels): every
    element against the oracle's full product."""
    import torch
    ta, tb = layout
    w = workloads.WORKLOADS[name]
    log(f"case workload {name} ta={ta} tb={tb}")
    A, B, C_ref, S = full_reference(w)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    sg.gemm(to_dev(stored(A, ta), dev), to_dev(stored(B, tb), dev), C, 1.0, 0.0, ta, tb)
    torch.cuda.synchronize()
    check(C.cpu().numpy(), C_ref, S, f"{name} ta={ta} tb={tb}")


@pytest.mark.parametrize("name", ["sgemm_4096", "sgemm_2048", "sgemm_1024", "sgemm_1024_int",
                                  "sgemm_1024x1024x16384"])
def test_compile_time_shape_kernels(dev, name):
    """SGEMM_SCHED_FIXED (the kernel compiled for the product's exact shape):
    every element against the oracle (the integer variant exact), and the
    same bits as the runtime kernel of the same configuration, which sums in
    the same order."""
    w = workloads.WORKLOADS[name]
    log(f"case compile-time shape {name} {w.shape}")
    A, B, C_ref, S = full_reference(w)
    C_fixed = gpu_matmul(A, B, dev, sched=sg.SCHED_FIXED)
    C_dp = gpu_matmul(A, B, dev, sched=sg.SCHED_DP)
    assert np.array_equal(C_fixed.view(np.uint32), C_dp.view(np.uint32))
    if w.dist == "int4":
        assert np.array_equal(C_fixed.astype(np.float64), C_ref)
    else:
        check(C_fixed, C_ref, S, f"{name} fixed")


def test_compile_time_shape_refuses_other_calls(dev):
    """Only the dense plain product of a compiled shape runs on those kernels;
    a padded leading dimension, scaling, a transposed operand or another
    shape is refused before any work (C untouched)."""
    import torch
    M = N = K = 1024
    A, B = workloads.generate(M, N, K, "int4", 130)
    Ad, Bd = to_dev(A, dev), to_dev(B, dev)
    Cbuf = torch.full((M, N + 4), 5.0, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    cases = {
        "padded_ldc": lambda: sg.sgemm_raw(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, Cbuf.data_ptr(), N + 4, s,
                                           sg.CFG_AUTO, sg.SCHED_FIXED),
        "scaled": lambda: sg.gemm_raw(0, 0, M, N, K, 2.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0, Cbuf.data_ptr(),
                                      N + 4, s, sg.CFG_AUTO, sg.SCHED_FIXED),
        "transposed_b": lambda: sg.gemm_raw(0, 1, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), K, 0.0,
                                            Cbuf.data_ptr(), N + 4, s, sg.CFG_AUTO, sg.SCHED_FIXED),
        "other_shape": lambda: sg.sgemm_raw(M, N, 512, Ad.data_ptr(), K, Bd.data_ptr(), N, Cbuf.data_ptr(), N + 4,
                                            s, sg.CFG_AUTO, sg.SCHED_FIXED),
    }
    for case, fn in cases.items():
        log(f"case compile-time shape refusal {case}")
        assert fn() == sg.ERR_CONFIG, case
    torch.cuda.synchronize()
    assert bool((Cbuf == 5.0).all().item())


# Leading dimensions just beyond the reach of the direct-to-LDS kernels'
# 32-bit source offsets (BM or BK rows of A, BK or BN rows of B, times the
# leading dimension, under 2^32 bytes; 2^31 for the edge-masking ones): the
# automatic choice falls back (register-staged kernel for whole tiles, the
# general kernel for edges and transposed operands) and a forced
# direct-to-LDS configuration is refused.  Buffers of 2-4 GiB.
LD_CASES = {
    # name: (trans_a, trans_b, M, N, K, lda, ldb)
    "nn_lda": (0, 0, 64, 128, 64, 2 ** 24 + 4, 128),
    "nn_ldb": (0, 0, 128, 64, 64, 64, 2 ** 24 + 4),
    "tn_lda": (1, 0, 128, 128, 64, 2 ** 24 + 4, 128),        # whole tiles: 2^32 limit
    "nt_ldb_ragged": (0, 1, 100, 64, 64, 64, 2 ** 23 + 4),   # edge masking: 2^31 limit
}


@pytest.mark.parametrize("case", list(LD_CASES))
def test_leading_dimensions_beyond_32bit_offsets(dev, case):
    import torch
    ta, tb, M, N, K, lda, ldb = LD_CASES[case]
    log(f"case large ld {case}: ta={ta} tb={tb} shape=({M},{N},{K}) lda={lda} ldb={ldb}")
    A, B = workloads.generate(M, N, K, "int4", 90)
    As, Bs = stored(A, ta), stored(B, tb)

    def padded(X, ld):
        rows, cols = X.shape
        buf = torch.zeros((rows - 1) * ld + cols, dtype=torch.float32, device=dev)
        view = torch.as_strided(buf, (rows, cols), (ld, 1))
        view.copy_(to_dev(X, dev))
        return buf, view

    Abuf, Av = padded(As, lda)
    Bbuf, Bv = padded(Bs, ldb)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    with pytest.raises(sg.SgemmError) as e:
        sg.gemm(Av, Bv, C, 1.0, 0.0, ta, tb, config=sg.CFG_DL_64x64x64)
    assert e.value.status == sg.ERR_CONFIG
    for sched in (sg.SCHED_DP, sg.SCHED_STREAMK):
        C.fill_(float("nan"))
        sg.gemm(Av, Bv, C, 1.0, 0.0, ta, tb, sched=sched)
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(As, Bs, None, 1.0, 0.0, ta, tb)
        assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)   # integers: exact
    del Abuf, Bbuf, Av, Bv
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Seeded random cases across the whole interface: shape, storage orders,
# alpha / beta, padded leading dimensions, float-offset pointers, forced
# configuration and schedule.  A forced configuration may refuse
# (SGEMM_ERR_CONFIG) only if it is neither the automatic choice nor the
# general kernel; every result is checked element by element against the
# FP64 oracle, and C's padding must stay untouched.
# ---------------------------------------------------------------------------

def random_case(rng):
    def dim():
        r = rng.random()
        if r < 0.3:
            return int(rng.integers(1, 40))
        if r < 0.6:
            return int(rng.choice([64, 128, 192, 256, 384, 512]))
        return int(rng.integers(40, 600))
    M, N, K = dim(), dim(), dim()
    ta, tb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    alpha, beta = [(1.0, 0.0), (1.0, 0.0), (-0.5, 0.0), (1.5, 2.0), (0.0, -1.0), (2.0, 1.0)][int(rng.integers(0, 6))]
    pads = [int(rng.choice([0, 0, 0, 4, 1, 3])) for _ in range(3)]
    offs = [int(rng.choice([0, 0, 0, 0, 1, 2])) for _ in range(3)]
    config = int(rng.choice([sg.CFG_AUTO] * 4 + list(range(1, sg.NUM_CFGS))))
    sched = int(rng.choice(SCHEDS))
    return M, N, K, ta, tb, alpha, beta, pads, offs, config, sched


@pytest.mark.parametrize("seed", range(160))
def test_random_interface_cases(dev, seed):
    import torch
    rng = np.random.default_rng(7000 + seed)
    M, N, K, ta, tb, alpha, beta, pads, offs, config, sched = random_case(rng)
    log(f"case random seed={seed}: shape=({M},{N},{K}) ta={ta} tb={tb} alpha={alpha} beta={beta} "
        f"pads={pads} offs={offs} config={sg.CFG_NAMES[config]} sched={sg.SCHED_NAMES[sched]}")
    A, B = workloads.generate(M, N, K, "normal", 8000 + seed)
    As, Bs = stored(A, ta), stored(B, tb)
    C0 = c0_of(M, N, 8100 + seed)

    def placed(X, pad, off):
        rows, cols = X.shape
        ld = cols + pad
        buf = torch.full((rows * ld + off + 4,), float("nan"), dtype=torch.float32, device=dev)
        view = torch.as_strided(buf, (rows, cols), (ld, 1), off)
        view.copy_(to_dev(X, dev))
        return buf, view, ld

    _, Av, _ = placed(As, pads[0], offs[0])
    _, Bv, _ = placed(Bs, pads[1], offs[1])
    Cbuf, Cv, ldc = placed(C0, pads[2], offs[2])
    try:
        sg.gemm(Av, Bv, Cv, alpha, beta, ta, tb, config=config, sched=sched)
    except sg.SgemmError as e:
        assert e.status == sg.ERR_CONFIG and config not in (sg.CFG_AUTO, sg.CFG_GENERIC_64x64x16), e
        assert np.array_equal(Cv.cpu().numpy(), C0), "C changed on an error"
        return
    torch.cuda.synchronize()
    C_ref, S = oracle.gemm_blas(As, Bs, C0, alpha, beta, ta, tb)
    check(Cv.cpu().numpy(), C_ref, S, f"random {seed}")
    full = torch.as_strided(Cbuf, (M, ldc), (ldc, 1), offs[2]).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "ldc padding was written"


# The automatic choice over shapes like those its cost model was fitted on:
# sides log-uniform in 16..8192, multiples of 16 (of 4 one time in four),
# every storage order, integer inputs (each partial sum is an integer below
# 2^24, so every plan, split or whole, must give the exact product).
@pytest.mark.parametrize("seed", range(96))
def test_automatic_choice_random_shapes(dev, seed):
    import math
    import torch
    rng = np.random.default_rng(9100 + seed)

    def side():
        q = 4 if rng.random() < 0.25 else 16
        return max(q, int(round(math.exp(rng.uniform(math.log(16), math.log(8192))) / q)) * q)
    while True:
        M, N, K = side(), side(), side()
        if 1e6 <= M * N * K <= 1e9:
            break
    ta, tb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    p = sg.plan(M, N, K, num_cus=torch.cuda.get_device_properties(dev).multi_processor_count, trans_a=ta,
                trans_b=tb)
    log(f"case auto random seed={seed}: shape=({M},{N},{K}) ta={ta} tb={tb} config={sg.CFG_NAMES[p['config']]} "
        f"sched={sg.SCHED_NAMES[p['sched']]} dp={p['dp_tiles']} sk={p['sk_tiles']} repacked={p['repacked']}")
    A, B = workloads.generate(M, N, K, "int4", 9200 + seed)
    As, Bs = stored(A, ta), stored(B, tb)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    sg.gemm(to_dev(As, dev), to_dev(Bs, dev), C, 1.0, 0.0, ta, tb)
    torch.cuda.synchronize()
    C_ref, _ = oracle.gemm_blas(As, Bs, None, 1.0, 0.0, ta, tb)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref), f"auto random {seed}"


@pytest.mark.parametrize("views", ["a_t", "b_t", "both_t", "gemm_flip"])
def test_python_binding_takes_transposed_views(dev, views):
    """Column-major views (X.t() of a row-major X, padded rows included) run
    as the other storage order, without a copy, and give the product of the
    logical matrices."""
    import torch
    M, N, K = 200, 136, 260
    log(f"case binding views {views}")
    A, B = workloads.generate(M, N, K, "int4", 97)
    C_ref, _ = oracle.gemm(A, B)
    # Row-major storage of A^T and B^T with padded rows; their .t() views
    # are the logical A (M x K) and B (K x N), column-major.
    At = torch.zeros((K, M + 12), dtype=torch.float32, device=dev)[:, :M]
    At.copy_(to_dev(np.ascontiguousarray(A.T), dev))
    Bt = torch.zeros((N, K + 4), dtype=torch.float32, device=dev)[:, :K]
    Bt.copy_(to_dev(np.ascontiguousarray(B.T), dev))
    Ad, Bd = to_dev(A, dev), to_dev(B, dev)
    if views == "a_t":
        C = sg.matmul(At.t(), Bd)
    elif views == "b_t":
        C = sg.matmul(Ad, Bt.t())
    elif views == "both_t":
        C = sg.matmul(At.t(), Bt.t())
    else:
        # gemm with trans_a on a column-major view: the view is A^T (K x M),
        # so op of it is A, run as A stored M x K.
        C = sg.gemm(Ad.t(), Bt.t(), trans_a=True)
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)


# Large products whose layout the vector kernels cannot load are run on
# zero-padded aligned copies of A and B (automatic choice only), C written
# in place: odd N, odd K, odd M with A stored K x M, a float-offset pointer,
# odd leading dimensions, beta != 0, and C alone off the vector grid.  Each above the size from which the
# copies pay (2^25 multiply-adds).
REPACK_CASES = {
    # name: (ta, tb, M, N, K, pads (A, B, C), offsets (A, B, C), alpha, beta)
    "odd_n": (0, 0, 1024, 1031, 2049 + 7, (0, 0, 0), (0, 0, 0), 1.0, 0.0),
    "odd_k": (0, 0, 1200, 1280, 1401, (0, 0, 0), (0, 0, 0), 1.0, 0.0),
    "ta_odd_m": (1, 0, 1201, 1024, 1792, (0, 0, 0), (0, 0, 0), 1.0, 0.0),
    "tb_odd_k": (0, 1, 1024, 1152, 1827, (0, 0, 0), (0, 0, 0), -0.5, 0.0),
    "tt_odd_all": (1, 1, 1237, 1113, 1601, (0, 0, 0), (0, 0, 0), 1.0, 0.0),
    "a_offset": (0, 0, 1280, 1280, 1408, (0, 0, 0), (1, 0, 0), 1.0, 0.0),
    "odd_ld_beta": (0, 0, 1280, 1283, 1344, (3, 1, 5), (0, 2, 1), 1.5, -2.0),
    # Only C off the vector grid: nothing copied, C stored one float at a time.
    "c_offset_beta": (0, 0, 1024, 1024, 1024, (0, 0, 0), (0, 0, 1), 1.0, 1.0),
    "tt_c_odd_ld": (1, 1, 1024, 1024, 1024, (0, 0, 3), (0, 0, 0), -1.0, 0.5),
    # A side shorter than the thin kernels leave to the tiled ones: 9 columns
    # (B's rows of 9 floats) and 33 rows.
    "nine_columns": (0, 0, 4096, 9, 4100, (0, 0, 0), (0, 0, 0), 1.0, 0.0),
    "thirty_three_rows_beta": (0, 0, 33, 4097, 4096, (0, 0, 0), (0, 0, 0), 2.0, 1.0),
}


@pytest.mark.parametrize("case", list(REPACK_CASES))
def test_repacked_large_products(dev, case):
    import torch
    ta, tb, M, N, K, pads, offs, alpha, beta = REPACK_CASES[case]
    log(f"case repack {case}: ta={ta} tb={tb} shape=({M},{N},{K}) pads={pads} offs={offs}")
    A, B = workloads.generate(M, N, K, "int4", 91)
    As, Bs = stored(A, ta), stored(B, tb)
    C0 = workloads.generate(M, 1, N, "int4", 92)[0]

    def placed(X, pad, off):
        rows, cols = X.shape
        ld = cols + pad
        buf = torch.full((rows * ld + off + 4,), float("nan"), dtype=torch.float32, device=dev)
        view = torch.as_strided(buf, (rows, cols), (ld, 1), off)
        view.copy_(to_dev(X, dev))
        return buf, view, ld

    _, Av, _ = placed(As, pads[0], offs[0])
    _, Bv, _ = placed(Bs, pads[1], offs[1])
    Cbuf, Cv, ldc = placed(C0, pads[2], offs[2])
    for sched in (sg.SCHED_AUTO, sg.SCHED_STREAMK):
        Cv.copy_(to_dev(C0, dev))
        sg.gemm(Av, Bv, Cv, alpha, beta, ta, tb, sched=sched)
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(As, Bs, C0, alpha, beta, ta, tb)
        assert np.array_equal(Cv.cpu().numpy().astype(np.float64), C_ref), sg.SCHED_NAMES[sched]
        full = torch.as_strided(Cbuf, (M, ldc), (ldc, 1), offs[2]).cpu().numpy()
        assert np.all(np.isnan(full[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("limit", ["0", "-1"], ids=["always_repack", "never_repack"])
def test_repack_threshold_override(dev, limit, monkeypatch):
    """SGEMM_F32_REPACK_MIN_MACS moves the size from which misaligned
    products are repacked: 0 repacks a small odd-shaped product, -1 leaves
    a large one on the general kernel; both give the oracle's result
    (integer inputs: exact)."""
    import torch
    monkeypatch.setenv("SGEMM_F32_REPACK_MIN_MACS", limit)
    M, N, K = (96, 101, 75) if limit == "0" else (700, 643, 901)
    log(f"case repack override {limit}: shape=({M},{N},{K})")
    A, B = workloads.generate(M, N, K, "int4", 93)
    for ta, tb in LAYOUTS:
        As, Bs = stored(A, ta), stored(B, tb)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        sg.gemm(to_dev(As, dev), to_dev(Bs, dev), C, 1.0, 0.0, ta, tb)
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(As, Bs, None, 1.0, 0.0, ta, tb)
        assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref), (ta, tb)


def test_graph_capture_of_a_repacked_call(dev):
    """A repacked call (odd N, beta != 0: A, B and C copied, C copied back)
    captured after an eager call of the same shape replays correctly, with
    new A and C between replays (integer inputs: exact)."""
    import torch
    M, N, K = 640, 517, 768
    log(f"case graph capture repacked shape=({M},{N},{K})")
    s = torch.cuda.Stream(device=dev)
    A0, B = workloads.generate(M, N, K, "int4", 98)
    Ad, Bd = to_dev(A0, dev), to_dev(B, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    with torch.cuda.stream(s):
        sg.gemm(Ad, Bd, C, 1.0, 1.0)                       # eager: repacking buffer ready
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sg.gemm(Ad, Bd, C, 2.0, -1.0)
    torch.cuda.synchronize()
    for r in range(3):
        A_r = workloads.generate(M, N, K, "int4", 210 + r)[0]
        C_r = workloads.generate(M, 1, N, "int4", 220 + r)[0]
        Ad.copy_(to_dev(A_r, dev))
        E = to_dev(C_r, dev)
        sg.gemm(Ad, Bd, E, 2.0, -1.0)                      # eager reference on the device
        C.copy_(to_dev(C_r, dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(A_r, B, C_r, 2.0, -1.0, 0, 0)
        got = C.cpu().numpy()
        assert np.array_equal(got.astype(np.float64), C_ref), f"replay {r}"
        assert np.array_equal(got, E.cpu().numpy()), f"replay {r} vs eager"


# Shapes that take each tile-order and configuration route of the automatic
# choice for narrow or ragged C: (shape, storage orders, expected
# configuration, expected tile-row group).  Integer inputs: exact results.
ROUTE_CASES = {
    "col_order_3_rows_split": ((192, 8192, 2048), (0, 0), "dl_64x64x64", 3),
    "col_order_3_rows_tt": ((192, 8192, 2048), (1, 1), "dl_64x64x64", 3),
    "col_order_5_rows_32deep": ((320, 8192, 384), (0, 0), "dl_64x64x32", 5),
    "row_order_narrow_32deep": ((8192, 320, 512), (0, 0), "dl_64x64x32", 1),
    "row_order_dp_32deep": ((16384, 128, 256), (0, 1), "dl_64x64x32", 1),
    "coverage_picks_128": ((65536, 128, 256), (0, 0), "dl_128x128x32", 1),
    "one_wave_split_whole": ((1024, 1028, 2048), (1, 0), "dl_64x64x64", None),
}


@pytest.mark.parametrize("case", list(ROUTE_CASES))
def test_planner_routes_for_narrow_and_ragged_c(dev, case):
    import torch
    (M, N, K), (ta, tb), cfg_name, group = ROUTE_CASES[case]
    p = sg.plan(M, N, K, num_cus=torch.cuda.get_device_properties(dev).multi_processor_count,
                trans_a=ta, trans_b=tb)
    assert sg.CFG_NAMES[p["config"]] == cfg_name
    if group is not None:
        assert p["group_m"] == group
    log(f"case route {case}: shape=({M},{N},{K}) ta={ta} tb={tb} plan={p}")
    A, B = workloads.generate(M, N, K, "int4", 99)
    As, Bs = stored(A, ta), stored(B, tb)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    sg.gemm(to_dev(As, dev), to_dev(Bs, dev), C, 1.0, 0.0, ta, tb)
    torch.cuda.synchronize()
    C_ref, _ = oracle.gemm_blas(As, Bs, None, 1.0, 0.0, ta, tb)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)


# C with more elements than a 32-bit index reaches (65536 x 32800 = 2.15e9
# floats, 8.6 GB): every route that writes C, checked on whole rows at the
# far end, whole columns and random points (integer inputs: exact).
BIG_C_CASES = {
    # name: (M, N, K, config, beta)
    "dl_edge": (65536, 32800, 32, sg.CFG_AUTO, 0.0),
    "repacked_odd_n": (65536, 32801, 32, sg.CFG_AUTO, 0.0),
    "general_kernel": (65536, 32800, 32, sg.CFG_GENERIC_64x64x16, 0.0),
    "k_zero_scale": (65536, 32800, 0, sg.CFG_AUTO, 2.0),
}


@pytest.mark.parametrize("case", list(BIG_C_CASES))
def test_c_beyond_32bit_element_offsets(dev, case):
    import torch
    M, N, K, config, beta = BIG_C_CASES[case]
    log(f"case big C {case}: shape=({M},{N},{K}) config={sg.CFG_NAMES[config]} beta={beta}")
    assert M * N > 2 ** 31
    A, B = workloads.generate(M, N, K, "int4", 94)
    C = torch.full((M, N), 1.5, dtype=torch.float32, device=dev)
    sg.gemm(to_dev(A, dev), to_dev(B, dev), C, 1.0, beta, config=config)
    torch.cuda.synchronize()
    rng = np.random.default_rng(95)
    full_rows = np.array([0, M - 2, M - 1])
    full_cols = np.array([int(rng.integers(0, N)), N - 1])
    r = np.concatenate([np.repeat(full_rows, N), np.tile(np.arange(M), 2), rng.integers(M // 2, M, 20000)])
    c = np.concatenate([np.tile(np.arange(N), 3), np.repeat(full_cols, M), rng.integers(0, N, 20000)])
    got = C[torch.from_numpy(r).to(dev), torch.from_numpy(c).to(dev)].cpu().numpy().astype(np.float64)
    if K == 0:
        expected = np.full(r.shape, 1.5 * beta)
    else:
        expected, _ = oracle.gemm_points(A, B, r, c)
    assert np.array_equal(got, expected)
    del C
    torch.cuda.empty_cache()


# Products with at most 16 rows: the skinny kernel (vector-ALU FMAs over the
# M rows, B streamed, K split over the grid and the splits added in order).
# (M, N, K, trans_a, A pad / offset, C pad / offset, alpha, beta, schedule)
SKINNY_CASES = {
    "gemv": (1, 4096, 4096, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "m3_ragged": (3, 1028, 777, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "m8_split": (8, 4096, 4096, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "m16_dp": (16, 4096, 300, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_DP),
    "m16_long_k": (16, 260, 65536, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "m5_ta_beta": (5, 2048, 1500, 1, (0, 0), (0, 0), -1.5, 0.5, sg.SCHED_AUTO),
    "m16_odd_lda_ldc": (16, 1024, 1024, 0, (3, 1), (5, 2), 2.0, -1.0, sg.SCHED_STREAMK),
    "m1_ta_offset": (1, 512, 8192, 1, (0, 1), (1, 1), 1.0, 0.0, sg.SCHED_AUTO),
    # 43 strips of 256 columns: 5 K splits, 215 workgroups, one round.
    "m2_uneven_strips": (2, 11008, 4096, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    # 9-16 rows on the matrix cores, through the automatic choice.
    "m12_auto": (12, 2048, 4096, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "m9_ta_beta_split": (9, 3000, 2500, 1, (0, 0), (0, 0), 0.5, -2.0, sg.SCHED_AUTO),
}


@pytest.mark.parametrize("case", list(SKINNY_CASES))
def test_skinny_rows(dev, case):
    import torch
    M, N, K, ta, (apad, aoff), (cpad, coff), alpha, beta, sched = SKINNY_CASES[case]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # Through the automatic choice where it takes the skinny kernel (for
    # 9-16 rows only once B has more than 2^22 elements), else forced.
    auto = sg.plan(M, N, K, sg.CFG_AUTO, sched, num_cus=cus, trans_a=ta)["config"] == sg.CFG_SKINNY_16x256
    config = sg.CFG_AUTO if auto else sg.CFG_SKINNY_16x256
    p = sg.plan(M, N, K, config, sched, num_cus=cus, trans_a=ta)
    assert p["config"] == sg.CFG_SKINNY_16x256
    log(f"case skinny {case}: shape=({M},{N},{K}) ta={ta} A pad/off={apad}/{aoff} C pad/off={cpad}/{coff} "
        f"alpha={alpha} beta={beta} plan={p}")
    A, B = workloads.generate(M, N, K, "int4", 101)
    As = stored(A, ta)
    C0 = workloads.generate(M, 1, N, "int4", 102)[0]

    def placed(X, pad, off):
        rows, cols = X.shape
        ld = cols + pad
        buf = torch.full((rows * ld + off + 4,), float("nan"), dtype=torch.float32, device=dev)
        view = torch.as_strided(buf, (rows, cols), (ld, 1), off)
        view.copy_(to_dev(X, dev))
        return buf, view, ld

    _, Av, _ = placed(As, apad, aoff)
    Cbuf, Cv, ldc = placed(C0, cpad, coff)
    Bd = to_dev(B, dev)
    for rep in range(2):   # the same bits every time
        Cv.copy_(to_dev(C0, dev))
        sg.gemm(Av, Bd, Cv, alpha, beta, ta, 0, config=config, sched=sched)
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(As, B, C0, alpha, beta, ta, 0)
        assert np.array_equal(Cv.cpu().numpy().astype(np.float64), C_ref), f"repeat {rep}"
    full = torch.as_strided(Cbuf, (M, ldc), (ldc, 1), coff).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "ldc padding was written"


def test_skinny_rows_full_size_sampled(dev):
    """16 x 8192 x 16384 (B: 512 MiB) on the skinny kernel, every output
    against the oracle (integer inputs: |partial sums| <= 16 K = 2^18, exact
    in FP32)."""
    import torch
    M, N, K = 16, 8192, 16384
    log(f"case skinny full size ({M},{N},{K})")
    A, B = workloads.generate(M, N, K, "int4", 103)
    C = gpu_matmul(A, B, dev, sg.CFG_SKINNY_16x256)
    C_ref, _ = oracle.gemm(A, B)
    assert np.array_equal(C.astype(np.float64), C_ref)


# Products with at most 8 columns: the row-dot kernel (per-row dot products
# streaming A, B held in LDS, K split over the grid and the splits added in
# order).  (M, N, K, trans_b, A pad, B pad / offset, C pad / offset, alpha,
# beta, schedule); A's padding keeps its rows on 16-byte boundaries.
ROWDOT_CASES = {
    "gemv": (16384, 1, 4096, 0, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "n2_k_tail": (3000, 2, 1021, 0, 3, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "n3_tb_beta": (1000, 3, 5000, 1, 0, (0, 0), (0, 0), -0.5, 2.0, sg.SCHED_AUTO),
    "n5_split_many": (256, 5, 65536, 0, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
    "n8_dp": (4099, 8, 2044, 0, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_DP),
    "n8_streamk_odd_ld": (2500, 8, 3000, 1, 4, (3, 1), (5, 2), 2.0, -1.0, sg.SCHED_STREAMK),
    "n1_b_offset": (777, 1, 9999, 0, 1, (0, 1), (1, 1), 1.0, 0.0, sg.SCHED_AUTO),
    # 375 row blocks and no K split: one round of resident workgroups.
    "n1_one_round": (3000, 1, 4096, 0, 0, (0, 0), (0, 0), 1.0, 0.0, sg.SCHED_AUTO),
}


@pytest.mark.parametrize("case", list(ROWDOT_CASES))
def test_rowdot_columns(dev, case):
    import torch
    M, N, K, tb, apad, (bpad, boff), (cpad, coff), alpha, beta, sched = ROWDOT_CASES[case]
    assert (K + apad) % 4 == 0
    # The plan query assumes dense operands: shown for the cases that are.
    p = sg.plan(M, N, K, sg.CFG_ROWDOT_N8, sched, trans_b=tb) if apad == 0 else "padded A"
    log(f"case rowdot {case}: shape=({M},{N},{K}) tb={tb} A pad={apad} B pad/off={bpad}/{boff} "
        f"C pad/off={cpad}/{coff} alpha={alpha} beta={beta} plan={p}")
    A, B = workloads.generate(M, N, K, "int4", 104)
    Bs = stored(B, tb)
    C0 = workloads.generate(M, 1, N, "int4", 105)[0]

    def placed(X, pad, off):
        rows, cols = X.shape
        ld = cols + pad
        buf = torch.full((rows * ld + off + 4,), float("nan"), dtype=torch.float32, device=dev)
        view = torch.as_strided(buf, (rows, cols), (ld, 1), off)
        view.copy_(to_dev(X, dev))
        return buf, view, ld

    _, Av, _ = placed(A, apad, 0)
    _, Bv, _ = placed(Bs, bpad, boff)
    Cbuf, Cv, ldc = placed(C0, cpad, coff)
    for rep in range(2):   # the same bits every time
        Cv.copy_(to_dev(C0, dev))
        sg.gemm(Av, Bv, Cv, alpha, beta, 0, tb, config=sg.CFG_ROWDOT_N8, sched=sched)
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(A, Bs, C0, alpha, beta, 0, tb)
        assert np.array_equal(Cv.cpu().numpy().astype(np.float64), C_ref), f"repeat {rep}"
    full = torch.as_strided(Cbuf, (M, ldc), (ldc, 1), coff).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("shape", [(16384, 1, 16384), (32768, 2, 4096), (65536, 4, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_rowdot_is_the_automatic_choice(dev, shape):
    """Where the automatic choice runs the row-dot kernel, it matches the
    oracle exactly (integer inputs, K <= 16384)."""
    import torch
    M, N, K = shape
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    assert sg.plan(M, N, K, num_cus=cus)["config"] == sg.CFG_ROWDOT_N8
    log(f"case rowdot auto {shape}")
    A, B = workloads.generate(M, N, K, "int4", 106)
    C = gpu_matmul(A, B, dev)
    C_ref, _ = oracle.gemm(A, B)
    assert np.array_equal(C.astype(np.float64), C_ref)


@pytest.mark.parametrize("shape", [(4, 4096, 4096), (8192, 8, 8192)], ids=["skinny", "rowdot"])
def test_graph_capture_of_thin_products(dev, shape):
    """The skinny and row-dot kernels with K split (partials in the stream's
    workspace, a second kernel adding them) captured after an eager call of
    the same shape: every replay, with new A and eager work in between,
    matches the oracle and the eager result exactly (integer inputs)."""
    import torch
    M, N, K = shape
    p = sg.plan(M, N, K, num_cus=torch.cuda.get_device_properties(dev).multi_processor_count)
    assert p["config"] in (sg.CFG_SKINNY_16x256, sg.CFG_ROWDOT_N8) and p["sk_tiles"] > 0
    log(f"case graph capture thin {shape} plan={p}")
    s = torch.cuda.Stream(device=dev)
    A0, B = workloads.generate(M, N, K, "int4", 107)
    Ad, Bd = to_dev(A0, dev), to_dev(B, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    with torch.cuda.stream(s):
        sg.gemm(Ad, Bd, C)                                  # eager: workspace ready
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sg.gemm(Ad, Bd, C)
    torch.cuda.synchronize()
    for r in range(3):
        A_r = workloads.generate(M, N, K, "int4", 230 + r)[0]
        Ad.copy_(to_dev(A_r, dev))
        E = sg.matmul(Ad, Bd)                               # eager reference on the device
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm(A_r, B)
        got = C.cpu().numpy()
        assert np.array_equal(got.astype(np.float64), C_ref), f"replay {r}"
        assert np.array_equal(got, E.cpu().numpy()), f"replay {r} vs eager"


# The thin-product kernels with their streamed operand off the 16-byte grid
# (4-byte loads): skinny with B at a float offset / odd ldb / odd N, row-dot
# with A at a float offset / odd lda.  (M, N, K, streamed pad, streamed
# offset, beta, expected configuration); integer inputs, exact.
THIN_MISALIGNED = {
    "skinny_odd_n_offset": (4, 4097, 2000, 0, 1, 0.0, sg.CFG_SKINNY_16x256),
    "skinny_odd_ldb": (7, 1030, 3001, 3, 0, 1.0, sg.CFG_SKINNY_16x256),
    "skinny_16_rows_odd_n": (16, 4097, 1500, 0, 0, 0.0, sg.CFG_SKINNY_16x256),
    "rowdot_odd_k": (5000, 1, 4097, 0, 0, 0.0, sg.CFG_ROWDOT_N8),
    "rowdot_offset_n3": (3000, 3, 2500, 1, 2, -1.0, sg.CFG_ROWDOT_N8),
}


@pytest.mark.parametrize("case", list(THIN_MISALIGNED))
def test_thin_kernels_with_unaligned_streamed_operand(dev, case):
    import torch
    M, N, K, pad, off, beta, cfg = THIN_MISALIGNED[case]
    skinny = cfg == sg.CFG_SKINNY_16x256
    log(f"case thin unaligned {case}: shape=({M},{N},{K}) pad={pad} off={off} beta={beta}")
    A, B = workloads.generate(M, N, K, "int4", 108)
    C0 = workloads.generate(M, 1, N, "int4", 109)[0]

    def placed(X, pad, off):
        rows, cols = X.shape
        ld = cols + pad
        buf = torch.full((rows * ld + off + 4,), float("nan"), dtype=torch.float32, device=dev)
        view = torch.as_strided(buf, (rows, cols), (ld, 1), off)
        view.copy_(to_dev(X, dev))
        return view

    Av = to_dev(A, dev) if skinny else placed(A, pad, off)
    Bv = placed(B, pad, off) if skinny else to_dev(B, dev)
    C = to_dev(C0, dev)
    sg.gemm(Av, Bv, C, 1.0, beta)
    torch.cuda.synchronize()
    C_ref, _ = oracle.gemm_blas(A, B, C0, 1.0, beta)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), C_ref)
    # The plan query (dense operands) picks the same kernel for this shape.
    assert sg.plan(M, N, K)["config"] == cfg


# Few rows with B stored N x K (x W^T with W row-major): the product runs
# transposed, C^T = B A^T, on the row-dot kernel, C written transposed.
# (M, N, K, trans_a, C pad / offset, alpha, beta)
TRANSPOSED_THIN = {
    "gemv_wt": (1, 16384, 4096, 0, (0, 0), 1.0, 0.0),
    "m2_ta_beta": (2, 300, 300, 1, (0, 0), 1.5, -0.5),
    "m5_odd_k_padded_c": (5, 1000, 777, 0, (3, 1), 2.0, 1.0),
    "m8_split": (8, 16384, 8192, 0, (0, 0), 1.0, 0.0),
    "m3_long_k_ta": (3, 4097, 20000, 1, (1, 2), -1.0, 0.25),
}


@pytest.mark.parametrize("case", list(TRANSPOSED_THIN))
def test_few_rows_with_b_stored_n_by_k_run_transposed(dev, case):
    import torch
    M, N, K, ta, (cpad, coff), alpha, beta = TRANSPOSED_THIN[case]
    log(f"case transposed thin {case}: shape=({M},{N},{K}) ta={ta} C pad/off={cpad}/{coff} alpha={alpha} beta={beta}")
    A, B = workloads.generate(M, N, K, "int4", 111)
    C0 = workloads.generate(M, 1, N, "int4", 112)[0]
    As = stored(A, ta)
    Bs = np.ascontiguousarray(B.T)   # B stored N x K
    ldc = N + cpad
    buf = torch.full((M * ldc + coff + 4,), float("nan"), dtype=torch.float32, device=dev)
    Cv = torch.as_strided(buf, (M, N), (ldc, 1), coff)
    Cv.copy_(to_dev(C0, dev))
    sg.gemm(to_dev(As, dev), to_dev(Bs, dev), Cv, alpha, beta, ta, 1)
    torch.cuda.synchronize()
    C_ref, _ = oracle.gemm_blas(As, Bs, C0, alpha, beta, ta, 1)
    assert np.array_equal(Cv.cpu().numpy().astype(np.float64), C_ref)
    full = torch.as_strided(buf, (M, ldc), (ldc, 1), coff).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "ldc padding was written"
    # The plan query (dense operands) reports the transposed product where
    # the layout is dense and vector-aligned or M <= 2 or B is large.
    p = sg.plan(M, N, K, trans_a=ta, trans_b=1)
    if p["transposed"]:
        assert p["config"] == sg.CFG_ROWDOT_N8


# Few columns with A stored K x M (X^T v with X row-major): the product runs
# transposed, C^T = op(B)^T A_stored, on the skinny kernel, C written
# transposed.  (M, N, K, trans_b, C pad / offset, alpha, beta)
TRANSPOSED_FEW_COLUMNS = {
    "xt_v": (16384, 1, 4096, 0, (0, 0), 1.0, 0.0),
    "n8_tb_beta": (3000, 8, 2500, 1, (0, 0), 1.5, -0.5),
    "n12_split_padded_c": (4096, 12, 8192, 0, (2, 1), 2.0, 1.0),
    "n16_odd_m": (4099, 16, 3000, 0, (0, 0), 1.0, 0.0),
    "n3_small_tb": (1000, 3, 1000, 1, (1, 1), -1.0, 0.5),
}


@pytest.mark.parametrize("case", list(TRANSPOSED_FEW_COLUMNS))
def test_few_columns_with_a_stored_k_by_m_run_transposed(dev, case):
    import torch
    M, N, K, tb, (cpad, coff), alpha, beta = TRANSPOSED_FEW_COLUMNS[case]
    log(f"case transposed few columns {case}: shape=({M},{N},{K}) tb={tb} C pad/off={cpad}/{coff} "
        f"alpha={alpha} beta={beta}")
    A, B = workloads.generate(M, N, K, "int4", 113)
    C0 = workloads.generate(M, 1, N, "int4", 114)[0]
    As = stored(A, 1)   # A stored K x M
    Bs = stored(B, tb)
    ldc = N + cpad
    buf = torch.full((M * ldc + coff + 4,), float("nan"), dtype=torch.float32, device=dev)
    Cv = torch.as_strided(buf, (M, N), (ldc, 1), coff)
    Cv.copy_(to_dev(C0, dev))
    sg.gemm(to_dev(As, dev), to_dev(Bs, dev), Cv, alpha, beta, 1, tb)
    torch.cuda.synchronize()
    C_ref, _ = oracle.gemm_blas(As, Bs, C0, alpha, beta, 1, tb)
    assert np.array_equal(Cv.cpu().numpy().astype(np.float64), C_ref)
    full = torch.as_strided(buf, (M, ldc), (ldc, 1), coff).cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "ldc padding was written"
    p = sg.plan(M, N, K, trans_a=1, trans_b=tb)
    assert p["transposed"] == 1 and p["config"] == sg.CFG_SKINNY_16x256


@pytest.mark.parametrize("case", ["x_wt", "xt_v"])
def test_graph_capture_of_transposed_thin_products(dev, case):
    """The transposed routes (x W^T on the row-dot kernel, X^T v on the
    skinny kernel, both with K split) captured after an eager call: every
    replay, with a new small operand and eager work in between, matches the
    oracle and the eager result exactly (integer inputs)."""
    import torch
    if case == "x_wt":
        M, N, K, ta, tb = 2, 4096, 16384, 0, 1       # A: x (2 x K), B stored N x K
    else:
        M, N, K, ta, tb = 4096, 4, 16384, 1, 0       # A stored K x M, B: v (K x 4)
    p = sg.plan(M, N, K, num_cus=torch.cuda.get_device_properties(dev).multi_processor_count,
                trans_a=ta, trans_b=tb)
    assert p["transposed"] == 1 and p["sk_tiles"] > 0
    log(f"case graph capture transposed thin {case} ({M},{N},{K}) ta={ta} tb={tb} plan={p}")
    s = torch.cuda.Stream(device=dev)
    A0, B0 = workloads.generate(M, N, K, "int4", 115)
    As, Bs = stored(A0, ta), stored(B0, tb)
    Ad, Bd = to_dev(As, dev), to_dev(Bs, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    with torch.cuda.stream(s):
        sg.gemm(Ad, Bd, C, 1.0, 0.0, ta, tb)                # eager: workspace ready
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        sg.gemm(Ad, Bd, C, 1.0, 0.0, ta, tb)
    torch.cuda.synchronize()
    small_is_a = case == "x_wt"
    for r in range(3):
        X = workloads.generate(M, N, K, "int4", 240 + r)[0 if small_is_a else 1]
        if small_is_a:
            As = stored(X, ta); Ad.copy_(to_dev(As, dev))
        else:
            Bs = stored(X, tb); Bd.copy_(to_dev(Bs, dev))
        E = torch.empty_like(C)
        sg.gemm(Ad, Bd, E, 1.0, 0.0, ta, tb)                # eager reference on the device
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C_ref, _ = oracle.gemm_blas(As, Bs, np.zeros((M, N), np.float32), 1.0, 0.0, ta, tb)
        got = C.cpu().numpy()
        assert np.array_equal(got.astype(np.float64), C_ref), f"replay {r}"
        assert np.array_equal(got, E.cpu().numpy()), f"replay {r} vs eager"
