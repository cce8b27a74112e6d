"""The no-allocation entry point, sgemm_f32_gemm_noalloc, through the C-ABI:
its results against sgemm_f32_gemm's on the same inputs.

It runs the same kernels as sgemm_f32_gemm with the Stream-K partial tiles
and the repacked copies taken from the library's fixed per-device scratch
array.  Where that holds them the plan is the same, so the results are the
same bit for bit; a split schedule too large for it runs data-parallel
(compared on integer inputs: exact either way); repacked copies too large
for it are refused with SGEMM_ERR_SCRATCH and C is left untouched.  Each
case makes two calls in a row, the second with a smaller input, so that the
second reuses the array the first left behind.
"""
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


def stored(X, trans):
    return np.ascontiguousarray(X.T) if trans else X


def run_both(dev, ta, tb, M, N, K, alpha, beta, dist, seed, c_pad=0):
    """C from sgemm_f32_gemm and from sgemm_f32_gemm_noalloc on the same
    operands (C0 the same start for both), plus the host copies."""
    import torch
    A, B = workloads.generate(M, N, K, dist, seed)
    As, Bs = stored(A, ta), stored(B, tb)
    C0 = workloads.generate(M, 1, N, dist, seed + 1)[0]
    Ad = torch.from_numpy(np.ascontiguousarray(As)).to(dev)
    Bd = torch.from_numpy(np.ascontiguousarray(Bs)).to(dev)
    ldc = N + c_pad
    outs = []
    for fn in (sg.gemm_raw, sg.gemm_noalloc_raw):
        Cbuf = torch.full((M, ldc), float("nan"), dtype=torch.float32, device=dev)
        Cbuf[:, :N] = torch.from_numpy(C0).to(dev)
        s = torch.cuda.current_stream(dev)
        st = fn(ta, tb, M, N, K, alpha, Ad.data_ptr(), As.shape[1], Bd.data_ptr(), Bs.shape[1], beta,
                Cbuf.data_ptr(), ldc, s.cuda_stream)
        assert st == sg.OK, (fn.__name__, st, sg.status_string(st))
        outs.append(Cbuf)
    torch.cuda.synchronize()
    ref, noalloc = (c.cpu().numpy() for c in outs)
    assert np.all(np.isnan(noalloc[:, N:])), "ldc padding was written"
    return As, Bs, C0, ref[:, :N], noalloc[:, :N]


# (name, [first call, second smaller call]); each call
# (ta, tb, M, N, K, alpha, beta, dist).
CASES = {
    # Stream-K partials in the scratch array (64x64 tiles, split remainder).
    "streamk": [(0, 0, 1000, 1028, 2048, 1.0, 0.0, "uniform"), (520, 516, 1500, 1.0, 0.0, "uniform")],
    # Repacked copies (odd N / odd K) and the split partials behind them.
    "repacked": [(0, 0, 1031, 1027, 1409, 1.0, 0.0, "uniform"), (0, 1, 515, 771, 1021, -0.5, 2.0, "normal")],
    # Whole tiles: no scratch at all; storage orders and beta.
    "whole_tiles": [(1, 1, 2048, 2048, 1024, 1.5, -1.0, "normal"), (1, 0, 1024, 1024, 512, 1.0, 0.0, "uniform")],
    # Thin products on the skinny and row-dot kernels with their K splits.
    "thin": [(0, 0, 8, 8192, 8192, 1.0, 0.0, "uniform"), (4096, 1, 4096, 1.0, 0.0, "uniform")],
}


def unpack(call):
    if len(call) == 6:   # (M, N, K, alpha, beta, dist) after a first call: same storage order
        return (0, 0) + tuple(call)
    return call


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_gemm(dev, case):
    for i, call in enumerate(CASES[case]):
        ta, tb, M, N, K, alpha, beta, dist = unpack(call)
        p = sg.plan(M, N, K, trans_a=ta, trans_b=tb)
        log(f"case noalloc {case} call {i}: ta={ta} tb={tb} shape=({M},{N},{K}) alpha={alpha} beta={beta} "
            f"config={sg.CFG_NAMES[p['config']]} sched={sg.SCHED_NAMES[p['sched']]} "
            f"workspace={p['workspace_bytes']} repacked={p['repacked']}")
        # C's rows padded by 4 floats (kept on the 16-byte grid), or by 3 in
        # one call (C stored a float at a time, through the repacking path
        # with nothing to copy).
        c_pad = 3 if (case, i) == ("whole_tiles", 0) else 4
        As, Bs, C0, ref, noalloc = run_both(dev, ta, tb, M, N, K, alpha, beta, dist, 300 + 10 * i, c_pad=c_pad)
        C_ref, S = oracle.gemm_blas(As, Bs, C0, alpha, beta, ta, tb)
        ok, worst = oracle.within_bound(noalloc, C_ref, S, TOL)
        log(f"  max|err|/S = {worst:.3e}")
        assert ok
        # Same plan, same kernels: the same bits as the allocating call.
        assert np.array_equal(ref.view(np.uint32), noalloc.view(np.uint32))


def test_noalloc_split_too_large_runs_whole_tiles(dev):
    """256x256 tiles with a split remainder need 128 MiB of partial tiles,
    beyond the 64 MiB array: the no-allocation call runs whole tiles
    (integer inputs, so both schedules give the exact product), then a
    smaller split call that fits reuses the array."""
    M, N, K = 4096, 4608, 1024
    p = sg.plan(M, N, K)
    assert p["sched"] == sg.SCHED_STREAMK and p["workspace_bytes"] > sg.NOALLOC_SCRATCH_BYTES
    for i, (m, n, k) in enumerate([(M, N, K), (1000, 1028, 1024)]):
        log(f"case noalloc split beyond the array, call {i}: shape=({m},{n},{k})")
        As, Bs, _, ref, noalloc = run_both(dev, 0, 0, m, n, k, 1.0, 0.0, "int4", 400 + i)
        exact, _ = oracle.gemm(As, Bs)
        assert np.array_equal(noalloc.astype(np.float64), exact)
        assert np.array_equal(ref.astype(np.float64), exact)


def test_noalloc_refuses_copies_beyond_the_array(dev):
    """A repacked product whose copies exceed the array: SGEMM_ERR_SCRATCH
    before anything is enqueued (C untouched); a smaller repacked call after
    it runs."""
    import torch
    M, N, K = 4099, 4097, 4096   # B's copy alone is 64 MiB + a row
    A, B = workloads.generate(M, N, K, "int4", 500)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    C = torch.full((M, N), 7.0, dtype=torch.float32, device=dev)
    log(f"case noalloc refuses copies: shape=({M},{N},{K})")
    st = sg.gemm_noalloc_raw(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0, C.data_ptr(), N,
                             torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert st == sg.ERR_SCRATCH
    assert bool((C == 7.0).all().item())
    del Ad, Bd, C
    As, Bs, _, ref, noalloc = run_both(dev, 0, 0, 515, 771, 1021, 1.0, 0.0, "int4", 501)
    exact, _ = oracle.gemm(As, Bs)
    assert np.array_equal(noalloc.astype(np.float64), exact)


# Seeded sweep: (seed, draws, smallest and largest side, most multiply-adds).
NOALLOC_SWEEPS = {"small": (21, 400, 1, 4096, 4e9), "large": (23, 150, 128, 8192, 2e10)}


def noalloc_draws(seed, count, lo, hi, max_macs):
    """Random products (host only): shape (any side, or multiples of 4, 16 or
    64), storage orders, a padded ldc now and then, alpha and beta."""
    import math
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        def side():
            v = int(math.exp(rng.uniform(math.log(lo), math.log(hi))))
            q = int(rng.choice([1, 4, 16, 64]))
            return max(1, v // q * q)
        M, N, K = side(), side(), side()
        if M * N * K > max_macs:
            continue
        out.append((M, N, K, int(rng.integers(2)), int(rng.integers(2)), int(rng.choice([0, 0, 3, 8])),
                    float(rng.choice([1.0, 2.0, -1.0])), float(rng.choice([0.0, 0.0, 1.0, -2.0])),
                    int(rng.integers(2 ** 31))))
    return out


@pytest.mark.parametrize("name", list(NOALLOC_SWEEPS))
def test_noalloc_integer_sweep(dev, name):
    """Random products through sgemm_f32_gemm_noalloc on integer inputs in
    {-4..4}: every partial sum is an integer below 2^24 (K < 2^19), so the
    result must equal the exact product (float64 matmul on the device) bit
    for bit, whatever plan the call ran.  A call whose repacked copies exceed
    the scratch array must be refused with SGEMM_ERR_SCRATCH and leave C as
    it was."""
    import torch
    seed, count, lo, hi, max_macs = NOALLOC_SWEEPS[name]
    ran = refused = 0
    for i, (M, N, K, ta, tb, pad, alpha, beta, s) in enumerate(noalloc_draws(seed, count, lo, hi, max_macs)):
        assert 2 * 16 * K + 8 < 2 ** 24
        g = np.random.default_rng(s)
        As = g.integers(-4, 5, size=(K, M) if ta else (M, K)).astype(np.float32)
        Bs = g.integers(-4, 5, size=(N, K) if tb else (K, N)).astype(np.float32)
        C0 = g.integers(-4, 5, size=(M, N)).astype(np.float32)
        log(f"noalloc sweep {name} #{i}: ({M},{N},{K}) ta={ta} tb={tb} ldc={N + pad} alpha={alpha} beta={beta}")
        Ad, Bd = torch.from_numpy(As).to(dev), torch.from_numpy(Bs).to(dev)
        Cbuf = torch.full((M, N + pad), float("nan"), dtype=torch.float32, device=dev)
        Cbuf[:, :N] = torch.from_numpy(C0).to(dev)
        st = sg.gemm_noalloc_raw(ta, tb, M, N, K, alpha, Ad.data_ptr(), As.shape[1], Bd.data_ptr(), Bs.shape[1],
                                 beta, Cbuf.data_ptr(), N + pad, torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize()
        C = Cbuf.cpu().numpy()
        assert np.all(np.isnan(C[:, N:])), "ldc padding was written"
        if st == sg.ERR_SCRATCH:
            assert np.array_equal(C[:, :N], C0), "a refused call wrote C"
            refused += 1
            continue
        assert st == sg.OK, (st, sg.status_string(st))
        opA = Ad.t() if ta else Ad
        opB = Bd.t() if tb else Bd
        ref = (alpha * (opA.double() @ opB.double()) + beta * torch.from_numpy(C0).to(dev).double()).cpu().numpy()
        wrong = int(np.sum(C[:, :N].astype(np.float64) != ref))
        assert wrong == 0, f"#{i}: {wrong} elements differ from the exact product"
        ran += 1
    log(f"noalloc sweep {name}: {ran} ran, {refused} refused (scratch), all exact")
    assert ran >= count // 2


def test_noalloc_calls_from_two_threads_on_one_stream(dev):
    """Two host threads make no-allocation calls on ONE stream with no host
    synchronisation: repacked products (copies in the shared scratch array)
    and split ones (partials there).  Each call's copies, product and sum
    must run back to back on the stream, or another thread's copies or
    partials would land in between.  Integer inputs: every result exact."""
    import threading
    import torch
    log("case noalloc, two threads, one stream")
    shapes = [(515, 771, 1021), (1000, 1028, 1024)]
    assert sg.plan(*shapes[0])["repacked"] == 1 and sg.plan(*shapes[1])["sched"] == sg.SCHED_STREAMK
    s = torch.cuda.Stream(device=dev)
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = workloads.generate(M, N, K, "int4", 600 + i)
        outs = [torch.full((M, N), float("nan"), dtype=torch.float32, device=dev) for _ in range(10)]
        data.append((M, N, K, A, B, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev), outs))
    torch.cuda.synchronize()
    errors = []
    go = threading.Barrier(2)

    def worker(i):
        try:
            M, N, K, _, _, Ad, Bd, outs = data[i]
            go.wait()
            for C in outs:
                st = sg.gemm_noalloc_raw(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0, C.data_ptr(),
                                         N, s.cuda_stream)
                assert st == sg.OK, st
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for _, _, _, A, B, _, _, outs in data:
        exact, _ = oracle.gemm(A, B)
        for C in outs:
            assert np.array_equal(C.cpu().numpy().astype(np.float64), exact)


def test_noalloc_graph_capture_and_replay(dev):
    """A no-allocation split call (partials in the scratch array) captured
    into a HIP graph replays correctly, with new A written and eager work
    (an allocating call of another shape) run between the replays; every
    replay matches the oracle and the eager result exactly (integer
    inputs).  Nothing has to be sized by an eager call of the same shape
    first."""
    import torch
    M, N, K = 1000, 1028, 1024
    assert sg.plan(M, N, K)["sched"] == sg.SCHED_STREAMK
    log(f"case noalloc graph capture shape=({M},{N},{K})")
    s = torch.cuda.Stream(device=dev)
    A0, B = workloads.generate(M, N, K, "int4", 610)
    Ad, Bd = torch.from_numpy(A0).to(dev), torch.from_numpy(B).to(dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    # An eager call of another, smaller shape (nothing about this shape is prepared).
    small = torch.empty((64, 64), dtype=torch.float32, device=dev)
    assert sg.gemm_noalloc_raw(0, 0, 64, 64, 64, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0, small.data_ptr(), 64,
                               s.cuda_stream) == sg.OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st = sg.gemm_noalloc_raw(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0, C.data_ptr(), N,
                                 s.cuda_stream)
    assert st == sg.OK
    torch.cuda.synchronize()
    for r in range(3):
        A_r = workloads.generate(M, N, K, "int4", 620 + r)[0]
        Ad.copy_(torch.from_numpy(A_r).to(dev))
        E = sg.matmul(Ad, Bd)                     # eager, allocating entry point
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        exact, _ = oracle.gemm(A_r, B)
        got = C.cpu().numpy()
        assert np.array_equal(got.astype(np.float64), exact), f"replay {r}"
        assert np.array_equal(got, E.cpu().numpy()), f"replay {r} vs eager"
