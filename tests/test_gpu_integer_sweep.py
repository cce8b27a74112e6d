"""GPU: a seeded sweep of random products through sgemm_f32_gemm on integer
inputs in {-4..4}.  It covers random shapes (any side, or multiples of 4, 16
or 64), both storage orders of each operand, alpha and beta, and forced
configurations and schedules next to the automatic choice.

With such inputs every product is an integer of magnitude at most 16, and
every partial sum at most 16 K.  With alpha in {1, 2, -1}, beta in {0, 1, -2}
and K below 2^19, every value formed (partial sums, alpha times the sum, plus
beta C) is an integer below 2^24, exact in FP32 whatever the order of the
additions.  The result must then equal the exact product, which float64
matmul on the same device gives (its partial sums are integers far below
2^53).  A forced configuration that cannot run a shape or layout is refused
with SGEMM_ERR_CONFIG before anything is enqueued; such draws are skipped."""
import math

import numpy as np
import pytest

import fp32_sgemm_f32_amd as sg

FORCED = [sg.CFG_DL_256x256x16, sg.CFG_DL_128x128x32, sg.CFG_DL_64x64x64, sg.CFG_DL_64x64x32,
          sg.CFG_DL_64x64x64_K2, sg.CFG_DL_64x64x32_K2, sg.CFG_DL_128x128x32_K2, sg.CFG_DL_128x256x16,
          sg.CFG_DL_256x128x16, sg.CFG_MFMA_256x256x16, sg.CFG_MFMA_128x128x32, sg.CFG_MFMA_64x64x64,
          sg.CFG_MFMA_128x128x64, sg.CFG_VALU_128x128x8, sg.CFG_VALU_256x128x8, sg.CFG_GENERIC_64x64x16]

# (seed, draws, smallest and largest side, most multiply-adds per product)
SWEEPS = {
    "small": (7, 3000, 1, 4096, 4e9),
    "large": (11, 600, 128, 8192, 2e10),
}


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    sg.library()
    return torch.device("cuda:0")


def draws(seed, count, lo, hi, max_macs):
    """The sweep's cases, in order (host only)."""
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
        ta, tb = bool(rng.integers(2)), bool(rng.integers(2))
        cfg = sg.CFG_AUTO if rng.random() < 0.4 else int(rng.choice(FORCED))
        sched = int(rng.choice([sg.SCHED_AUTO, sg.SCHED_DP, sg.SCHED_STREAMK]))
        alpha = float(rng.choice([1.0, 2.0, -1.0]))
        beta = float(rng.choice([0.0, 0.0, 1.0, -2.0]))
        out.append((M, N, K, ta, tb, cfg, sched, alpha, beta, int(rng.integers(2 ** 31))))
    return out


def test_sweep_draws_are_exact_in_fp32():
    """Host check of the premise: every draw keeps its values below 2^24."""
    for name, (seed, count, lo, hi, max_macs) in SWEEPS.items():
        for M, N, K, *_ in draws(seed, count, lo, hi, max_macs):
            assert 2 * 16 * K + 2 * 4 < 2 ** 24, (name, M, N, K)


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(SWEEPS))
def test_integer_sweep_is_exact(dev, name):
    import torch
    seed, count, lo, hi, max_macs = SWEEPS[name]
    ran = 0
    for i, (M, N, K, ta, tb, cfg, sched, alpha, beta, s) in enumerate(draws(seed, count, lo, hi, max_macs)):
        g = np.random.default_rng(s)
        A = g.integers(-4, 5, size=(K, M) if ta else (M, K)).astype(np.float32)
        B = g.integers(-4, 5, size=(N, K) if tb else (K, N)).astype(np.float32)
        C0 = g.integers(-4, 5, size=(M, N)).astype(np.float32)
        label = (f"sweep {name} #{i}: ({M},{N},{K}) ta={int(ta)} tb={int(tb)} "
                 f"config={sg.CFG_NAMES.get(cfg, cfg)} sched={sg.SCHED_NAMES[sched]} alpha={alpha} beta={beta}")
        Ad, Bd, C0d = (torch.from_numpy(x).to(dev) for x in (A, B, C0))
        C = C0d.clone()
        log(label)
        try:
            sg.gemm(Ad, Bd, C, alpha=alpha, beta=beta, trans_a=ta, trans_b=tb, config=cfg, sched=sched)
        except sg.SgemmError as e:
            assert e.status == sg.ERR_CONFIG and cfg != sg.CFG_AUTO, (label, e)
            continue
        opA = Ad.t() if ta else Ad
        opB = Bd.t() if tb else Bd
        ref = alpha * (opA.double() @ opB.double()) + beta * C0d.double()
        torch.cuda.synchronize()
        wrong = int((C.double() != ref).sum())
        assert wrong == 0, f"{label}: {wrong} elements differ from the exact product"
        ran += 1
    log(f"sweep {name}: {ran} of {count} draws ran, all exact")
    assert ran >= count // 3
