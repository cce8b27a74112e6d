"""Timing sweep behind the planner's cost model (one GPU).

For seeded random dense row-major shapes, sides log-uniform, it times the
automatic choice and each of the four direct-to-LDS configurations
(256x256x16, 128x128x32, 64x64x64, 64x64x32) under the data-parallel, the
Stream-K (every tile split) and the automatic schedule, back to back: 0.1 s
of untimed calls, then the median of 15 calls each bracketed by its own HIP
event pair.  One CSV row per (shape, candidate), with the plan it ran.

    python -m fp32_sgemm_f32_amd.tuning.sweep_plans SEED COUNT [MAX_MACS] [MIN_MACS] > rows.csv

plan_sweeps.csv holds four such sweeps (seeds 21 and 22 with the default
bounds, 31 with MAX_MACS 3e11, and 41 with MAX_MACS 3e11 and MIN_MACS 5e10 on
sides up to 16384), labelled a-d.  fit_cost_model.py fits the model to them.
"""
import csv
import math
import statistics
import sys
import time

import numpy as np

import fp32_sgemm_f32_amd as sg

CONFIGS = [sg.CFG_DL_256x256x16, sg.CFG_DL_128x128x32, sg.CFG_DL_64x64x64, sg.CFG_DL_64x64x32]
SCHEDS = [sg.SCHED_DP, sg.SCHED_STREAMK, sg.SCHED_AUTO]
FIELDS = ["sweep", "M", "N", "K", "req_config", "req_sched", "config", "sched", "dp_tiles", "sk_tiles",
          "grid", "sk_grid", "ipt", "us"]


def shapes(seed, count, max_macs, min_macs, max_side):
    rng = np.random.default_rng(seed)

    def logu(lo, hi, q):
        return max(q, int(round(math.exp(rng.uniform(math.log(lo), math.log(hi))) / q)) * q)
    done = 0
    while done < count:
        M, N, K = logu(64, max_side, 16), logu(64, max_side, 16), logu(64, 16384, 16)
        if min_macs <= M * N * K <= max_macs:
            done += 1
            yield M, N, K


def main(argv):
    import torch
    seed, count = int(argv[1]), int(argv[2])
    max_macs = float(argv[3]) if len(argv) > 3 else 4e10
    min_macs = float(argv[4]) if len(argv) > 4 else 2e7
    max_side = 16384 if len(argv) > 4 else 8192
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    out = csv.writer(sys.stdout)
    out.writerow(FIELDS)

    def timed(fn, n):
        st = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        en = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for i in range(n):
            st[i].record(stream)
            fn()
            en[i].record(stream)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) * 1e3 for a, b in zip(st, en))

    with torch.cuda.stream(stream):
        for M, N, K in shapes(seed, count, max_macs, min_macs, max_side):
            A = torch.rand((M, K), device=dev) * 2 - 1
            B = torch.rand((K, N), device=dev) * 2 - 1
            C = torch.empty((M, N), device=dev)
            for cfg, sched in [(sg.CFG_AUTO, sg.SCHED_AUTO)] + [(c, s) for c in CONFIGS for s in SCHEDS]:
                def call():
                    st = sg.sgemm_raw(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                                      stream.cuda_stream, cfg, sched)
                    if st != 0:
                        raise sg.SgemmError(st)
                try:
                    call()
                except sg.SgemmError:
                    continue
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < 0.1:
                    for _ in range(4):
                        call()
                    torch.cuda.synchronize()
                p = sg.plan(M, N, K, cfg, sched)
                out.writerow([str(seed), M, N, K, cfg, sched, sg.CFG_NAMES[p["config"]], sg.SCHED_NAMES[p["sched"]],
                              p["dp_tiles"], p["sk_tiles"], p["grid"], p["sk_grid"], p["iters_per_tile"],
                              round(timed(call, 15), 2)])
                sys.stdout.flush()
            del A, B, C
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main(sys.argv)
