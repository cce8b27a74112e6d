"""Benchmark of the FP32 GEMM (C = A @ B, row-major, AB only) on one MI355X.

Prints ONE JSON line on stdout: FP32 SGEMM TFLOP/s (2*M*N*K / t) of the
headline 4096^3 workload (or --workload), with inputs resident in HBM, K
back-to-back calls timed between two device synchronisations (after W
untimed calls, continued to at least --warm-seconds so that the shader clock
has ramped up), plus:
  * "roofline": per-launch kernel time from HIP events recorded on the
    launch stream, against the MI355X FP32 matrix peak (157.3 TFLOP/s);
  * "cpu_baseline": the FP64 CPU oracle timed on a bounded row sample of the
    same product, on this host's cores.
The line also carries the median single-call time with a 512 MiB buffer
written before each call (caches flushed: "cold_median_event_tflops").
Details (every workload with --all, the plan, a torch.matmul context figure)
go to stderr and to --detail FILE.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--warm-seconds 0.5] [--workload NAME]
                       [--config N] [--sched N] [--all] [--no-cpu-baseline]
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

PEAK_FP32_TFLOPS = 157.3          # MI355X dense FP32 (vector with packed FMA, or matrix)
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E
PEAK_HBM_GBS = 8000.0
# The pages' own kernel at 4096^3 on an H100 (context, other hardware): "Beyond
# Kernel 7", section "The confirmed result", k13f 2761.2 us = 49.8 TFLOP/s.
PAGES_4096_TFLOPS = 49.8

# HBM-side bytes per launch of the headline kernel, from two rocprofv3 --pmc
# runs (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each scaled by what the
# same counter reads for a plain 256 MiB device copy (FETCH_SIZE 2.0, WRITE_SIZE
# 1.0); see profiles/sgemm_4096_dl_256x256x16_counters.md.  Valid only for the
# kernel sources they were taken on (digest below); otherwise reported null.
TRAFFIC = {
    "kernel": "dl_256x256x16", "workload": "sgemm_4096",
    "source_digest": "c901998312e62bc7",
    "bytes": 469864950,
}
KERNEL_SOURCES = ("fp32_sgemm_f32_amd/csrc/gemm_mfma_dl.hip", "fp32_sgemm_f32_amd/csrc/gemm_common.h")


def code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed: what the
    compiler sees of it (string literals in these sources hold no comment
    markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest(read=None) -> str:
    """Digest of the headline kernel's sources, comments and layout ignored."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="keep making untimed warm-up calls until this long has passed (clock ramp)")
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--shape", default=None, metavar="MxNxK",
                    help="instead of a named workload: this shape, dense row-major operands "
                         "(lda = K, ldb = ldc = N), U[-1,1] seed 0 unless --dist / --seed")
    ap.add_argument("--dist", default="uniform", choices=workloads.DISTRIBUTIONS)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--config", type=int, default=0)
    ap.add_argument("--sched", type=int, default=0)
    ap.add_argument("--all", action="store_true", help="also time every workload (details only)")
    ap.add_argument("--cold", action="store_true", help="with --all: also time the other workloads with "
                    "caches flushed before each call (the headline always is)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-flushed timing of the headline")
    ap.add_argument("--torch", action="store_true", help="also time torch.matmul (context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--detail", default=None, help="write a detail JSON file")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead: time a plain device copy of this many MiB (calibrates "
                         "the HBM byte counters of a profiler run)")
    return ap.parse_args()


def ensure_library():
    import fp32_sgemm_f32_amd as sg
    if not os.path.exists(sg.LIB_PATH):
        from fp32_sgemm_f32_amd import build
        build.build()
    sg.library()
    return sg


def warm_up(fn, calls, min_seconds):
    """`calls` untimed calls, continued until at least min_seconds of them
    have run: the shader clock ramps up over tens of milliseconds, longer
    than a few calls of a small product take.  Returns the calls made."""
    import torch
    done = 0
    t0 = time.perf_counter()
    while done < calls or time.perf_counter() - t0 < min_seconds:
        for _ in range(max(1, min(calls, 8))):
            fn()
            done += 1
        torch.cuda.synchronize()
    return done


def time_region(fn, stream, steps, warmup, min_warm_s=0.0):
    """The timed region: `steps` back-to-back calls between two device
    synchronisations, with one HIP event pair recorded on `stream` around
    them (nothing between the calls).  Returns (wall s, event ms, warm-up
    calls made)."""
    import torch
    warm = warm_up(fn, warmup, min_warm_s)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end), warm


def time_calls(fn, stream, steps, warmup, flush=None, min_warm_s=0.0):
    """Per-call HIP-event times (ms) on `stream` (an event pair around each
    call: the distribution of single-call times), plus the total wall of the
    run and the warm-up calls made."""
    import torch
    warm = warm_up(fn, warmup, min_warm_s)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return per, wall, warm


def bench_workload(sg, w, args, dev, stream, cold=False, with_torch=False):
    import torch
    A, B = workloads.generate_workload(w)
    Ad = torch.from_numpy(A).to(dev)
    Bd = torch.from_numpy(B).to(dev)
    Cd = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    del A, B

    def call():
        st = sg.sgemm_raw(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N, Cd.data_ptr(), w.N,
                          stream.cuda_stream, args.config, args.sched)
        if st != sg.OK:
            raise sg.SgemmError(st)

    # Sanity check before timing (the parity proof is the test suite): a
    # sample of rows against an FP64 product on the device.
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    rows = torch.arange(0, w.M, max(1, w.M // 64), device=dev)
    ref = Ad[rows].double() @ Bd.double()
    scale = Ad[rows].double().abs() @ Bd.double().abs()
    err = (Cd[rows].double() - ref).abs()
    sane = bool(torch.all(err <= 1e-5 * scale).item()) and bool(torch.isfinite(Cd).all().item())
    del ref, scale, err

    with torch.cuda.stream(stream):
        wall, region_ms, warm = time_region(call, stream, args.steps, args.warmup, args.warm_seconds)
        # Single-call distribution, in a second pass (the event pairs around
        # each call put gaps between the kernels, so they stay out of the
        # timed region).
        per, _, _ = time_calls(call, stream, args.steps, 0)
    flops = w.flops
    res = {
        "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist, "seed": w.seed,
        "sane": sane,
        "steps": args.steps, "warmup": args.warmup, "warmup_calls": warm,
        "wall_s": wall,
        "ms_per_step": wall / args.steps * 1e3,
        "tflops": flops * args.steps / wall / 1e12,
        "region_event_ms_per_call": region_ms / args.steps,
        "event_ms_median": statistics.median(per),
        "event_ms_mean": statistics.fmean(per),
        "event_ms_min": min(per),
        "event_ms_p90": float(np.percentile(per, 90)),
        "tflops_median": flops / (statistics.median(per) * 1e-3) / 1e12,
        "plan": sg.plan(w.M, w.N, w.K, args.config, args.sched,
                        num_cus=torch.cuda.get_device_properties(dev).multi_processor_count),
    }
    if cold:
        flush_buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        with torch.cuda.stream(stream):
            per_c, _, _ = time_calls(call, stream, max(20, args.steps // 2), 3,
                                  flush=lambda: flush_buf.fill_(1.0), min_warm_s=args.warm_seconds)
        res["cold_event_ms_median"] = statistics.median(per_c)
        res["cold_tflops_median"] = flops / (statistics.median(per_c) * 1e-3) / 1e12
        del flush_buf
    if with_torch:
        torch.backends.cuda.matmul.allow_tf32 = False
        out = torch.empty_like(Cd)
        with torch.cuda.stream(stream):
            per_t, _, _ = time_calls(lambda: torch.matmul(Ad, Bd, out=out), stream, args.steps, args.warmup,
                                  min_warm_s=args.warm_seconds)
        res["torch_matmul_event_ms_median"] = statistics.median(per_t)
        res["torch_matmul_tflops_median"] = flops / (statistics.median(per_t) * 1e-3) / 1e12
    del Ad, Bd, Cd
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, budget_s):
    """The FP64 oracle on the same product, blocks of rows in order, until
    about budget_s seconds of work; where the whole product takes less, it
    is computed again from its first row (passes over the same work).
    Returns the TFLOP/s it sustains (2*rows*N*K per s)."""
    import oracle
    threads = oracle.default_threads()
    A, B = workloads.generate_workload(w)
    oracle._load()
    rows_done, spent = 0, 0.0
    step = max(threads, 32)
    while spent < budget_s and w.M > 0:
        r0 = rows_done % w.M
        r1 = min(w.M, r0 + step)
        t0 = time.perf_counter()
        oracle.gemm(A[r0:r1], B, threads=threads)
        spent += time.perf_counter() - t0
        rows_done += r1 - r0
    value = 2.0 * rows_done * w.N * w.K / spent / 1e12
    if rows_done >= w.M:
        what = f"the whole {w.M}x{w.N}x{w.K} product, {rows_done / w.M:.2f} passes"
    else:
        what = f"rows 0..{rows_done - 1} of the {w.M}x{w.N}x{w.K} product ({rows_done}x{w.N} outputs, full K)"
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, FP64 triple loop (also forms sum|a*b|), {spent:.1f} s on {threads} threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this GEMM has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    sg = ensure_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name}, {props.multi_processor_count} CUs, {props.total_memory / 2**30:.0f} GiB")

    if args.copy_mib:
        n = args.copy_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            per, wall, _ = time_calls(lambda: dst.copy_(src), stream, args.steps, args.warmup)
        t = statistics.median(per) * 1e-3
        print(json.dumps({"metric": "device copy GB/s (read + write)", "value": round(2 * n * 4 / t / 1e9, 1),
                          "unit": "GB/s", "bytes_read": n * 4, "bytes_written": n * 4,
                          "median_ms": round(t * 1e3, 4), "steps": args.steps}), flush=True)
        return

    if args.shape:
        M, N, K = (int(x) for x in args.shape.lower().split("x"))
        w = workloads.Workload(f"sgemm_{M}x{N}x{K}", M, N, K, args.dist, args.seed)
    else:
        w = workloads.WORKLOADS[args.workload]
    head = bench_workload(sg, w, args, dev, stream, cold=not args.no_cold, with_torch=args.torch)
    log(json.dumps(head))
    detail = {"headline": head, "device": props.name, "cus": props.multi_processor_count}
    if args.all:
        rest = []
        for name, ww in workloads.WORKLOADS.items():
            if name == w.name:
                continue
            r = bench_workload(sg, ww, args, dev, stream, cold=args.cold, with_torch=args.torch)
            log(json.dumps(r))
            rest.append(r)
        detail["others"] = rest
        if not args.no_cpu_baseline:
            # The FP64 oracle on each workload (a bounded row sample, whole
            # product where it fits the budget) beside the GPU's median.
            for r in [head] + rest:
                ww = w if r is head else workloads.WORKLOADS[r["workload"]]
                cpu_r = cpu_baseline(ww, min(args.cpu_seconds, 6.0))
                r["cpu_oracle"] = cpu_r
                r["gpu_over_oracle"] = r["tflops_median"] / cpu_r["value"]
                log(f"{ww.name}: oracle {cpu_r['value'] * 1e3:.1f} GFLOP/s ({cpu_r['sample']}); "
                    f"GPU median {r['tflops_median']:.1f} TFLOP/s = {r['gpu_over_oracle']:.0f}x")

    achieved = w.flops / (head["region_event_ms_per_call"] * 1e-3) / 1e12
    traffic = None
    if (TRAFFIC["kernel"] == sg.CFG_NAMES[head["plan"]["config"]] and TRAFFIC["workload"] == w.name
            and TRAFFIC["source_digest"] == kernel_source_digest()):
        traffic = TRAFFIC["bytes"]
    # The vector-ALU kernel is bounded by the FP32 vector rate (157.3 TFLOP/s
    # too), the skinny and row-dot kernels (at most 16 rows / 8 columns) by
    # HBM: their algorithmic bytes are A, B and C once, 4 (MK + KN + MN);
    # the others by the FP32 matrix-core rate.
    cfg = head["plan"]["config"]
    if cfg in (sg.CFG_SKINNY_16x256, sg.CFG_ROWDOT_N8):
        gbps = 4 * (w.M * w.K + w.K * w.N + w.M * w.N) / (head["region_event_ms_per_call"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None, "traffic_unit": "bytes per launch"}
    else:
        bound = "alu" if cfg == sg.CFG_VALU_128x128x8 else "mfma"
        roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch"}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(json.dumps(cpu))
    cfg_name = sg.CFG_NAMES[head["plan"]["config"]]
    line = {
        "metric": "FP32 SGEMM TFLOPS (2MNK/s)",
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": head["warmup_calls"],
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(head["tflops"] / PAGES_4096_TFLOPS, 3) if w.name == "sgemm_4096" else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist, "seed": w.seed,
                   "kernel": cfg_name, "sched": sg.SCHED_NAMES[head["plan"]["sched"]],
                   "grid": head["plan"]["grid"], "parallelism": "single-gpu",
                   **({"repacked": True} if head["plan"]["repacked"] else {})},
        "frac_of_fp32_peak": round(head["tflops"] / PEAK_FP32_TFLOPS, 4),
        "median_event_tflops": round(head["tflops_median"], 3),
        "cold_median_event_tflops": (round(head["cold_tflops_median"], 3) if "cold_tflops_median" in head
                                     else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sane": head["sane"],
    }
    if args.detail:
        detail["line"] = line
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
