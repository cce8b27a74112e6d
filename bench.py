"""Benchmark of the FP32 GEMM (C = A @ B, row-major, AB only) on one MI355X.

Prints ONE JSON line on stdout: FP32 SGEMM TFLOP/s (2*M*N*K / t) of the
headline 4096^3 workload (or --workload / --shape).  The timing protocol is
the one the page "Beyond Kernel 7: Closing the Gap to cuBLAS on an H100 FP32
GEMM" uses for its confirmed result, with the cache flush sized for MI355X:
before every timed call a 512 MiB buffer is written (more than the 32 MiB of
L2 plus the 256 MiB MALL, so A and B come from HBM), outside the HIP-event
pair that times the call; `value` is the median of the K single-call times.
The line also carries:
  * "warm": the same calls back to back with nothing between them (A and B
    then stay in the caches);
  * "sizes": the other measured workloads (1024^3 and its integer variant,
    2048^3, 256^3, 1024 x 1024 x 16384), flushed and warm medians each;
  * "roofline": algorithmic FLOPs per launch over the kernel's mean launch
    duration in the flushed timed region (HIP events on the launch stream),
    against the MI355X FP32 matrix peak (157.3 TFLOP/s);
  * "cpu_baseline": the FP64 CPU oracle timed on a bounded sample of the
    same product on this host's cores;
  * "fixed_shape": the same product on the kernel compiled for its exact
    shape (SGEMM_SCHED_FIXED), same protocol, beside the runtime kernel.
Details (the plan, a torch.matmul context figure with --torch) go to stderr
and to --detail FILE.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--warm-seconds 0.5] [--workload NAME]
                       [--shape MxNxK] [--config N] [--sched N] [--no-sizes] [--no-cpu-baseline]
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
FLUSH_MIB = 512                   # written before each timed call: > L2 (32 MiB) + MALL (256 MiB)
FLUSHED_WARMUP_CALLS, FLUSHED_WARMUP_S = 20, 0.1

# HBM-side bytes per launch of the headline kernel in the flushed protocol,
# from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE in KiB per dispatch),
# each scaled by what the same counter reads for a plain 256 MiB device copy
# (FETCH_SIZE 2.0, WRITE_SIZE 1.0); see
# profiles/sgemm_4096_dl_256x256x16_counters.md.  Valid only for the kernel
# sources they were taken on (digest below); otherwise reported null.
TRAFFIC = {
    "kernel": "dl_256x256x16", "workload": "sgemm_4096",
    "source_digest": "fa1511ea6658fa1b",
    "bytes": 469913489,
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
    ap.add_argument("--no-sizes", action="store_true", help="skip the other workloads")
    ap.add_argument("--size-steps", type=int, default=30, help="timed calls per other workload and protocol")
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


def time_region(fn, stream, steps):
    """`steps` back-to-back calls between two device synchronisations, with
    one HIP event pair recorded on `stream` around them (nothing between the
    calls).  Returns (wall s, event ms)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, start.elapsed_time(end)


def time_calls(fn, stream, steps, flush=None):
    """`steps` calls between two device synchronisations, each inside its
    own HIP event pair on `stream`; `flush` (if given) runs before each pair,
    outside it.  Returns (per-call ms, wall s of the whole region)."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def stats(per_ms, flops):
    med = statistics.median(per_ms)
    return {"median_ms": med, "mean_ms": statistics.fmean(per_ms), "min_ms": min(per_ms),
            "p90_ms": float(np.percentile(per_ms, 90)), "tflops_median": flops / (med * 1e-3) / 1e12}


def bench_workload(sg, w, dev, stream, flush, steps, warmup, warm_seconds, config=0, sched=0,
                   with_torch=False, alt_scheds=()):
    """One workload: a correctness sanity check, the warm-up, then the
    flushed timed region (the headline protocol), then the warm ones."""
    import torch
    A, B = workloads.generate_workload(w)
    Ad = torch.from_numpy(A).to(dev)
    Bd = torch.from_numpy(B).to(dev)
    Cd = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    del A, B

    def call_with(cfg, sch):
        def call():
            st = sg.sgemm_raw(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N, Cd.data_ptr(), w.N,
                              stream.cuda_stream, cfg, sch)
            if st != sg.OK:
                raise sg.SgemmError(st)
        return call

    call = call_with(config, sched)

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

    flops = w.flops
    with torch.cuda.stream(stream):
        warm_calls = warm_up(call, warmup, warm_seconds)
        # Flushed calls, untimed, before the flushed timed region: after a run
        # of back-to-back calls the first ~20 flushed ones on MI355X take up to
        # 20% longer and settle over ~20 ms (measured: 1092, 1084, 1070, ...
        # 915 us at 4096^3), a transient of the switch, not of the protocol.
        warm_up(lambda: (flush(), call()), FLUSHED_WARMUP_CALLS, FLUSHED_WARMUP_S)
        cold, cold_wall = time_calls(call, stream, steps, flush=flush)
        region_wall, region_ms = time_region(call, stream, steps)
        warm, _ = time_calls(call, stream, steps)
    res = {
        "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist, "seed": w.seed, "sane": sane,
        "steps": steps, "warmup_calls": warm_calls,
        "cold": dict(stats(cold, flops), wall_s=cold_wall),
        "warm": dict(stats(warm, flops), region_ms_per_call=region_ms / steps,
                     region_tflops=flops * steps / region_wall / 1e12),
        "plan": sg.plan(w.M, w.N, w.K, config, sched,
                        num_cus=torch.cuda.get_device_properties(dev).multi_processor_count),
    }
    # Other schedules of the same call (the compile-time-shape kernel), under
    # the same flushed protocol, right after.
    for sch in alt_scheds:
        fn = call_with(config, sch)
        with torch.cuda.stream(stream):
            warm_up(fn, warmup, warm_seconds)
            warm_up(lambda: (flush(), fn()), FLUSHED_WARMUP_CALLS, FLUSHED_WARMUP_S)
            per_c, _ = time_calls(fn, stream, steps, flush=flush)
            per_w, _ = time_calls(fn, stream, steps)
        res.setdefault("alt", {})[sg.SCHED_NAMES[sch]] = {"cold": stats(per_c, flops), "warm": stats(per_w, flops)}
    if with_torch:
        torch.backends.cuda.matmul.allow_tf32 = False
        out = torch.empty_like(Cd)
        fn = lambda: torch.matmul(Ad, Bd, out=out)  # noqa: E731
        with torch.cuda.stream(stream):
            warm_up(fn, warmup, warm_seconds)
            per_t, _ = time_calls(fn, stream, steps, flush=flush)
        res["torch_matmul_cold"] = stats(per_t, flops)
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


def size_entry(sg, r):
    c, wm = r["cold"], r["warm"]
    return {"kernel": sg.CFG_NAMES[r["plan"]["config"]], "sched": sg.SCHED_NAMES[r["plan"]["sched"]],
            "cold_median_tflops": round(c["tflops_median"], 3),
            "cold_frac": round(c["tflops_median"] / PEAK_FP32_TFLOPS, 4),
            "cold_median_us": round(c["median_ms"] * 1e3, 2),
            "warm_median_tflops": round(wm["tflops_median"], 3),
            "warm_frac": round(wm["tflops_median"] / PEAK_FP32_TFLOPS, 4),
            "warm_median_us": round(wm["median_ms"] * 1e3, 2), "sane": r["sane"]}


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
            warm_up(lambda: dst.copy_(src), args.warmup, 0.0)
            per, _ = time_calls(lambda: dst.copy_(src), stream, args.steps)
        t = statistics.median(per) * 1e-3
        print(json.dumps({"metric": "device copy GB/s (read + write)", "value": round(2 * n * 4 / t / 1e9, 1),
                          "unit": "GB/s", "bytes_read": n * 4, "bytes_written": n * 4,
                          "median_ms": round(t * 1e3, 4), "steps": args.steps}), flush=True)
        return

    flush_buf = torch.empty(FLUSH_MIB * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    flush = lambda: flush_buf.fill_(1.0)  # noqa: E731

    if args.shape:
        M, N, K = (int(x) for x in args.shape.lower().split("x"))
        w = workloads.Workload(f"sgemm_{M}x{N}x{K}", M, N, K, args.dist, args.seed)
    else:
        w = workloads.WORKLOADS[args.workload]
    # The kernel compiled for this exact product, if there is one (reported
    # beside the runtime kernel that `value` measures).
    try:
        fixed = [sg.SCHED_FIXED] if sg.plan(w.M, w.N, w.K, args.config, sg.SCHED_FIXED)["fixed_shape"] else []
    except sg.SgemmError:
        fixed = []
    head = bench_workload(sg, w, dev, stream, flush, args.steps, args.warmup, args.warm_seconds,
                          args.config, args.sched, with_torch=args.torch, alt_scheds=fixed)
    log(json.dumps(head))
    detail = {"headline": head, "device": props.name, "cus": props.multi_processor_count}

    sizes = {}
    if not args.no_sizes and not args.shape:
        for name, ww in workloads.WORKLOADS.items():
            if name == w.name:
                continue
            r = bench_workload(sg, ww, dev, stream, flush, args.size_steps, args.warmup, args.warm_seconds,
                               with_torch=args.torch)
            log(json.dumps(r))
            detail.setdefault("others", []).append(r)
            sizes[name] = size_entry(sg, r)

    cold = head["cold"]
    cfg = head["plan"]["config"]
    # The kernel's mean launch duration over the flushed timed region.
    mean_s = cold["mean_ms"] * 1e-3
    if cfg in (sg.CFG_SKINNY_16x256, sg.CFG_ROWDOT_N8):
        # At most 16 rows / 8 columns: bounded by HBM; algorithmic bytes are
        # A, B and C once, 4 (MK + KN + MN).
        gbps = 4 * (w.M * w.K + w.K * w.N + w.M * w.N) / mean_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None, "traffic_unit": "bytes per launch"}
    else:
        traffic = None
        if (TRAFFIC["kernel"] == sg.CFG_NAMES[cfg] and TRAFFIC["workload"] == w.name
                and TRAFFIC["source_digest"] == kernel_source_digest()):
            traffic = TRAFFIC["bytes"]
        achieved = w.flops / mean_s / 1e12
        # The vector-ALU kernel is bounded by the FP32 vector rate (157.3
        # TFLOP/s too), the others by the FP32 matrix-core rate.
        bound = "alu" if cfg in (sg.CFG_VALU_128x128x8, sg.CFG_VALU_256x128x8) else "mfma"
        roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch"}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(json.dumps(cpu))
    warm = head["warm"]
    line = {
        "metric": "FP32 SGEMM TFLOPS (2MNK/s)",
        "value": round(cold["tflops_median"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": head["warmup_calls"],
        "ms_per_step": round(cold["wall_s"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dist": w.dist, "seed": w.seed,
                   "kernel": sg.CFG_NAMES[cfg], "sched": sg.SCHED_NAMES[head["plan"]["sched"]],
                   "grid": head["plan"]["grid"], "parallelism": "single-gpu",
                   "protocol": f"median of {args.steps} single-call HIP-event times, {FLUSH_MIB} MiB "
                               "written before each call outside the events (caches flushed)",
                   **({"repacked": True} if head["plan"]["repacked"] else {})},
        "frac_of_fp32_peak": round(cold["tflops_median"] / PEAK_FP32_TFLOPS, 4),
        "median_us": round(cold["median_ms"] * 1e3, 2),
        "min_us": round(cold["min_ms"] * 1e3, 2),
        "p90_us": round(cold["p90_ms"] * 1e3, 2),
        "warm": {"median_tflops": round(warm["tflops_median"], 3),
                 "frac": round(warm["tflops_median"] / PEAK_FP32_TFLOPS, 4),
                 "median_us": round(warm["median_ms"] * 1e3, 2),
                 "region_tflops": round(warm["region_tflops"], 3)},
        "sizes": sizes,
        "fixed_shape": ({"cold_median_tflops": round(head["alt"]["fixed"]["cold"]["tflops_median"], 3),
                         "warm_median_tflops": round(head["alt"]["fixed"]["warm"]["tflops_median"], 3),
                         "cold_vs_value": round(head["alt"]["fixed"]["cold"]["tflops_median"] / cold["tflops_median"], 4)}
                        if "alt" in head else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "vs_cpu_baseline": round(cold["tflops_median"] / cpu["value"], 1) if cpu else None,
        "sane": head["sane"] and all(s["sane"] for s in sizes.values()),
    }
    if args.detail:
        detail["line"] = line
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
