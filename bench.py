"""Benchmark: dense row-major GEMM on one MI355X.

A step is one gemm_f32 call, C = 1.5*A*B + 0.5*C at M = N = K = 4096 (fp32,
operands ~ U[-1,1), already resident in HBM).  The JSON line reports its
TFLOP/s (2*M*N*K per step), the kernel's fraction of the fp32 matrix-core
peak, the 16-bit 8192^3 and batched QK^T workloads as secondary figures, and
the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
       python bench.py --copy-probe            (plain 256 MiB copies, for counter calibration)
       python bench.py --summarize-profiles DIR (writes the profiles/ summary from rocprofv3 CSVs)

HBM traffic of the dominant kernel comes from rocprofv3 FETCH_SIZE / WRITE_SIZE
runs summarised under profiles/; it is reported only while the kernel sources
still hash to the value recorded with those counters.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "sgemm_fp32_4096_counters.txt")
COPY_PROBE_BYTES = 256 << 20


def kernel_source_sha():
    """sha256 over the HIP sources and headers the kernels are built from."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_f32_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel_name):
    """Bytes per launch measured by FETCH_SIZE + WRITE_SIZE (copy-calibrated), or None when
    no summary exists or the kernel sources changed since it was taken."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None
    vals = {}
    with open(PROFILE_SUMMARY) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_sha() or vals.get("kernel") != kernel_name:
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_means(directory, name_filter):
    """Mean counter value per (counter) over dispatches whose kernel name matches."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    sums, counts = {}, {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if name_filter not in r["Kernel_Name"]:
                    continue
                c = r["Counter_Name"]
                sums[c] = sums.get(c, 0.0) + float(r["Counter_Value"])
                counts[c] = counts.get(c, 0) + 1
    return {c: sums[c] / counts[c] for c in sums}


def _kernel_stats(directory, name_filter):
    files = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if name_filter in r["Name"]:
                    return r
    return None


def _dispatch_durations(directory, name_filter):
    """Per-dispatch kernel durations (ns) in launch order."""
    files = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    out = []
    for fn in files:
        with open(fn) as f:
            rows = [r for r in csv.DictReader(f) if name_filter in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        out += [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    return out


def summarize_profiles(d):
    """Write the profiles/ summary from rocprofv3 output under d:
    d/trace (kernel-trace --stats of the default bench step), d/fetch and d/write
    (FETCH_SIZE / WRITE_SIZE of the bench step), d/copy_fetch and d/copy_write
    (the same counters on --copy-probe)."""
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import workloads as wl
    p = wl.sgemm_4096()
    info, _ = mg.select(p.dtype, 0, 0, p.M, p.N, p.K, p.alpha, 1 << 20, p.lda, 0, 1 << 20, p.ldb, 0,
                        p.beta, 1 << 20, p.ldc, 0, 1)
    kname = info["name"]
    # kernel names appear demangled in the rocprofv3 CSVs
    inst = "gemm_kernel<float, %d, %d, %d, %d, %d, false, false, true, %d>" % (
        info["block_m"], info["block_n"], info["block_k"], info["waves_m"], info["waves_n"],
        info["pipe"])
    stats = _kernel_stats(os.path.join(d, "trace"), inst)
    durs = _dispatch_durations(os.path.join(d, "trace"), inst)
    timed = durs[5:]  # the traced command ran 5 warmup steps, then the timed ones
    fetch = _counter_means(os.path.join(d, "fetch"), inst).get("FETCH_SIZE")
    write = _counter_means(os.path.join(d, "write"), inst).get("WRITE_SIZE")
    cf = _counter_means(os.path.join(d, "copy_fetch"), "copyBuffer").get("FETCH_SIZE")
    cw = _counter_means(os.path.join(d, "copy_write"), "copyBuffer").get("WRITE_SIZE")
    expect_kib = COPY_PROBE_BYTES / 1024.0
    sf, sw = expect_kib / cf, expect_kib / cw
    traffic = int(round((fetch * sf + write * sw) * 1024))
    algo = (p.M * p.K + p.K * p.N) * 4 + p.M * p.N * 4 * 2
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o run -- "
           "python3 bench.py --steps 20 --warmup 5 --no-cpu --no-secondary;  "
           "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o run -- "
           "python3 bench.py --steps 5 --warmup 2 --no-cpu --no-secondary;  "
           "rocprofv3 --pmc WRITE_SIZE (same, -d DIR/write);  "
           "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE -d DIR/copy_fetch, DIR/copy_write -- "
           "python3 bench.py --copy-probe;  python3 bench.py --summarize-profiles DIR")
    lines = [
        "# rocprofv3 summary: SGEMM fp32 M=N=K=4096, alpha=1.5, beta=0.5 (the bench step)",
        "command: " + cmd,
        "kernel: " + kname,
        "kernel_symbol_contains: " + inst,
        "source_sha256: " + kernel_source_sha(),
        "calls: " + (stats["Calls"] if stats else "n/a"),
        "average_ns_timed_steps: %.0f" % (sum(timed) / len(timed) if timed else float("nan")),
        "average_ns: " + (stats["AverageNs"] if stats else "n/a"),
        "min_ns: " + (stats["MinNs"] if stats else "n/a"),
        "max_ns: " + (stats["MaxNs"] if stats else "n/a"),
        "FETCH_SIZE_KiB_per_dispatch: %.1f" % fetch,
        "WRITE_SIZE_KiB_per_dispatch: %.1f" % write,
        "copy_probe_bytes: %d" % COPY_PROBE_BYTES,
        "copy_FETCH_SIZE_KiB: %.1f" % cf,
        "copy_WRITE_SIZE_KiB: %.1f" % cw,
        "fetch_scale: %.4f" % sf,
        "write_scale: %.4f" % sw,
        "traffic_bytes_per_launch: %d" % traffic,
        "algorithmic_bytes_per_launch: %d" % algo,
        "traffic_over_algorithmic: %.3f" % (traffic / algo),
    ]
    os.makedirs(os.path.dirname(PROFILE_SUMMARY), exist_ok=True)
    with open(PROFILE_SUMMARY, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_probe():
    """Plain device copies of a known size (counter calibration for FETCH/WRITE_SIZE)."""
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy probe done", flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_device_problem(p, torch, dev):
    from dense_gemm_f32_amd import workloads as wl
    A, B, C0 = wl.make_inputs(p)
    dA, dB = A.to(dev), B.to(dev)
    dC = C0.to(dev) if C0 is not None else torch.zeros(p.c_elems, dtype=torch.float32, device=dev)
    return dA, dB, dC


def launcher(p, dA, dB, dC):
    import dense_gemm_f32_amd as mg
    if p.batch == 1:
        fn = {"f32": mg.gemm_f32, "f16": mg.gemm_f16, "bf16": mg.gemm_bf16}[p.dtype]
        return lambda: fn(int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, dA, p.lda, dB,
                          p.ldb, p.beta, dC, p.ldc)
    return lambda: mg.gemm_strided_batched(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K,
                                           p.alpha, dA, p.lda, p.strideA, dB, p.ldb, p.strideB,
                                           p.beta, dC, p.ldc, p.strideC, p.batch)


def time_kernel(torch, fn, iters):
    """Average duration of one launch, from HIP events recorded on the stream the
    library launches on (the current torch stream)."""
    s = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(iters):
        fn()
    stop.record(s)
    stop.synchronize()
    return start.elapsed_time(stop) / iters * 1e-3


def algorithmic_bytes(p):
    """Compulsory HBM traffic: A and B once, C written (and read when beta != 0)."""
    from dense_gemm_f32_amd import workloads as wl
    es = wl.ELEM_SIZE[p.dtype]
    per = (p.M * p.K + p.K * p.N) * es + p.M * p.N * 4 * (2 if p.beta != 0 else 1)
    return per * p.batch


def secondary(torch, dev, iters):
    from dense_gemm_f32_amd import workloads as wl
    import dense_gemm_f32_amd as mg
    out = {}
    for name in ("gemm_bf16_8192", "gemm_f16_8192", "qkt_batched", "sgemm_256", "sgemm_ragged"):
        p = wl.WORKLOADS[name]()
        dA, dB, dC = make_device_problem(p, torch, dev)
        fn = launcher(p, dA, dB, dC)
        # warm up to the steady clock the part settles at under this load
        for _ in range(30):
            fn()
        torch.cuda.synchronize()
        t = time_kernel(torch, fn, iters)
        tf = p.flops / t / 1e12
        info, grid = mg.select(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                               dA.data_ptr(), p.lda, p.strideA, dB.data_ptr(), p.ldb, p.strideB,
                               p.beta, dC.data_ptr(), p.ldc, p.strideC, p.batch)
        rec = {"tflops": round(tf, 2), "ms": round(t * 1e3, 4),
               "frac_matrix_peak": round(tf / PEAK_TFLOPS[p.dtype], 4),
               "kernel": info["name"], "grid": grid}
        if name == "qkt_batched":
            gbs = algorithmic_bytes(p) / t / 1e9
            rec["hbm_gbs"] = round(gbs, 1)
            rec["frac_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
            rec["bound"] = "hbm"
        else:
            rec["bound"] = "mfma"
        out[name] = rec
        log(f"secondary {name}: {rec}")
        del dA, dB, dC
        torch.cuda.empty_cache()
    return out


def cpu_baseline(p, A, B, C0, budget_s=15.0):
    """The oracle, as it stands, on the first R rows of the same workload."""
    import numpy as np
    import oracle
    from dense_gemm_f32_amd import workloads as wl
    An = wl.to_numpy_operand(A)
    Bn = wl.to_numpy_operand(B)
    Cn = C0.numpy() if C0 is not None else None
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))

    def rows(r):
        t0 = time.perf_counter()
        oracle.gemm(p.dtype, p.transA, p.transB, r, p.N, p.K, p.alpha, An[:r * p.lda], p.lda, Bn,
                    p.ldb, p.beta, None if Cn is None else Cn[:r * p.ldc], p.ldc)
        return time.perf_counter() - t0

    r = max(threads, 4)
    t = rows(r)
    r2 = int(min(p.M, max(r, r * budget_s / max(t, 1e-6))))
    r2 = max(threads, (r2 // threads) * threads)
    t2 = rows(r2)
    flops = 2.0 * r2 * p.N * p.K
    return {"value": flops / t2 / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"first {r2} of {p.M} output rows of the same {p.M}x{p.N}x{p.K} fp32 GEMM "
                      f"({flops / 1e9:.1f} GFLOP, fp64 accumulation, {t2:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize-profiles", metavar="DIR")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); a GEMM shards by "
              "rows or batch entries with no exchange, so the one-GPU rate is the figure.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import workloads as wl

    dev = torch.device("cuda:0")
    p = wl.sgemm_4096()
    A, B, C0 = wl.make_inputs(p)
    dA, dB, dC = A.to(dev), B.to(dev), C0.to(dev)
    step = launcher(p, dA, dB, dC)
    info, grid = mg.select(p.dtype, 0, 0, p.M, p.N, p.K, p.alpha, dA.data_ptr(), p.lda, 0,
                           dB.data_ptr(), p.ldb, 0, p.beta, dC.data_ptr(), p.ldc, 0, 1)
    log(f"workload sgemm 4096^3 alpha=1.5 beta=0.5: kernel {info['name']} grid {grid}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps, synchronised on both sides; HIP events recorded on
    # the stream the library launches on (the current torch stream) give the
    # kernel's own average duration over the same launches
    s = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(s)
    for _ in range(args.steps):
        step()
    ev1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3
    value = p.flops / (wall / args.steps) / 1e12
    t_kernel = ev0.elapsed_time(ev1) / args.steps * 1e-3
    log(f"timed {args.steps} steps: {ms:.4f} ms/step, {value:.2f} TFLOP/s; "
        f"kernel {t_kernel * 1e3:.4f} ms")

    achieved = p.flops / t_kernel / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["f32"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["f32"], 4),
                "traffic": stored_traffic(info["name"]), "kernel": info["name"],
                "kernel_ms": round(t_kernel * 1e3, 4), "algorithmic_flop_per_launch": p.flops,
                "algorithmic_bytes_per_launch": algorithmic_bytes(p)}

    sec = None if args.no_secondary else secondary(torch, dev, 30)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(p, A, B, C0)
        log(f"cpu_baseline: {cpu}")

    line = {
        "metric": "GEMM TFLOP/s + % of MI355X matrix peak (fp32 4096^3, bf16 8192^3)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded U[-1,1) operands, generated on the host, resident in HBM)",
        "config": {"workload": "sgemm_fp32_4096x4096x4096_alpha1.5_beta0.5", "M": p.M, "N": p.N,
                   "K": p.K, "alpha": p.alpha, "beta": p.beta, "kernel": info["name"],
                   "grid": grid},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": sec,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
