"""Benchmark: dense row-major GEMM on one MI355X.

A step is one gemm_f32 call, C = 1.5*A*B + 0.5*C at M = N = K = 4096 (fp32,
operands ~ U[-1,1), already resident in HBM).  The JSON line reports its
TFLOP/s (2*M*N*K per step), the kernel's fraction of the fp32 matrix-core
peak, the 16-bit 8192^3 and batched QK^T workloads as secondary figures, and
the CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0


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
    for name in ("gemm_bf16_8192", "gemm_f16_8192", "qkt_batched"):
        p = wl.WORKLOADS[name]()
        dA, dB, dC = make_device_problem(p, torch, dev)
        fn = launcher(p, dA, dB, dC)
        for _ in range(3):
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
    args = ap.parse_args()
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
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall / args.steps * 1e3
    value = p.flops / (wall / args.steps) / 1e12
    log(f"timed {args.steps} steps: {ms:.4f} ms/step, {value:.2f} TFLOP/s")

    # dominant (only) kernel: its own average duration from HIP events on its stream
    t_kernel = time_kernel(torch, step, max(args.steps, 20))
    achieved = p.flops / t_kernel / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["f32"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["f32"], 4),
                "traffic": None, "kernel": info["name"], "kernel_ms": round(t_kernel * 1e3, 4),
                "algorithmic_flop_per_launch": p.flops}

    sec = None if args.no_secondary else secondary(torch, dev, 20)
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
