"""Benchmark: dense row-major GEMM on one MI355X.

A step is one gemm_f32 call, C = 1.5*A*B + 0.5*C at M = N = K = 4096 (fp32,
operands ~ U[-1,1), already resident in HBM).  The JSON line reports its
TFLOP/s (2*M*N*K per step), the kernel's fraction of the fp32 matrix-core
peak, every workload of the scope table timed the same way (median, min and
max of single launches as well), and the CPU oracle timed on bounded samples.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
  python bench.py --profile-case NAME [--launches N]
                                   (30 warm-up + N launches of one workload, for rocprofv3)
  python bench.py --copy-probe     (plain 256 MiB copies: FETCH/WRITE_SIZE calibration)
  python bench.py --summarize-profiles DIR   (profiles/ summaries from rocprofv3 CSVs)

Profiling recipe (DIR under gpurun_out/, one rocprofv3 run per counter set):
  for NAME in the workloads:
    rocprofv3 --kernel-trace --stats --output-format csv -d DIR/NAME/trace -o run -- python3 bench.py --profile-case NAME
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/NAME/fetch -o run -- python3 bench.py --profile-case NAME --launches 5
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/NAME/write -o run -- python3 bench.py --profile-case NAME --launches 5
    rocprofv3 --pmc <UTIL_COUNTERS with the dtype's MOPS counter> --output-format csv -d DIR/NAME/util -o run -- python3 bench.py --profile-case NAME --launches 5
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copy/fetch -o run -- python3 bench.py --copy-probe
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/copy/write -o run -- python3 bench.py --copy-probe
  python3 bench.py --summarize-profiles DIR

HBM traffic per launch comes from those FETCH_SIZE / WRITE_SIZE summaries; it
is reported only while the kernel's sources still hash to the value recorded
with the counters.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6,     # MI355X dense matrix peaks
               "i8": 5000.0, "f64": 78.6}                        # (int8: TOP/s)
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 256 << 20
PRIMARY = "sgemm_4096"
CASES = ("sgemm_256", "sgemm_4096", "sgemm_ragged", "sgemm_ragged_splitk", "sgemm_ragged_streamk",
         "gemm_bf16_8192",
         "gemm_f16_8192", "qkt_batched", "qkt_batched_f16_out", "gemm_i8_8192", "dgemm_4096")
HBM_BOUND = ("qkt_batched", "qkt_batched_f16_out")
GRAPH_CASES = ("sgemm_256", "sgemm_ragged_splitk", "sgemm_ragged_streamk")  # also timed from a HIP graph
MOPS_COUNTER = {"f32": "SQ_INSTS_VALU_MFMA_MOPS_F32", "f16": "SQ_INSTS_VALU_MFMA_MOPS_F16",
                "bf16": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "i8": "SQ_INSTS_VALU_MFMA_MOPS_I8",
                "f64": "SQ_INSTS_VALU_MFMA_MOPS_F64"}
UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                 "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_SIMD = 256 * 4
N_XCD = 8
PROFILE_WARMUP = 30   # launches before the profiled ones, as in the timed bench


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------- profiles

def kernel_source_sha(dtype):
    """sha256 over the sources one dtype's kernels are built from."""
    csrc = os.path.join(ROOT, "dense_gemm_f32_amd", "csrc")
    h = hashlib.sha256()
    names = ("gemm_kernel.hpp", "variants.hpp", "kernels_%s.hip" % dtype)
    if dtype == "f64":
        names += ("gemm_f64.hpp",)
    for name in names:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()


def summary_path(kernel, case):
    return os.path.join(PROFILES, "%s__%s.txt" % (kernel, case))


def read_summary(path):
    vals = {}
    if os.path.exists(path):
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
    return vals


def stored_traffic(kernel, case, dtype):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the
    profile summary, or None when there is none or the sources changed since."""
    vals = read_summary(summary_path(kernel, case))
    if vals.get("source_sha256") != kernel_source_sha(dtype) or vals.get("kernel") != kernel:
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(directory, pattern):
    out = []
    for fn in glob.glob(os.path.join(directory, "**", pattern), recursive=True):
        with open(fn) as f:
            out += list(csv.DictReader(f))
    return out


def _counters(directory, name_filter):
    """{counter: [value per dispatch]} and the dispatch durations (ns) of matching kernels."""
    vals, durs = {}, {}
    for r in _csv_rows(directory, "*counter_collection.csv"):
        if name_filter not in r["Kernel_Name"]:
            continue
        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        durs[r.get("Dispatch_Id", len(durs))] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return vals, list(durs.values())


def _mean(xs):
    return sum(xs) / len(xs) if xs else None


def _dispatch_durations(directory, name_filter):
    rows = [r for r in _csv_rows(directory, "*kernel_trace.csv") if name_filter in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def _fmt(x, spec="%.4g"):
    return "n/a" if x is None else spec % x


def summarize_case(case, d, copy_dir):
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import workloads as wl
    p = wl.WORKLOADS[case]()
    info, grid = select_for(mg, p)
    kname = info["name"]
    # demangled for fp32; 16-bit instances stay mangled
    filt = ("gemm_f64_kernel" if p.dtype == "f64" else
            "gemm_sk_kernel" if p.streamk is not None else "gemm_kernel")
    durs = _dispatch_durations(os.path.join(d, "trace"), filt)
    timed = durs[PROFILE_WARMUP:] if len(durs) > PROFILE_WARMUP else durs  # after the warm-up
    fetch_v, _ = _counters(os.path.join(d, "fetch"), filt)
    write_v, _ = _counters(os.path.join(d, "write"), filt)
    util_v, util_d = _counters(os.path.join(d, "util"), filt)
    cf = _mean(_counters(os.path.join(copy_dir, "fetch"), "copyBuffer")[0].get("FETCH_SIZE", []))
    cw = _mean(_counters(os.path.join(copy_dir, "write"), "copyBuffer")[0].get("WRITE_SIZE", []))
    fetch = _mean(fetch_v.get("FETCH_SIZE", []))
    write = _mean(write_v.get("WRITE_SIZE", []))
    expect_kib = COPY_PROBE_BYTES / 1024.0
    sf = expect_kib / cf if cf else None
    sw = expect_kib / cw if cw else None
    traffic = (int(round((fetch * sf + write * sw) * 1024))
               if None not in (fetch, write, sf, sw) else None)
    algo = algorithmic_bytes(p)
    avg = _mean(timed)
    gui = _mean(util_v.get("GRBM_GUI_ACTIVE", []))
    udur = _mean(util_d)
    # counters span more than the kernel itself: only long kernels give a clock
    clock = gui / N_XCD / udur if gui and udur and udur > 200e3 else None
    mfma = _mean(util_v.get("SQ_VALU_MFMA_BUSY_CYCLES", []))
    mfma_frac = mfma / (gui / N_XCD) / N_SIMD if mfma and gui else None
    bank = _mean(util_v.get("SQ_LDS_BANK_CONFLICT", []))
    lds = _mean(util_v.get("SQ_LDS_IDX_ACTIVE", []))
    mops = _mean(util_v.get(MOPS_COUNTER[p.dtype], []))
    tflops = p.flops / (avg * 1e-9) / 1e12 if avg else None
    dt = p.dtype
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d DIR/{c}/trace -o run -- "
           "python3 bench.py --profile-case {c};  "
           "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/{c}/fetch -o run -- "
           "python3 bench.py --profile-case {c} --launches 5;  "
           "rocprofv3 --pmc WRITE_SIZE (same, -d DIR/{c}/write);  "
           "rocprofv3 --pmc {u} (same, -d DIR/{c}/util);  "
           "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE --output-format csv -d DIR/copy/fetch, "
           "DIR/copy/write -o run -- python3 bench.py --copy-probe;  "
           "python3 bench.py --summarize-profiles DIR").format(
               c=case, u=" ".join(UTIL_COUNTERS[:4] + (MOPS_COUNTER[dt],) + UTIL_COUNTERS[4:]))
    lines = [
        "# rocprofv3 summary: %s, %s M=%d N=%d K=%d batch=%d transA=%d transB=%d alpha=%g beta=%g"
        % (case, dt, p.M, p.N, p.K, p.batch, p.transA, p.transB, p.alpha, p.beta),
        "command: " + cmd,
        "workload: " + case,
        "kernel: " + kname,
        "grid: %d" % grid,
        "source_sha256: " + kernel_source_sha(dt),
        "dispatches_traced: %d" % len(durs),
        "average_ns_timed_launches: " + _fmt(avg, "%.0f"),
        "median_ns: " + _fmt(statistics.median(timed) if timed else None, "%.0f"),
        "min_ns: " + _fmt(min(timed) if timed else None, "%.0f"),
        "max_ns: " + _fmt(max(timed) if timed else None, "%.0f"),
        "tflops_at_average: " + _fmt(tflops, "%.2f"),
        "frac_matrix_peak: " + _fmt(tflops / PEAK_TFLOPS[dt] if tflops else None, "%.4f"),
    ]
    if p.splitk is not None:   # the chunk products above, then one reduction kernel
        red = _dispatch_durations(os.path.join(d, "trace"), "splitk_reduce")
        red = red[PROFILE_WARMUP:] if len(red) > PROFILE_WARMUP else red
        ravg = _mean(red)
        both = p.flops / ((avg + ravg) * 1e-9) / 1e12 if avg and ravg else None
        plan = mg.splitk_plan(dt, p.M, p.N, p.K, p.splitk, transA=int(p.transA),
                              transB=int(p.transB), lda=p.lda, ldb=p.ldb)
        lines += ["splitk_chunks: %d of %d" % (plan["chunks"], plan["chunk_len"]),
                  "reduce_kernel_average_ns: " + _fmt(ravg, "%.0f"),
                  "tflops_both_kernels: " + _fmt(both, "%.2f")]
    if p.streamk is not None:   # the stream-K launch above, then the fix-up of split tiles
        fix = _dispatch_durations(os.path.join(d, "trace"), "sk_fixup")
        fix = fix[PROFILE_WARMUP:] if len(fix) > PROFILE_WARMUP else fix
        favg = _mean(fix)
        both = p.flops / ((avg + favg) * 1e-9) / 1e12 if avg and favg else None
        plan = mg.streamk_plan(dt, p.M, p.N, p.K, p.streamk, transA=int(p.transA),
                               transB=int(p.transB), lda=p.lda, ldb=p.ldb)
        lines += ["streamk: %d workgroups over %d tiles of %d iterations of %d" %
                  (plan["workgroups"], plan["tiles"], plan["iterations"], plan["k_per_iteration"]),
                  "fixup_kernel_average_ns: " + _fmt(favg, "%.0f"),
                  "tflops_both_kernels: " + _fmt(both, "%.2f")]
    if case in HBM_BOUND and avg:
        gbs = algo / (avg * 1e-9) / 1e9
        lines += ["algorithmic_gbs_at_average: %.1f" % gbs,
                  "frac_hbm_peak: %.4f" % (gbs / PEAK_HBM_GBS)]
    lines += [
        "clock_ghz_counter_run: " + _fmt(clock, "%.3f"),
        "mfma_busy_frac_counter_run: " + _fmt(mfma_frac, "%.4f"),
        "%s_per_dispatch: %s" % (MOPS_COUNTER[dt], _fmt(mops, "%.6g")),
        "flop_per_mop: " + _fmt(p.flops / mops if mops else None, "%.1f"),
        "lds_bank_conflict_cycles_over_lds_active: " +
        _fmt(bank / lds if lds else (0.0 if bank == 0 else None), "%.4f"),
        "FETCH_SIZE_KiB_per_dispatch: " + _fmt(fetch, "%.1f"),
        "WRITE_SIZE_KiB_per_dispatch: " + _fmt(write, "%.1f"),
        "copy_probe_bytes: %d" % COPY_PROBE_BYTES,
        "copy_FETCH_SIZE_KiB: " + _fmt(cf, "%.1f"),
        "copy_WRITE_SIZE_KiB: " + _fmt(cw, "%.1f"),
        "fetch_scale: " + _fmt(sf, "%.4f"),
        "write_scale: " + _fmt(sw, "%.4f"),
        "traffic_bytes_per_launch: " + _fmt(traffic, "%d"),
        "algorithmic_bytes_per_launch: %d" % algo,
        "traffic_over_algorithmic: " + _fmt(traffic / algo if traffic else None, "%.3f"),
    ]
    os.makedirs(PROFILES, exist_ok=True)
    path = summary_path(kname, case)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines) + "\n", flush=True)
    return path


def summarize_profiles(d):
    copy_dir = os.path.join(d, "copy")
    for case in CASES:
        if os.path.isdir(os.path.join(d, case)):
            summarize_case(case, os.path.join(d, case), copy_dir)


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


# ---------------------------------------------------------------------------- timing

def select_for(mg, p, ptrs=(1 << 20, 1 << 20, 1 << 20)):
    """(variant info, grid) of the GEMM kernel a workload launches (for split-K: the
    partial-product kernel; for stream-K: the stream-K kernel)."""
    if p.streamk is not None:
        plan = mg.streamk_plan(p.dtype, p.M, p.N, p.K, p.streamk, transA=int(p.transA),
                               transB=int(p.transB), A=ptrs[0], lda=p.lda, B=ptrs[1], ldb=p.ldb)
        return plan["variant"], plan["workgroups"]
    if p.splitk is not None:
        plan = mg.splitk_plan(p.dtype, p.M, p.N, p.K, p.splitk, transA=int(p.transA),
                              transB=int(p.transB), A=ptrs[0], lda=p.lda, B=ptrs[1], ldb=p.ldb)
        return plan["variant"], plan["grid"]
    return mg.select(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, ptrs[0],
                     p.lda, p.strideA, ptrs[1], p.ldb, p.strideB, p.beta, ptrs[2], p.ldc,
                     p.strideC, p.batch, c_dtype=p.c_dtype)


def make_device_problem(p, torch, dev):
    from dense_gemm_f32_amd import workloads as wl
    A, B, C0 = wl.make_inputs(p)
    dA, dB = A.to(dev), B.to(dev)
    dC = (C0.to(dev) if C0 is not None
          else torch.zeros(p.c_elems, dtype=wl.TORCH_DTYPE[p.c_dtype], device=dev))
    return dA, dB, dC


def launcher(p, dA, dB, dC):
    import dense_gemm_f32_amd as mg
    if p.streamk is not None:
        import torch
        need = mg.streamk_plan(p.dtype, p.M, p.N, p.K, p.streamk, transA=int(p.transA),
                               transB=int(p.transB), A=dA, lda=p.lda, B=dB, ldb=p.ldb)["workspace_bytes"]
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dA.device)  # outside the timing
        return lambda: mg.gemm_streamk(p.dtype, p.c_dtype, int(p.transA), int(p.transB), p.M, p.N,
                                       p.K, p.alpha, dA, p.lda, dB, p.ldb, p.beta, dC, p.ldc,
                                       workgroups=p.streamk, workspace=ws)
    if p.splitk is not None:
        import torch
        need = mg.splitk_workspace_bytes(p.dtype, p.M, p.N, p.K, p.splitk, transA=int(p.transA),
                                         transB=int(p.transB), A=dA, lda=p.lda, B=dB, ldb=p.ldb)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dA.device)  # outside the timing
        return lambda: mg.gemm_splitk(p.dtype, p.c_dtype, int(p.transA), int(p.transB), p.M, p.N,
                                      p.K, p.alpha, dA, p.lda, dB, p.ldb, p.beta, dC, p.ldc,
                                      splits=p.splitk, workspace=ws)
    if p.dtype == "f64":
        if p.batch == 1:
            return lambda: mg.gemm_f64(int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, dA,
                                       p.lda, dB, p.ldb, p.beta, dC, p.ldc)
        return lambda: mg.gemm_f64_strided_batched(int(p.transA), int(p.transB), p.M, p.N, p.K,
                                                   p.alpha, dA, p.lda, p.strideA, dB, p.ldb,
                                                   p.strideB, p.beta, dC, p.ldc, p.strideC,
                                                   p.batch)
    if p.c_dtype != "f32":
        return lambda: mg.gemm_strided_batched_ex(p.dtype, p.c_dtype, int(p.transA), int(p.transB),
                                                  p.M, p.N, p.K, p.alpha, dA, p.lda, p.strideA, dB,
                                                  p.ldb, p.strideB, p.beta, dC, p.ldc, p.strideC,
                                                  p.batch)
    if p.batch == 1:
        fn = {"f32": mg.gemm_f32, "f16": mg.gemm_f16, "bf16": mg.gemm_bf16}[p.dtype]
        return lambda: fn(int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, dA, p.lda, dB,
                          p.ldb, p.beta, dC, p.ldc)
    return lambda: mg.gemm_strided_batched(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K,
                                           p.alpha, dA, p.lda, p.strideA, dB, p.ldb, p.strideB,
                                           p.beta, dC, p.ldc, p.strideC, p.batch)


def time_kernel(torch, fn, iters):
    """Average duration of one launch over back-to-back launches, from HIP events
    recorded on the stream the library launches on (the current torch stream)."""
    s = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(iters):
        fn()
    stop.record(s)
    stop.synchronize()
    return start.elapsed_time(stop) / iters * 1e-3


def time_each(torch, fn, iters, between=None):
    """Durations (s) of single launches, each bracketed by its own event pair;
    `between` runs before each launch, outside the bracket."""
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        if between is not None:
            between()
        e0.record(s)
        fn()
        e1.record(s)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs]


def time_graph(torch, fn, calls=20, replays=10):
    """Per-call time of `calls` library calls captured into one HIP graph (torch's graph
    capture records the kernels the calls enqueue) and replayed `replays` times."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(calls):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(replays):
        g.replay()
    stop.record(s)
    stop.synchronize()
    return start.elapsed_time(stop) / (calls * replays) * 1e-3


def algorithmic_bytes(p):
    """Compulsory HBM traffic: A and B once, C written (and read when beta != 0)."""
    from dense_gemm_f32_amd import workloads as wl
    es, ces = wl.ELEM_SIZE[p.dtype], wl.ELEM_SIZE[p.c_dtype]
    per = (p.M * p.K + p.K * p.N) * es + p.M * p.N * ces * (2 if p.beta != 0 else 1)
    return per * p.batch


def per_config(torch, dev, iters):
    """Every workload: 30 warm-up launches (the part settles at its power-limited
    clock), then `iters` back-to-back launches (mean) and `iters` single
    launches (median / min / max).  The fp32 4096^3 step is also timed with a
    cold cache: 512 MiB written between launches, outside the timed bracket."""
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import workloads as wl
    out = {}
    for name in CASES:
        p = wl.WORKLOADS[name]()
        dA, dB, dC = make_device_problem(p, torch, dev)
        fn = launcher(p, dA, dB, dC)
        for _ in range(30):
            fn()
        torch.cuda.synchronize()
        t = time_kernel(torch, fn, iters)
        each = time_each(torch, fn, iters)
        info, grid = select_for(mg, p, (dA.data_ptr(), dB.data_ptr(), dC.data_ptr()))
        tf = p.flops / t / 1e12
        rec = {"dtype": p.dtype, "c_dtype": p.c_dtype, "M": p.M, "N": p.N, "K": p.K, "batch": p.batch,
               "transA": int(p.transA), "transB": int(p.transB), "alpha": p.alpha,
               "beta": p.beta, "kernel": info["name"], "grid": grid,
               "ms": round(t * 1e3, 4), "median_ms": round(statistics.median(each) * 1e3, 4),
               "min_ms": round(min(each) * 1e3, 4), "max_ms": round(max(each) * 1e3, 4),
               "tflops": round(tf, 2), "frac_matrix_peak": round(tf / PEAK_TFLOPS[p.dtype], 4),
               "bound": "hbm" if name in HBM_BOUND else "mfma",
               "traffic": stored_traffic(info["name"], name, p.dtype),
               "algorithmic_bytes": algorithmic_bytes(p)}
        if name in HBM_BOUND:
            gbs = algorithmic_bytes(p) / t / 1e9
            rec["hbm_gbs"] = round(gbs, 1)
            rec["frac_hbm_peak"] = round(gbs / PEAK_HBM_GBS, 4)
        if name in GRAPH_CASES:
            tg = time_graph(torch, fn)
            rec["graph_ms"] = round(tg * 1e3, 4)
            rec["graph_tflops"] = round(p.flops / tg / 1e12, 2)
        if name == PRIMARY:
            scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
            cold = time_each(torch, fn, 10, between=lambda: scratch.fill_(1))
            cm = statistics.median(cold)
            rec["cold_cache_median_ms"] = round(cm * 1e3, 4)
            rec["cold_cache_tflops"] = round(p.flops / cm / 1e12, 2)
            del scratch
        out[name] = rec
        log(f"{name}: {rec}")
        del dA, dB, dC
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------- CPU oracle

def _oracle_rate(p, rows=None, batches=None):
    """(seconds, flop) of the oracle on the first `rows` output rows (or the first
    `batches` batch entries) of workload p."""
    import oracle
    from dense_gemm_f32_amd import workloads as wl
    A, B, C0 = wl.make_inputs(p)
    An, Bn = wl.to_numpy_operand(A), wl.to_numpy_operand(B)
    Cn = C0.numpy() if C0 is not None else None
    if batches is not None:
        t0 = time.perf_counter()
        oracle.gemm(p.dtype, p.transA, p.transB, p.M, p.N, p.K, p.alpha, An, p.lda, Bn, p.ldb,
                    p.beta, Cn, p.ldc, batch=batches, strideA=p.strideA, strideB=p.strideB,
                    strideC=p.strideC)
        return time.perf_counter() - t0, 2.0 * p.M * p.N * p.K * batches
    r = p.M if rows is None else min(rows, p.M)
    a_part = An if p.transA else An[:r * p.lda]
    t0 = time.perf_counter()
    oracle.gemm(p.dtype, p.transA, p.transB, r, p.N, p.K, p.alpha, a_part, p.lda, Bn, p.ldb,
                p.beta, None if Cn is None else Cn[:r * p.ldc], p.ldc)
    return time.perf_counter() - t0, 2.0 * r * p.N * p.K


def cpu_baseline(budget_s=15.0):
    """The oracle, as it stands, on the host cores: the bench workload on its first
    R output rows (R sized for about `budget_s`), and every other workload on a
    bounded sample (single-threaded as well for the two small fp32 ones)."""
    import oracle
    from dense_gemm_f32_amd import workloads as wl
    oracle.build(force=False)
    threads = oracle.max_threads()
    p = wl.WORKLOADS[PRIMARY]()
    t, _ = _oracle_rate(p, rows=threads)
    r2 = int(min(p.M, max(threads, threads * budget_s / max(t, 1e-6))))
    r2 = max(threads, (r2 // threads) * threads)
    t2, flop = _oracle_rate(p, rows=r2)
    res = {"value": flop / t2 / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"first {r2} of {p.M} output rows of the same {p.M}x{p.N}x{p.K} fp32 GEMM "
                     f"({flop / 1e9:.1f} GFLOP, fp64 accumulation, {t2:.1f} s)"}
    samples = {"sgemm_256": {}, "sgemm_ragged": {}, "gemm_bf16_8192": {"rows": threads},
               "gemm_f16_8192": {"rows": threads}, "qkt_batched": {"batches": 2},
               "qkt_batched_f16_out": {"batches": 2}, "gemm_i8_8192": {"rows": threads},
               "dgemm_4096": {"rows": threads}}
    per = {}
    for name, kw in samples.items():
        q = wl.WORKLOADS[name]()
        s, f = _oracle_rate(q, **kw)
        what = (f"first {kw['rows']} rows" if "rows" in kw else
                f"first {kw['batches']} of {q.batch} batch entries" if "batches" in kw else "whole")
        per[name] = {"gflops": round(f / s / 1e9, 3), "seconds": round(s, 3), "threads": threads,
                     "sample": what, "est_full_seconds": round(s * q.flops / f, 3)}
    oracle.set_threads(1)
    try:
        for name, rows in (("sgemm_256", None), ("sgemm_ragged", 64)):
            q = wl.WORKLOADS[name]()
            s, f = _oracle_rate(q, rows=rows)
            per[name + "_1thread"] = {"gflops": round(f / s / 1e9, 3), "seconds": round(s, 3),
                                      "threads": 1,
                                      "sample": "whole" if rows is None else f"first {rows} rows",
                                      "est_full_seconds": round(s * q.flops / f, 3)}
    finally:
        oracle.set_threads(threads)
    res["per_config"] = per
    return res


# ---------------------------------------------------------------------------- main

def profile_case(name, launches, warmup):
    """Warm-up then timed launches of one workload (run under rocprofv3)."""
    import torch
    from dense_gemm_f32_amd import workloads as wl
    dev = torch.device("cuda:0")
    p = wl.WORKLOADS[name]()
    dA, dB, dC = make_device_problem(p, torch, dev)
    fn = launcher(p, dA, dB, dC)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    print(f"profile case {name}: {warmup} + {launches} launches done", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize-profiles", metavar="DIR")
    ap.add_argument("--profile-case", metavar="NAME", choices=CASES)
    ap.add_argument("--launches", type=int, default=20)
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.profile_case:
        profile_case(args.profile_case, args.launches,
                     PROFILE_WARMUP if args.warmup is None else args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); a GEMM shards by "
              "rows or batch entries with no exchange, so the one-GPU rate is the figure.",
              file=sys.stderr)
        sys.exit(2)
    # The part raises its clock over the first ~25 ms of this load (a kernel
    # trace shows the launch time fall from 1.12 to 0.96 ms over the first 25
    # launches): 50 untimed steps reach the steady state.
    warmup = 50 if args.warmup is None else args.warmup

    import torch
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import workloads as wl

    dev = torch.device("cuda:0")
    p = wl.WORKLOADS[PRIMARY]()
    A, B, C0 = wl.make_inputs(p)
    dA, dB, dC = A.to(dev), B.to(dev), C0.to(dev)
    step = launcher(p, dA, dB, dC)
    info, grid = select_for(mg, p, (dA.data_ptr(), dB.data_ptr(), dC.data_ptr()))
    log(f"workload sgemm 4096^3 alpha=1.5 beta=0.5: kernel {info['name']} grid {grid}")

    for _ in range(warmup):
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
                "traffic": stored_traffic(info["name"], PRIMARY, p.dtype),
                "kernel": info["name"], "kernel_ms": round(t_kernel * 1e3, 4),
                "algorithmic_flop_per_launch": p.flops,
                "algorithmic_bytes_per_launch": algorithmic_bytes(p)}
    del dA, dB, dC
    torch.cuda.empty_cache()

    per = None if args.no_secondary else per_config(torch, dev, 30)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline()
        log(f"cpu_baseline: {cpu}")

    line = {
        "metric": "GEMM TFLOP/s + % of MI355X matrix peak (fp32 4096^3, bf16 8192^3)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
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
        "per_config": per,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
