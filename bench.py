"""Benchmark: dense row-major GEMM on one MI355X.

A step is one gemm_f32 call, C = 1.5*A*B + 0.5*C at M = N = K = 4096 (fp32,
operands ~ U[-1,1), already resident in HBM).  The JSON line reports its
TFLOP/s (2*M*N*K per step), the kernel's fraction of the fp32 matrix-core
peak, every workload of the scope table timed the same way (median, min and
max of single launches as well) with its sustained clock and socket power and
a parity check of one fresh launch against the oracle on sampled elements
(max|err|, tolerance, bit-exactness; run in the CPU leg, outside every timed
region), the register-only 16-bit matrix-core rate on N(0,1) data (the
power-limited ceiling on this board), and the CPU oracle timed on bounded
samples.

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
    if dtype == "f32":
        names += ("gemm_small.hpp",)
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
            "gemm_sk_kernel" if p.streamk is not None else
            "gemm_small_kernel" if info["pipe"] == 6 else "gemm_kernel")
    durs = _dispatch_durations(os.path.join(d, "trace"), filt)
    timed = durs[PROFILE_WARMUP:] if len(durs) > PROFILE_WARMUP else durs  # after the warm-up
    fetch_v, _ = _counters(os.path.join(d, "fetch"), filt)
    write_v, _ = _counters(os.path.join(d, "write"), filt)
    util_v, util_d = _counters(os.path.join(d, "util"), filt)
    cf = _mean(_counters(os.path.join(copy_dir, "fetch"), "copyBuffer")[0].get("FETCH_SIZE", []))
    cw = _mean(_counters(os.path.join(copy_dir, "write"), "copyBuffer")[0].get("WRITE_SIZE", []))
    # read-only calibration: a reduction over the same number of bytes (its FETCH_SIZE
    # should take the copy's scale if the counter's unit is the same for plain reads)
    rf = _mean(_counters(os.path.join(copy_dir, "read"), "reduce")[0].get("FETCH_SIZE", []))
    floor, floor_rounds = xcd_fetch_floor(p, info, grid)
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
           "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copy/read -o run -- "
           "python3 bench.py --read-probe;  "
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
    if p.streamk is not None:   # one launch: split tiles are completed by their last contributor
        plan = mg.streamk_plan(dt, p.M, p.N, p.K, p.streamk, transA=int(p.transA),
                               transB=int(p.transB), lda=p.lda, ldb=p.ldb)
        lines += ["streamk: %d workgroups over %d tiles of %d iterations of %d" %
                  (plan["workgroups"], plan["tiles"], plan["iterations"], plan["k_per_iteration"])]
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
        "read_probe_FETCH_SIZE_KiB: " + _fmt(rf, "%.1f"),
        "fetch_scale: " + _fmt(sf, "%.4f"),
        "fetch_scale_read_probe: " + _fmt(expect_kib / rf if rf else None, "%.4f"),
        "write_scale: " + _fmt(sw, "%.4f"),
        "traffic_bytes_per_launch: " + _fmt(traffic, "%d"),
        "algorithmic_bytes_per_launch: %d" % algo,
        "traffic_over_algorithmic: " + _fmt(traffic / algo if traffic else None, "%.3f"),
        "fetch_bytes_per_launch: " + _fmt(fetch * sf * 1024 if fetch and sf else None, "%d"),
        "xcd_fetch_floor_bytes: " + _fmt(floor, "%d"),
        "xcd_round_fetch_bytes: " + _fmt(floor_rounds, "%d"),
        "fetch_over_xcd_floor: " + _fmt(fetch * sf * 1024 / floor if fetch and sf and floor else None, "%.3f"),
        "fetch_over_xcd_rounds: " + _fmt(fetch * sf * 1024 / floor_rounds
                                         if fetch and sf and floor_rounds else None, "%.3f"),
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


def read_probe():
    """A device reduction over COPY_PROBE_BYTES (reads them once, writes a few bytes):
    the read-only calibration of FETCH_SIZE beside the copy."""
    import torch
    x = torch.ones(COPY_PROBE_BYTES // 4, device="cuda:0")
    for _ in range(5):
        y = x.sum()
    torch.cuda.synchronize()
    assert float(y) == COPY_PROBE_BYTES // 4
    print("read probe done", flush=True)


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
        # zero-filled once: the arrival counters at its start; every call leaves them zero
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dA.device)  # outside the timing
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


class Telemetry:
    """GPU clock (mean over the XCDs) and socket power from the SMU's metrics
    table through amdsmi.  The table refreshes about once a second (measured),
    so readings come from a sustained run of a few seconds, after its first
    second.  Without amdsmi every reading is None."""

    def __init__(self):
        self.h = None
        self.error = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # no amdsmi, no permission: no readings
            self.error = repr(e)

    def read(self):
        if self.h is None:
            return None
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
            clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float)) and c > 0]
            clk = statistics.mean(clks) if clks else m.get("current_gfxclk")
            pw = m.get("current_socket_power")
            return (float(clk) if isinstance(clk, (int, float)) else None,
                    float(pw) if isinstance(pw, (int, float)) else None)
        except Exception:
            return None

    def sustained(self, torch, fn, launch_s, seconds=2.5, settle=1.2):
        """Run fn back to back for about `seconds`, sampling every 20 ms; the
        medians of the samples taken after `settle` seconds (the table has
        refreshed at least once under the load)."""
        if self.h is None:
            return None
        import threading
        samples, stop = [], threading.Event()
        t_start = time.perf_counter()

        def poll():
            while not stop.is_set():
                r = self.read()
                if r is not None and time.perf_counter() - t_start >= settle:
                    samples.append(r)
                time.sleep(0.02)

        th = threading.Thread(target=poll)
        th.start()
        batch = max(1, int(0.02 / max(launch_s, 1e-7)))
        t0 = time.perf_counter()
        try:
            while time.perf_counter() - t0 < seconds:
                for _ in range(batch):
                    fn()
                torch.cuda.synchronize()
        finally:
            stop.set()
            th.join()
        clks = [c for c, _ in samples if c is not None]
        pws = [w for _, w in samples if w is not None]
        return {"clock_mhz": round(statistics.median(clks)) if clks else None,
                "socket_power_w": round(statistics.median(pws)) if pws else None,
                "window_s": seconds, "readings": len(set(samples))}


def mfma_ceiling(torch, dev, tel):
    """Register-only matrix-core rate (libmgemm_diag.so) on the operand values of the
    workloads: N(0,1) rounded to bf16 and to binary16, and int8 uniform in -128..127.
    The power-limited ceiling no GEMM of that type on this board and data can exceed.
    None when the diagnostic library is not built."""
    import ctypes
    path = os.path.join(ROOT, "dense_gemm_f32_amd", "libmgemm_diag.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mgemm_diag_mfma_ceiling.restype = ctypes.c_int
    lib.mgemm_diag_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p]
    lib.mgemm_diag_ceiling_operand_bytes.restype = ctypes.c_int64
    lib.mgemm_diag_ceiling_out_floats.restype = ctypes.c_int64
    lib.mgemm_diag_ceiling_ops.restype = ctypes.c_double
    lib.mgemm_diag_ceiling_ops.argtypes = [ctypes.c_int, ctypes.c_int]
    nbytes = lib.mgemm_diag_ceiling_operand_bytes()
    out = torch.empty(lib.mgemm_diag_ceiling_out_floats(), dtype=torch.float32, device=dev)
    iters = 40000
    res = {}
    for name, kind in (("bf16", 1), ("f16", 0), ("i8", 2)):   # MGEMM_DIAG_* in mgemm_diag.h
        g = torch.Generator().manual_seed(1004)
        if name == "i8":
            ops = torch.randint(-128, 128, (nbytes,), generator=g, dtype=torch.int8).to(dev)
            data = "int8 uniform in -128..127"
        else:
            ops = torch.randn(nbytes // 2, generator=g).to(wl_dtype(torch, name)).to(dev)
            data = "N(0,1) rounded to %s" % name
        st = torch.cuda.current_stream()
        fn = lambda: lib.mgemm_diag_mfma_ceiling(kind, ops.data_ptr(), out.data_ptr(),
                                                 iters, ctypes.c_void_p(st.cuda_stream))
        for _ in range(3):
            assert fn() == 0
        each = time_each(torch, fn, 5)
        t = statistics.median(each)
        tf = lib.mgemm_diag_ceiling_ops(kind, iters) / t / 1e12
        rec = {"tflops": round(tf, 1), "frac_matrix_peak": round(tf / PEAK_TFLOPS[name], 4),
               "data": data, "ms": round(t * 1e3, 3)}
        tel_r = tel.sustained(torch, fn, t) if tel else None
        if tel_r:
            rec.update(tel_r)
        res[name] = rec
        log(f"mfma ceiling {name}: {rec}")
        del ops
    return res


def wl_dtype(torch, name):
    return {"bf16": torch.bfloat16, "f16": torch.float16}[name]


def sample_positions(p, n_random=4096, seed=7):
    """Output elements the parity check compares: the first and last row and
    column of the first and last batch entry, and random ones."""
    import numpy as np
    rng = np.random.default_rng(seed)
    bs, is_, js = [], [], []
    for b in sorted({0, p.batch - 1}):
        for i in sorted({0, p.M - 1}):
            bs.append(np.full(p.N, b)); is_.append(np.full(p.N, i)); js.append(np.arange(p.N))
        for j in sorted({0, p.N - 1}):
            bs.append(np.full(p.M, b)); is_.append(np.arange(p.M)); js.append(np.full(p.M, j))
    bs.append(rng.integers(0, p.batch, n_random))
    is_.append(rng.integers(0, p.M, n_random))
    js.append(rng.integers(0, p.N, n_random))
    return np.concatenate(bs), np.concatenate(is_), np.concatenate(js)


def gather_c(torch, p, dC, pos):
    """C's sampled elements (float64 on the host) after a launch."""
    b, i, j = pos
    idx = torch.as_tensor(b * p.strideC + i * p.ldc + j, dtype=torch.int64, device=dC.device)
    return dC[idx].double().cpu().numpy()


def algorithmic_bytes(p):
    """Compulsory HBM traffic: A and B once, C written (and read when beta != 0)."""
    from dense_gemm_f32_amd import workloads as wl
    es, ces = wl.ELEM_SIZE[p.dtype], wl.ELEM_SIZE[p.c_dtype]
    per = (p.M * p.K + p.K * p.N) * es + p.M * p.N * ces * (2 if p.beta != 0 else 1)
    return per * p.batch


def xcd_fetch_floor(p, info, grid):
    """Operand bytes a plain launch must fetch from memory, two ways; (None, None) for
    split-K and stream-K launches.  Each of the 8 XCDs has its own L2.  The kernels'
    assignment: workgroup w runs on XCD w % 8, the ids are remapped to one contiguous range
    of logical ids per XCD, and logical ids walk the tiles in groups of min(8, tile rows)
    tile rows.
      once: every A row panel and B column panel that the tiles on one XCD use, once per
            XCD (a lower bound whatever the L2 holds);
      rounds: the same per round of workgroups running together on an XCD (its 32 CUs
            times the workgroups per CU that LDS allows), panels not kept from one round
            to the next (an L2 too small for a round's panels).
    C is added to both when it is read (beta != 0)."""
    from dense_gemm_f32_amd import workloads as wl
    if p.streamk is not None or p.splitk is not None or grid <= 0:
        return None, None
    bm, bn = info["block_m"], info["block_n"]
    es = wl.ELEM_SIZE[p.dtype]
    tiles_m, tiles_n = -(-p.M // bm), -(-p.N // bn)
    group_m = max(1, min(tiles_m, 8))
    per_b = tiles_m * tiles_n
    per_cu = max(1, min(8, (160 << 10) // max(info["lds_bytes"], 1)))
    round_size = 32 * per_cu
    q, rem = grid // N_XCD, grid % N_XCD

    def panels(ids):
        a_pan, b_pan = set(), set()
        for L in ids:
            b = L // per_b
            t = L - b * per_b
            width = group_m * tiles_n
            g = t // width
            first = g * group_m
            gsz = min(tiles_m - first, group_m)
            w2 = t - g * width
            a_pan.add((b if p.strideA else 0, first + w2 % gsz))
            b_pan.add((b if p.strideB else 0, w2 // gsz))
        return (sum(min(bm, p.M - tm * bm) for _, tm in a_pan) * p.K * es +
                sum(min(bn, p.N - tn * bn) for _, tn in b_pan) * p.K * es)

    once = rounds = 0
    for x in range(N_XCD):
        start = x * q + min(x, rem)
        ids = range(start, start + q + (1 if x < rem else 0))
        once += panels(ids)
        rounds += sum(panels(ids[i:i + round_size]) for i in range(0, len(ids), round_size))
    c_read = p.M * p.N * wl.ELEM_SIZE[p.c_dtype] * p.batch if p.beta != 0 else 0
    return once + c_read, rounds + c_read


def per_config(torch, dev, iters, tel=None, checks=None):
    """Every workload: 30 warm-up launches (the part settles at its power-limited
    clock), then `iters` back-to-back launches (mean) and `iters` single
    launches (median / min / max), then 2.5 s of back-to-back launches with the
    clock and socket power sampled.  The fp32 4096^3 step is
    also timed with a cold cache: 512 MiB written between launches, outside the
    timed bracket.  Last, C is restored and one fresh launch is made whose
    sampled output elements go to `checks` (compared with the oracle in the CPU
    leg, outside every timed region)."""
    import dense_gemm_f32_amd as mg
    from dense_gemm_f32_amd import workloads as wl
    out = {}
    for name in CASES:
        p = wl.WORKLOADS[name]()
        dA, dB, dC = make_device_problem(p, torch, dev)
        dC_init = dC.clone()
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
        if tel is not None:
            rec["telemetry"] = tel.sustained(torch, fn, t)
        if checks is not None:
            dC.copy_(dC_init)
            fn()
            torch.cuda.synchronize()
            pos = sample_positions(p)
            checks[name] = (pos, gather_c(torch, p, dC, pos))
        out[name] = rec
        log(f"{name}: {rec}")
        del dA, dB, dC, dC_init
        torch.cuda.empty_cache()
    return out


def parity_checks(per, checks):
    """CPU leg: the oracle's values at each workload's sampled elements against
    the fresh launch's (max|err|, the workload's tolerance, bit-exactness)."""
    import numpy as np
    import oracle
    from dense_gemm_f32_amd import workloads as wl
    for name, (pos, got) in checks.items():
        p = wl.WORKLOADS[name]()
        A, B, C0 = wl.make_inputs(p)
        Cn = None if C0 is None else (C0.numpy() if p.c_dtype in ("i32", "f64") else C0.float().numpy())
        t0 = time.perf_counter()
        ref = oracle.gemm_elems(p.dtype, p.transA, p.transB, p.M, p.N, p.K, p.alpha,
                                wl.to_numpy_operand(A), p.lda, wl.to_numpy_operand(B), p.ldb,
                                p.beta, Cn, p.ldc, *pos, batch=p.batch, strideA=p.strideA,
                                strideB=p.strideB, strideC=p.strideC)
        secs = time.perf_counter() - t0
        if p.c_dtype in ("f16", "bf16"):   # what an exact accumulation stores in C's type
            exp = oracle.decode16(p.c_dtype, oracle.round16(p.c_dtype, ref))
        elif p.c_dtype == "i32":
            exp = oracle.wrap_i32(ref).astype(np.float64)
        else:
            exp = ref
        err = float(np.max(np.abs(got - ref)))
        scale = float(np.max(np.abs(ref)))
        tol = (p.tolerance_coeff() * np.sqrt(max(p.K, 1)) + p.output_rounding()) * scale
        exact = bool(np.array_equal(got, exp))
        must_be_exact = p.dist == "int"
        per[name]["check"] = {
            "elements": int(got.size), "max_abs_err": err, "tol": tol,
            "err_over_tol": (err / tol) if tol else None, "bit_exact": exact,
            "exact_required": must_be_exact,
            "pass": bool(exact if must_be_exact else (err <= tol and not np.isnan(got).any())),
            "oracle_seconds": round(secs, 2)}
        log(f"check {name}: {per[name]['check']}")


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


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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
           "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
           "affinity_cpus": len(os.sched_getaffinity(0)),
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
    ap.add_argument("--read-probe", action="store_true")
    ap.add_argument("--summarize-profiles", metavar="DIR")
    ap.add_argument("--profile-case", metavar="NAME", choices=CASES)
    ap.add_argument("--launches", type=int, default=20)
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe()
        return
    if args.read_probe:
        read_probe()
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

    tel = Telemetry()
    if tel.h is None:
        log(f"no GPU telemetry: {tel.error}")
    ceiling = None if args.no_secondary else mfma_ceiling(torch, dev, tel)
    checks = {}
    per = None if args.no_secondary else per_config(torch, dev, 30, tel, checks)
    if per and (per[PRIMARY].get("telemetry") or {}).get("clock_mhz"):
        # the same kernel, sustained: the clock the roofline fraction was reached at
        roofline["clock_mhz"] = per[PRIMARY]["telemetry"]["clock_mhz"]
    if per and ceiling:
        for name in ("gemm_bf16_8192", "gemm_f16_8192", "gemm_i8_8192"):
            c = ceiling[per[name]["dtype"]]["tflops"]
            per[name]["frac_of_mfma_ceiling"] = round(per[name]["tflops"] / c, 4)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline()
        log(f"cpu_baseline: {cpu}")
        if per:   # the oracle is used in this leg only
            parity_checks(per, checks)

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
        "mfma_ceiling": ceiling,
        "per_config": per,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
