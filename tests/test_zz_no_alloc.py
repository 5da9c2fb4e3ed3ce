"""gemm_splitk_noalloc (split-K whose partial sums live in the library's fixed per-GPU
scratch) against gemm_splitk (a caller's workspace): the same plan and kernels, so the
outputs must be identical, and both must match the oracle.  Two calls in a row, the second
on a smaller problem, so the second reads scratch left over from the first."""
import numpy as np
import pytest
import torch

import dense_gemm_f32_amd as mg
from dense_gemm_f32_amd import workloads as wl
from parity import Run, check_exact, check_tolerance, expected_exact, log

pytestmark = pytest.mark.gpu


def _noalloc(r: Run, stream=None):
    p = r.p
    mg.gemm_splitk_noalloc(p.dtype, p.c_dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                           r.dA, p.lda, r.dB, p.ldb, p.beta, r.dC, p.ldc, splits=p.splitk,
                           stream=stream)


def _both(p: wl.Problem, exact: bool, what: str):
    plan = mg.splitk_plan(p.dtype, p.M, p.N, p.K, p.splitk, transA=int(p.transA),
                          transB=int(p.transB), lda=p.lda, ldb=p.ldb)
    assert plan["chunks"] > 1 and plan["workspace_bytes"] <= mg.NOALLOC_SCRATCH_BYTES, plan
    log(f"[no-alloc] {what}: {plan['chunks']} chunks, {plan['workspace_bytes']} scratch bytes")
    a = Run(p)
    _noalloc(a)
    got = a.result()
    b = Run(p)
    b.launch()                      # gemm_splitk with a torch-allocated workspace
    want = b.result()
    assert np.array_equal(got, want, equal_nan=True), f"{what}: differs from gemm_splitk"
    ref = a.oracle_full()
    if exact:
        check_exact(got, expected_exact(p, ref), f"{what} vs oracle")
    else:
        check_tolerance(got, ref, p, f"{what} vs oracle")


def test_noalloc_matches_splitk_on_two_calls_in_a_row():
    # a large first call (the ragged shape in three chunks, odd leading dimensions) then a
    # smaller one: the second reuses scratch that still holds the first call's partial sums
    first = wl.Problem("f32", 1000, 1027, 999, alpha=2.0, beta=-1.0, dist="int", int_lo=-20,
                       int_hi=20, c_dist="int", seed=140, splitk=0)
    second = wl.Problem("f32", 300, 260, 1500, alpha=1.5, beta=0.5, dist="int", int_lo=-9,
                        int_hi=9, c_dist="int", seed=141, splitk=4)
    _both(first, True, "f32 1000x1027x999 automatic")
    _both(second, True, "f32 300x260x1500 x4 (smaller, after the first)")


def test_noalloc_other_types_and_float_data():
    _both(wl.Problem("bf16", 257, 190, 3000, transA=True, alpha=0.75, beta=-1.25, dist="normal",
                     c_dist="uniform", c_dtype="bf16", seed=142, splitk=6), False,
          "bf16 -> bf16 C, 257x190x3000 x6")
    _both(wl.Problem("i8", 150, 133, 700, transB=True, alpha=3.0, beta=-2.0, dist="int",
                     int_lo=-128, int_hi=127, c_dist="int", c_dtype="i32", seed=143, splitk=2), True,
          "int8 -> int32, 150x133x700 x2")
    _both(wl.Problem("f64", 200, 190, 2050, alpha=1.5, beta=0.5, dist="uniform", c_dist="uniform",
                     seed=144, splitk=0), False, "fp64 200x190x2050 automatic")


def test_noalloc_one_chunk_and_quick_returns_use_no_scratch():
    for p in (wl.Problem("f32", 64, 64, 32, dist="int", int_lo=-9, int_hi=9, seed=145, splitk=8),
              wl.Problem("f32", 90, 70, 512, alpha=0.0, beta=-0.5, dist="uniform", seed=146,
                         splitk=4)):
        r = Run(p)
        _noalloc(r)
        check_exact(r.result(), r.oracle_full(), f"no-alloc {p.M}x{p.N}x{p.K} alpha={p.alpha}")


def test_noalloc_refuses_more_than_its_scratch():
    # 4 x 4096 x 4096 fp32 partial sums are 256 MiB: refused before any launch, C untouched
    M = N = 4096
    K = 4096
    C = torch.full((M * N,), 7.0, device="cuda")
    A = torch.zeros(M * K, device="cuda")
    B = torch.zeros(K * N, device="cuda")
    with pytest.raises(mg.MgemmError) as e:
        mg.gemm_splitk_noalloc("f32", "f32", 0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N, splits=4)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())


def test_noalloc_on_a_side_stream():
    p = wl.Problem("f32", 300, 260, 1500, dist="int", int_lo=-9, int_hi=9, seed=147, splitk=4)
    r = Run(p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _noalloc(r)
    s.synchronize()
    check_exact(r.result(), r.oracle_full(), "no-alloc on a side stream")
