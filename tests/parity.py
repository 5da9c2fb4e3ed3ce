"""Shared helpers for the GPU parity tests: run a Problem through the C ABI and
compare with the oracle, in full or on sampled elements."""
from __future__ import annotations

import sys

import numpy as np
import torch

import dense_gemm_f32_amd as mg
import oracle
from dense_gemm_f32_amd import workloads as wl

DEV = torch.device("cuda:0")
GUARD = 64                    # sentinel elements before and after C
SENTINEL = -1920.0            # exact in fp32, binary16 and bfloat16


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Run:
    """One problem's inputs (host + device) and the GPU result."""

    def __init__(self, p: wl.Problem, c_fill=None):
        self.p = p
        self.A, self.B, self.C0 = wl.make_inputs(p)
        self.dA = self.A.to(DEV)
        self.dB = self.B.to(DEV)
        n = p.c_elems
        c = torch.full((n + 2 * GUARD,), SENTINEL, dtype=wl.TORCH_DTYPE[p.c_dtype])
        if self.C0 is not None:
            c[GUARD:GUARD + n] = self.C0
        elif c_fill is not None:
            c[GUARD:GUARD + n] = c_fill
        self.c_init = c.double().numpy().copy()
        self.dCbuf = c.to(DEV)
        self.dC = self.dCbuf[GUARD:GUARD + n]

    def launch(self, stream=None, workspace=None):
        p = self.p
        if p.streamk is not None:
            assert p.batch == 1
            mg.gemm_streamk(p.dtype, p.c_dtype, int(p.transA), int(p.transB), p.M, p.N, p.K,
                            p.alpha, self.dA, p.lda, self.dB, p.ldb, p.beta, self.dC, p.ldc,
                            workgroups=p.streamk, workspace=workspace, stream=stream)
        elif p.splitk is not None:
            assert p.batch == 1
            mg.gemm_splitk(p.dtype, p.c_dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                           self.dA, p.lda, self.dB, p.ldb, p.beta, self.dC, p.ldc, splits=p.splitk,
                           workspace=workspace, stream=stream)
        elif p.dtype == "f64":
            if p.batch == 1 and p.strideA == p.a_rows * p.lda and not getattr(p, "force_batched", False):
                mg.gemm_f64(int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, self.dA, p.lda,
                            self.dB, p.ldb, p.beta, self.dC, p.ldc, stream=stream)
            else:
                mg.gemm_f64_strided_batched(int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                                            self.dA, p.lda, p.strideA, self.dB, p.ldb, p.strideB,
                                            p.beta, self.dC, p.ldc, p.strideC, p.batch,
                                            stream=stream)
        elif p.c_dtype != "f32":
            mg.gemm_strided_batched_ex(p.dtype, p.c_dtype, int(p.transA), int(p.transB), p.M, p.N,
                                       p.K, p.alpha, self.dA, p.lda, p.strideA, self.dB, p.ldb,
                                       p.strideB, p.beta, self.dC, p.ldc, p.strideC, p.batch,
                                       stream=stream)
        elif p.batch == 1 and p.strideA == p.a_rows * p.lda and not getattr(p, "force_batched", False):
            fn = {"f32": mg.gemm_f32, "f16": mg.gemm_f16, "bf16": mg.gemm_bf16}[p.dtype]
            fn(int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha, self.dA, p.lda, self.dB,
               p.ldb, p.beta, self.dC, p.ldc, stream=stream)
        else:
            mg.gemm_strided_batched(p.dtype, int(p.transA), int(p.transB), p.M, p.N, p.K, p.alpha,
                                    self.dA, p.lda, p.strideA, self.dB, p.ldb, p.strideB, p.beta,
                                    self.dC, p.ldc, p.strideC, p.batch, stream=stream)

    def result(self):
        """(batch, M, N) result as float64 (exact for every C type), after checking the
        guard band and padding."""
        torch.cuda.synchronize()
        p = self.p
        buf = self.dCbuf.double().cpu().numpy()
        assert np.all(buf[:GUARD] == SENTINEL) and np.all(buf[GUARD + p.c_elems:] == SENTINEL), \
            "write outside C"
        c = buf[GUARD:GUARD + p.c_elems]
        if p.ldc > p.N or p.strideC > p.M * p.ldc:
            logical = wl._logical_mask(p.c_elems, p.batch, p.M, p.N, p.ldc, p.strideC)
            init = self.c_init[GUARD:GUARD + p.c_elems]
            same = (c[~logical] == init[~logical]) | (np.isnan(c[~logical]) & np.isnan(init[~logical]))
            assert same.all(), "write into C padding"
        out = np.empty((p.batch, p.M, p.N), np.float64)
        for b in range(p.batch):
            m = c[b * p.strideC:b * p.strideC + (p.M - 1) * p.ldc + p.N]
            m = np.concatenate([m, np.zeros(p.M * p.ldc - m.size, np.float64)]).reshape(p.M, p.ldc)
            out[b] = m[:, :p.N]
        return out

    def oracle_args(self):
        p = self.p
        return (p.dtype, p.transA, p.transB, p.M, p.N, p.K, p.alpha, wl.to_numpy_operand(self.A),
                p.lda, wl.to_numpy_operand(self.B), p.ldb, p.beta,
                None if self.C0 is None else
                (self.C0.numpy() if p.c_dtype in ("i32", "f64") else self.C0.float().numpy()), p.ldc)

    def oracle_full(self):
        p = self.p
        return oracle.gemm(*self.oracle_args(), batch=p.batch, strideA=p.strideA,
                           strideB=p.strideB, strideC=p.strideC)

    def oracle_elems(self, b, i, j):
        p = self.p
        return oracle.gemm_elems(*self.oracle_args(), b, i, j, batch=p.batch, strideA=p.strideA,
                                 strideB=p.strideB, strideC=p.strideC)


def sample_positions(p: wl.Problem, n_random=20000, seed=0, tile=256):
    """Element positions to check at full size: whole first/last rows and columns of
    every batch entry sampled, rows and columns at tile boundaries, plus random ones."""
    rng = np.random.default_rng(seed)
    bs, is_, js = [], [], []
    batches = sorted({0, p.batch - 1, *rng.integers(0, p.batch, 4).tolist()})
    for b in batches:
        for i in sorted({0, p.M - 1, min(tile - 1, p.M - 1), min(tile, p.M - 1)}):
            bs.append(np.full(p.N, b)); is_.append(np.full(p.N, i)); js.append(np.arange(p.N))
        for j in sorted({0, p.N - 1, min(tile - 1, p.N - 1), min(tile, p.N - 1)}):
            bs.append(np.full(p.M, b)); is_.append(np.arange(p.M)); js.append(np.full(p.M, j))
    bs.append(rng.integers(0, p.batch, n_random))
    is_.append(rng.integers(0, p.M, n_random))
    js.append(rng.integers(0, p.N, n_random))
    return np.concatenate(bs), np.concatenate(is_), np.concatenate(js)


def expected_exact(p: wl.Problem, ref):
    """What an exact accumulation stores: the oracle's value, rounded to C's type
    (to nearest, ties to even) when C is 16-bit, wrapped to int32 for int8 inputs."""
    if p.c_dtype in ("f32", "f64"):
        return ref
    if p.c_dtype == "i32":   # int8 inputs: the exact integer result wrapped to int32
        return oracle.wrap_i32(ref).astype(np.float64)
    return oracle.decode16(p.c_dtype, oracle.round16(p.c_dtype, ref))


def check_tolerance(got, ref, p: wl.Problem, what=""):
    """max|err| <= (c*sqrt(K) + u)*max|ref| with c = 1e-5 (fp32 inputs), 2e-3 (16-bit
    inputs) or 1e-5 * 2^-29 (fp64 inputs) and u the rounding of a 16-bit C (half an ulp;
    0 for fp32 and double C)."""
    got = np.asarray(got, np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN in output"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    tol = (p.tolerance_coeff() * np.sqrt(max(p.K, 1)) + p.output_rounding()) * scale
    log(f"  {what}: max|err|={err:.3e} tol={tol:.3e} err/tol={err / tol if tol else 0:.2e}")
    assert err <= tol, f"{what}: max|err| {err} > {tol}"
    return err, tol


def check_exact(got, ref, what=""):
    got = np.asarray(got, np.float64)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    log(f"  {what}: {bad.size} mismatches of {ref.size}")
    assert bad.size == 0, f"{what}: first mismatch at {bad[0]}: {got.ravel()[bad[0]]} vs {ref.ravel()[bad[0]]}"
