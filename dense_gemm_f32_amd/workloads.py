"""Seeded synthetic GEMM inputs and the named workloads.

This module draws random operands and lays them out in memory.  It holds no
GEMM arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it.

Recipe (one ``torch.Generator`` on the CPU per problem, seeded explicitly):
draw A, then B, then C, each over its whole stored buffer (padding included).
- ``"uniform"``: U[-1, 1) as ``2*rand - 1`` in fp32 (in fp64 for double
  operands, so that every significand bit is drawn);
- ``"normal"``:  N(0, 1) as ``randn`` in fp32 (fp64 for double operands),
  then rounded to the operand type (round-to-nearest-even for bf16 / fp16);
- ``"int"``:     integers uniform in [lo, hi] (``randint``), stored exactly
  in the operand type.

The named workloads follow the shapes the pages measure on:
- 256^3 and 4096^3 SGEMM ("Sgemm [128,128,8]" harness; "cuda11/matmul"
  timing tables);
- a ragged SGEMM whose sizes are no multiple of any tile, with integer-valued
  operands in {0..99} (the residual-tile example of the CSDN tile-algorithm
  page, which fills with ``rand() % 100``);
- 16-bit inputs with a float accumulator, int8 inputs with an int32
  accumulator and double inputs with a double accumulator (WMMA API page,
  type table);
- strided-batched QK^T with B stored [n, d] ("cuda11/matmul", section
  "Pytorch", the einsum 'bhqd,bhkd->bhqk' example), with fp32 C and, as the
  tutorial's Triton kernel stores its accumulator in C's own type, with a
  binary16 C.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "i8": torch.int8, "i32": torch.int32, "f64": torch.float64}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4, "f64": 8}


@dataclasses.dataclass
class Problem:
    dtype: str                 # "f32" | "f16" | "bf16" | "i8" | "f64" (operand type)
    M: int
    N: int
    K: int
    transA: bool = False
    transB: bool = False
    batch: int = 1
    alpha: float = 1.0
    beta: float = 0.0
    dist: str = "uniform"      # "uniform" | "normal" | "int"
    int_lo: int = 0
    int_hi: int = 99
    c_dist: Optional[str] = None   # distribution of C0; None -> same as dist
    seed: int = 0
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    strideA: Optional[int] = None
    strideB: Optional[int] = None
    strideC: Optional[int] = None
    pad_value: Optional[float] = None  # fill for padding beyond the logical matrix
    c_dtype: str = "f32"       # C's type: "f32", the operand type for 16-bit output, "i32" for
                               # i8; double operands always take "f64"
    splitk: Optional[int] = None   # None: one-pass kernels; n: split-K with n chunks (0: automatic)
    streamk: Optional[int] = None  # None: not stream-K; n: stream-K over n workgroups (0: default)

    def __post_init__(self):
        if self.dtype == "f64":
            self.c_dtype = "f64"
        a_rows, a_cols = (self.K, self.M) if self.transA else (self.M, self.K)
        b_rows, b_cols = (self.N, self.K) if self.transB else (self.K, self.N)
        self.a_rows, self.a_cols = a_rows, a_cols
        self.b_rows, self.b_cols = b_rows, b_cols
        if self.lda is None:
            self.lda = max(a_cols, 1)
        if self.ldb is None:
            self.ldb = max(b_cols, 1)
        if self.ldc is None:
            self.ldc = max(self.N, 1)
        if self.strideA is None:
            self.strideA = a_rows * self.lda
        if self.strideB is None:
            self.strideB = b_rows * self.ldb
        if self.strideC is None:
            self.strideC = self.M * self.ldc

    @property
    def flops(self) -> float:
        """2*M*N*K per batch entry, the pages' flop count."""
        return 2.0 * self.M * self.N * self.K * self.batch

    def buffer_elems(self, rows, ld, stride):
        if self.batch == 0 or rows == 0:
            return 0
        return (self.batch - 1) * stride + (rows - 1) * ld + ld

    @property
    def a_elems(self):
        return self.buffer_elems(self.a_rows, self.lda, self.strideA)

    @property
    def b_elems(self):
        return self.buffer_elems(self.b_rows, self.ldb, self.strideB)

    @property
    def c_elems(self):
        return self.buffer_elems(self.M, self.ldc, self.strideC)

    def tolerance_coeff(self) -> float:
        """c in max|err| <= c * sqrt(K) * max|ref| (fp32: 1e-5, 16-bit: 2e-3, int8: 0;
        fp64: the fp32 constant scaled by the ratio of unit roundoffs, 1e-5 * 2^-29)."""
        return {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "i8": 0.0,
                "f64": 1e-5 * 2.0 ** -29}[self.dtype]

    def output_rounding(self) -> float:
        """Relative rounding of the stored C: half an ulp of its type (0 for fp32,
        which the accumulator itself is)."""
        return {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8, "i32": 0.0,
                "f64": 0.0}[self.c_dtype]


def _draw(gen, n, dist, lo, hi, fdt=torch.float32):
    if dist == "uniform":
        return 2.0 * torch.rand(n, generator=gen, dtype=fdt) - 1.0
    if dist == "normal":
        return torch.randn(n, generator=gen, dtype=fdt)
    if dist == "int":
        return torch.randint(lo, hi + 1, (n,), generator=gen).to(fdt)
    raise ValueError(f"unknown distribution {dist!r}")


def _logical_mask(total, batch, rows, cols, ld, stride):
    """Boolean mask over a flat buffer: True where a logical matrix element lives."""
    mask = np.zeros(total, dtype=bool)
    if total == 0:
        return mask
    r = np.arange(rows)[:, None] * ld + np.arange(cols)[None, :]
    for b in range(batch):
        mask[b * stride + r.ravel()] = True
    return mask


def make_inputs(p: Problem):
    """CPU torch tensors (flat) A, B (operand dtype) and C0 (C's type, or None when beta == 0
    and no C distribution was asked for)."""
    gen = torch.Generator()
    gen.manual_seed(p.seed)
    tdt = TORCH_DTYPE[p.dtype]
    fdt = torch.float64 if p.dtype == "f64" else torch.float32
    bufs = []
    for elems, rows, cols, ld, stride in ((p.a_elems, p.a_rows, p.a_cols, p.lda, p.strideA),
                                          (p.b_elems, p.b_rows, p.b_cols, p.ldb, p.strideB)):
        x = _draw(gen, elems, p.dist, p.int_lo, p.int_hi, fdt).to(tdt)
        if p.pad_value is not None and elems:
            mask = torch.from_numpy(_logical_mask(elems, p.batch, rows, cols, ld, stride))
            x[~mask] = p.pad_value
        bufs.append(x)
    C0 = None
    if p.beta != 0.0 or p.c_dist is not None:
        cd = p.c_dist or p.dist
        if p.c_dtype == "i32":   # integer C: drawn as int64, stored exactly
            C0 = torch.randint(p.int_lo, p.int_hi + 1, (p.c_elems,), generator=gen).to(torch.int32)
        else:
            C0 = _draw(gen, p.c_elems, cd, p.int_lo, p.int_hi, fdt)
        if p.c_dtype not in ("f32", "i32", "f64"):
            C0 = C0.to(TORCH_DTYPE[p.c_dtype])
    return bufs[0], bufs[1], C0


def to_numpy_operand(x: torch.Tensor) -> np.ndarray:
    """Operand buffer as numpy: float32, float64 or int8 values, or uint16 bit patterns for
    16-bit types."""
    x = x.detach().cpu().contiguous()
    if x.dtype in (torch.float32, torch.float64, torch.int8, torch.int32):
        return x.numpy()
    return x.view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------------------
# Named workloads.  Seeds are 1000 + the workload's number.
# --------------------------------------------------------------------------------------

def sgemm_256() -> Problem:
    """SGEMM fp32 256^3, A, B ~ U[-1,1), alpha=1, beta=0."""
    return Problem("f32", 256, 256, 256, dist="uniform", seed=1001)


def sgemm_4096() -> Problem:
    """SGEMM fp32 4096^3, A, B, C ~ U[-1,1), alpha=1.5, beta=0.5."""
    return Problem("f32", 4096, 4096, 4096, alpha=1.5, beta=0.5, dist="uniform", seed=1002)


def sgemm_ragged() -> Problem:
    """SGEMM fp32 M=1000, N=1027, K=999, integer-valued operands in {0..99}."""
    return Problem("f32", 1000, 1027, 999, dist="int", int_lo=0, int_hi=99, seed=1003)


def sgemm_ragged_splitk() -> Problem:
    """The ragged SGEMM through split-K with the automatic chunk count (3 chunks of 352,
    the last 295: 816 workgroups of 64x64 instead of 272)."""
    p = sgemm_ragged()
    p.splitk = 0
    return p


def sgemm_ragged_streamk() -> Problem:
    """The ragged SGEMM through stream-K with the default 512 workgroups (two per CU) sharing
    the 272 tiles' 32 K-iterations each; split tiles are completed in the same launch."""
    p = sgemm_ragged()
    p.streamk = 0
    return p


def gemm16_8192(dtype: str = "bf16") -> Problem:
    """8192^3 with bf16 (or fp16) N(0,1) operands, fp32 accumulate and fp32 C."""
    return Problem(dtype, 8192, 8192, 8192, dist="normal", seed=1004)


def qkt_batched() -> Problem:
    """Attention scores Q K^T: 128 (8 x 16 heads) x [1024 x 1024 x 64], fp16 N(0,1),
    K stored [n, d] (transB), alpha = 1/sqrt(64), beta = 0."""
    return Problem("f16", 1024, 1024, 64, transB=True, batch=128, alpha=1.0 / math.sqrt(64),
                   dist="normal", seed=1005)


def gemm_i8_8192() -> Problem:
    """8192^3 with int8 operands in [-128, 127], int32 accumulate and int32 C; A and B
    both K-contiguous (B stored [n, k])."""
    return Problem("i8", 8192, 8192, 8192, transB=True, dist="int", int_lo=-128, int_hi=127,
                   c_dtype="i32", seed=1007)


def dgemm_4096() -> Problem:
    """DGEMM fp64 4096^3, A, B, C ~ U[-1,1) drawn in fp64, alpha=1.5, beta=0.5 (the SGEMM
    workload's shape and scalars in the double row of the type table)."""
    return Problem("f64", 4096, 4096, 4096, alpha=1.5, beta=0.5, dist="uniform", seed=1008)


def qkt_batched_f16_out() -> Problem:
    """The attention-score batch with a binary16 C (fp32 accumulate, rounded on store)."""
    p = qkt_batched()
    p.c_dtype = "f16"
    p.seed = 1006
    return p


WORKLOADS = {
    "sgemm_256": sgemm_256,
    "sgemm_4096": sgemm_4096,
    "sgemm_ragged": sgemm_ragged,
    "sgemm_ragged_splitk": sgemm_ragged_splitk,
    "sgemm_ragged_streamk": sgemm_ragged_streamk,
    "gemm_bf16_8192": lambda: gemm16_8192("bf16"),
    "gemm_f16_8192": lambda: gemm16_8192("f16"),
    "qkt_batched": qkt_batched,
    "qkt_batched_f16_out": qkt_batched_f16_out,
    "gemm_i8_8192": gemm_i8_8192,
    "dgemm_4096": dgemm_4096,
}


def int_shadow(p: Problem, lo: int, hi: int) -> Problem:
    """The same shape with integer-valued operands in [lo, hi] (and C0 too, when used),
    chosen so that every partial sum stays below 2^24 and the result is exact in fp32."""
    return dataclasses.replace(p, dist="int", int_lo=lo, int_hi=hi,
                               c_dist="int" if p.c_dist or p.beta != 0.0 else None)
