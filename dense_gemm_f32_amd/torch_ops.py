"""PyTorch front end over the C ABI: mm, bmm, broadcasting matmul and attention scores.

These functions only map torch tensors onto the ABI's arguments: a
row-major matrix or a transposed view of one becomes op = N or T with its
leading dimension, a batch dimension becomes a batch stride (0 for a
broadcast operand), and the output is allocated with torch.  Every multiply
runs in libmgemm's kernels; a layout the ABI cannot express (for instance a
column-sliced view) is first copied to a contiguous tensor.

The calls mirror the PyTorch forms of the "cuda11/matmul" tutorial
(dlog.com.cn), section "Pytorch": torch.mm, torch.bmm, matmul broadcasting a
(10,3,4) batch against a (4,5) matrix, and einsum('bhqd,bhkd->bhqk') for
attention scores.

Input types: float32, float16, bfloat16 (fp32 accumulate; fp32 output, or
the inputs' own 16-bit type), float64 (float64 output) and int8 (int32
output, wrapping).  Every type takes row-major and transposed views in place.
mm splits K over the device for deep-K shapes that would leave it idle
(the library's automatic split count), with a torch-allocated workspace.
"""
from __future__ import annotations

import math

from . import _lib

_DTYPES = None


def _dtype_name(t):
    global _DTYPES
    if _DTYPES is None:
        import torch
        _DTYPES = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
                   torch.float64: "f64", torch.int8: "i8", torch.int32: "i32"}
    name = _DTYPES.get(t)
    if name is None or name == "i32":
        raise TypeError(f"unsupported dtype {t}: fp32, fp16, bf16, fp64 or int8 inputs")
    return name


def _default_out(name):
    """C's type when none is asked for: fp32 (16-bit and fp32 inputs), the
    inputs' type for fp64, int32 for int8."""
    import torch
    return {"f64": torch.float64, "i8": torch.int32}.get(name, torch.float32)


def _matrix_layout(x):
    """(op, ld) for a 2-D view whose elements sit at row-major or column-major
    positions of some buffer; None when neither describes it."""
    r, c = x.shape
    s0, s1 = x.stride()
    if (s1 == 1 or c <= 1) and (r <= 1 or s0 >= max(c, 1)):
        return 0, max(s0 if r > 1 else c, c, 1)
    if (s0 == 1 or r <= 1) and (c <= 1 or s1 >= max(r, 1)):
        return 1, max(s1 if c > 1 else r, r, 1)
    return None


def _operand(x):
    """(tensor, op, ld) with x copied to a contiguous tensor if its layout needs it."""
    lay = _matrix_layout(x)
    if lay is None:
        x = x.contiguous()
        lay = _matrix_layout(x)
    return x, lay[0], lay[1]


def _batched_operand(x):
    """(tensor, op, ld, batch stride) for a 3-D (batch, rows, cols) view."""
    lay = _matrix_layout(x[0]) if x.shape[0] > 0 else (0, max(x.shape[2], 1))
    b_stride = x.stride(0)
    rows, cols = x.shape[1], x.shape[2]
    if lay is not None and x.shape[0] > 1 and b_stride != 0:
        op, ld = lay
        span = (cols - 1) * ld + rows if op else (rows - 1) * ld + cols
        if b_stride < span:
            lay = None
    if lay is None or b_stride < 0:
        x = x.contiguous()
        lay = _matrix_layout(x[0]) if x.shape[0] > 0 else (0, max(cols, 1))
        b_stride = x.stride(0)
    if x.shape[0] == 1:
        b_stride = 0
    return x, lay[0], lay[1], b_stride


def _check_pair(a, b):
    if a.dtype != b.dtype:
        raise TypeError(f"operands differ in dtype: {a.dtype} vs {b.dtype}")
    name = _dtype_name(a.dtype)
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("operands must be GPU tensors on one device")
    return name


def _out(shape, out_dtype, a, out, beta=0.0, in_name="f32"):
    import torch
    if beta != 0.0 and out is None:
        raise ValueError("beta != 0 needs out (the C that beta scales)")
    if out is not None:
        if tuple(out.shape) != tuple(shape) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous tensor of shape {tuple(shape)}")
        return out
    return torch.empty(shape, dtype=out_dtype or _default_out(in_name), device=a.device)


def _c_name(c, in_name):
    import torch
    if in_name == "i8":
        if c.dtype != torch.int32:
            raise TypeError(f"output dtype {c.dtype}: int8 inputs give int32")
        return "i32"
    if in_name == "f64":
        if c.dtype != torch.float64:
            raise TypeError(f"output dtype {c.dtype}: fp64 inputs give fp64")
        return "f64"
    name = _dtype_name(c.dtype)
    if name not in ("f32", in_name):
        raise TypeError(f"output dtype {c.dtype}: fp32 or the inputs' own type")
    return name


def _launch(name, c_name, op_a, op_b, M, N, K, alpha, a, lda, sa, b, ldb, sb, beta, c, ldc, sc,
            batch, splitk=None):
    """One library call: fp64 through its own entry points, a single matrix
    through split-K when that pays (or is asked for), the rest through
    gemm_strided_batched_ex."""
    if batch == 1 and splitk != 1:
        chunks = _lib.splitk_chunks(name, M, N, K, splitk or 0, transA=op_a, transB=op_b, A=a,
                                    lda=lda, B=b, ldb=ldb)
        if chunks > 1:
            _lib.gemm_splitk(name, c_name, op_a, op_b, M, N, K, alpha, a.data_ptr(), lda,
                             b.data_ptr(), ldb, beta, c, ldc, splits=splitk or 0)
            return
    if name == "f64":
        _lib.gemm_f64_strided_batched(op_a, op_b, M, N, K, alpha, a.data_ptr(), lda, sa,
                                      b.data_ptr(), ldb, sb, beta, c, ldc, sc, batch)
    else:
        _lib.gemm_strided_batched_ex(name, c_name, op_a, op_b, M, N, K, alpha, a.data_ptr(), lda,
                                     sa, b.data_ptr(), ldb, sb, beta, c, ldc, sc, batch)


def mm(a, b, *, alpha=1.0, beta=0.0, out=None, out_dtype=None, splitk=None):
    """alpha * a @ b (+ beta * out): a (M, K), b (K, N).  fp32 accumulate and
    fp32 result for fp32/16-bit inputs (or out_dtype = the inputs' 16-bit
    type); fp64 for fp64; int32 for int8.  splitk: None chooses split-K
    automatically for deep-K shapes, 1 turns it off, n asks for n chunks."""
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"mm: shapes {tuple(a.shape)} and {tuple(b.shape)} do not chain")
    name = _check_pair(a, b)
    M, K = a.shape
    N = b.shape[1]
    a, op_a, lda = _operand(a)
    b, op_b, ldb = _operand(b)
    c = _out((M, N), out_dtype, a, out, beta, name)
    _launch(name, _c_name(c, name), op_a, op_b, M, N, K, alpha, a, lda, 0, b, ldb, 0, beta, c,
            max(N, 1), M * N, 1, splitk)
    return c


def bmm(a, b, *, alpha=1.0, beta=0.0, out=None, out_dtype=None):
    """Batched alpha * a[i] @ b[i] (+ beta * out[i]); a (B, M, K), b (B, K, N).
    A batch dimension of size 1 (or a stride-0 expanded one) is shared by every
    entry of the other operand."""
    if a.dim() != 3 or b.dim() != 3 or a.shape[2] != b.shape[1]:
        raise ValueError(f"bmm: shapes {tuple(a.shape)} and {tuple(b.shape)} do not chain")
    if a.shape[0] != b.shape[0] and 1 not in (a.shape[0], b.shape[0]):
        raise ValueError(f"bmm: batch sizes {a.shape[0]} and {b.shape[0]} differ")
    name = _check_pair(a, b)
    batch = max(a.shape[0], b.shape[0])
    M, K, N = a.shape[1], a.shape[2], b.shape[2]
    a, op_a, lda, sa = _batched_operand(a)
    b, op_b, ldb, sb = _batched_operand(b)
    c = _out((batch, M, N), out_dtype, a, out, beta, name)
    _launch(name, _c_name(c, name), op_a, op_b, M, N, K, alpha, a, lda, sa, b, ldb, sb, beta, c,
            max(N, 1), M * N, batch, splitk=1)
    return c


def matmul(a, b, *, out_dtype=None):
    """a @ b for 2-D and batched operands: (M,K)@(K,N), (B,M,K)@(K,N) (b shared
    by the batch, as in the tutorial's (10,3,4)@(4,5) example),
    (M,K)@(B,K,N), (B,M,K)@(B,K,N), and any number of leading batch
    dimensions that match."""
    if a.dim() == 2 and b.dim() == 2:
        return mm(a, b, out_dtype=out_dtype)
    if a.dim() < 2 or b.dim() < 2:
        raise ValueError("matmul: operands need at least 2 dimensions")
    lead_a, lead_b = tuple(a.shape[:-2]), tuple(b.shape[:-2])
    if lead_a and lead_b and lead_a != lead_b:
        raise ValueError(f"matmul: batch shapes {lead_a} and {lead_b} differ")
    lead = lead_a or lead_b
    batch = math.prod(lead)
    a3 = a.reshape(batch, *a.shape[-2:]) if lead_a else a.unsqueeze(0)
    b3 = b.reshape(batch, *b.shape[-2:]) if lead_b else b.unsqueeze(0)
    c = bmm(a3, b3, out_dtype=out_dtype)
    return c.reshape(*lead, a.shape[-2], b.shape[-1])


def attention_scores(q, k, scale=None, *, out_dtype=None):
    """scale * q @ k^T per (batch, head): q (B, H, S, D), k (B, H, T, D) ->
    (B, H, S, T), i.e. einsum('bhqd,bhkd->bhqk') scaled; scale defaults to
    1/sqrt(D) (1 for int8 inputs, whose scale must be an integer).  k is read
    in place as the transposed operand."""
    if q.dim() != 4 or k.dim() != 4 or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError(f"attention_scores: shapes {tuple(q.shape)} and {tuple(k.shape)}")
    name = _check_pair(q, k)
    B, H, S, D = q.shape
    T = k.shape[2]
    if scale is None:
        scale = 1.0 if name == "i8" else 1.0 / math.sqrt(D)
    if name == "i8" and float(scale) != int(scale):
        raise ValueError("attention_scores: int8 inputs take an integer scale")
    q3, op_q, ldq, sq = _batched_operand(q.reshape(B * H, S, D))
    k3, op_k, ldk, sk = _batched_operand(k.reshape(B * H, T, D))
    # scores = q k^T: op(B) = k^T, so k's own layout flips
    op_kt = 1 - op_k
    c = _out((B, H, S, T), out_dtype, q, None, 0.0, name)
    _launch(name, _c_name(c, name), op_q, op_kt, S, T, D, float(scale), q3, ldq, sq, k3, ldk, sk,
            0.0, c, max(T, 1), S * T, B * H, splitk=1)
    return c
