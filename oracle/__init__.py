"""Oracle for dense row-major GEMM -- test infrastructure, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc): the textbook
triple loop with an fp64 accumulator, summing over k in ascending order, then
``alpha*acc + beta*C`` in fp64 (C unread when beta == 0).  Double operands
take the same loop in binary128 (``__float128``), rounded once to double at
the end.  This module only marshals numpy arrays into that library.

Sources: "Sgemm [128,128,8]" (jianshu), host_gemm and the kernel's design
comment (C = alpha*A*B + beta*C, row-major); "cuda11/matmul" (dlog.com.cn),
the CPU sgemm of section "什么是矩阵乘法"; WMMA API page (adg.csdn.net),
"1. 概述" type table (16-bit inputs with a float accumulator, 8-bit integers
with an int accumulator, doubles with a double accumulator).

16-bit operands are passed as ``numpy.uint16`` arrays holding the raw
binary16 / bfloat16 bit patterns; fp32 operands as ``numpy.float32``;
int8 operands as ``numpy.int8`` (C then ``numpy.int32``); double operands as
``numpy.float64`` (C then ``numpy.float64``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "f64": 5}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (next to the source)."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-std=c11", "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64, dbl,
                                vp, i64, i64, vp, i64, i64, dbl, vp, i64, i64, i64,
                                vp, i64, i64]
    lib.oracle_gemm_elems.restype = ctypes.c_int
    lib.oracle_gemm_elems.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                      dbl, vp, i64, i64, vp, i64, i64, dbl, vp, i64, i64,
                                      i64, i64, vp, vp, vp, vp]
    lib.oracle_f16_to_double.restype = dbl
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = dbl
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_double_to_f16.restype = ctypes.c_uint16
    lib.oracle_double_to_f16.argtypes = [dbl]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_double_to_bf16.argtypes = [dbl]
    lib.oracle_round16.restype = ctypes.c_int
    lib.oracle_round16.argtypes = [ctypes.c_int, vp, vp, i64]
    lib.oracle_wrap_i32.restype = ctypes.c_int
    lib.oracle_wrap_i32.argtypes = [vp, vp, i64]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def round16(dtype, x):
    """Round float64 values to binary16 ("f16") or bfloat16 ("bf16"), to nearest
    with ties to even; returns the uint16 bit patterns (same shape)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    if _load().oracle_round16(DTYPES[dtype], x.ctypes.data, out.ctypes.data, x.size) != 0:
        raise ValueError("round16: dtype must be f16 or bf16")
    return out


def decode16(dtype, bits):
    """float64 values of 16-bit patterns (binary16 or bfloat16)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    fn = f16_to_double if dtype == "f16" else bf16_to_double
    flat = np.array([fn(int(b)) for b in bits.ravel()], dtype=np.float64) if bits.size < 4096 else None
    if flat is None:
        # vectorised through a lookup table of all 65536 patterns
        table = _decode_table(dtype)
        return table[bits]
    return flat.reshape(bits.shape)


_TABLES = {}


def _decode_table(dtype):
    if dtype not in _TABLES:
        fn = f16_to_double if dtype == "f16" else bf16_to_double
        _TABLES[dtype] = np.array([fn(b) for b in range(65536)], dtype=np.float64)
    return _TABLES[dtype]


def set_threads(n: int) -> None:
    """Threads for the following calls (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check_operand(x, dtype):
    want = {"f32": np.float32, "i8": np.int8, "f64": np.float64}.get(dtype, np.uint16)
    if x.dtype != want:
        raise TypeError(f"{dtype} operand must be {np.dtype(want).name}, got {x.dtype}")
    if not x.flags.c_contiguous:
        raise ValueError("operands must be C-contiguous buffers")


def _check_c(C, dtype):
    want = {"i8": np.int32, "f64": np.float64}.get(dtype, np.float32)
    if C is not None and (C.dtype != want or not C.flags.c_contiguous):
        raise TypeError(f"C must be a C-contiguous {np.dtype(want).name} buffer")


def wrap_i32(x):
    """int32 C of int8 inputs: exact integer results (float64) modulo 2^32, as int32."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.int32)
    if _load().oracle_wrap_i32(x.ctypes.data, out.ctypes.data, x.size) != 0:
        raise ValueError("wrap_i32: values must be integers below 2^53 in magnitude")
    return out


def gemm(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
         batch=1, strideA=0, strideB=0, strideC=0):
    """Full output as float64 of shape (batch, M, N).

    A, B, C are flat (or any C-contiguous) buffers addressed with the given
    leading dimensions and batch strides (in elements).  C may be None when
    beta == 0.
    """
    _check_operand(A, dtype)
    _check_operand(B, dtype)
    _check_c(C, dtype)
    out = np.empty((batch, M, N), dtype=np.float64)
    rc = _load().oracle_gemm(DTYPES[dtype], int(bool(transA)), int(bool(transB)), M, N, K,
                             float(alpha), _ptr(A), lda, strideA, _ptr(B), ldb, strideB,
                             float(beta), _ptr(C), ldc, strideC, batch,
                             _ptr(out), N, M * N)
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return out


def gemm_elems(dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               bidx, iidx, jidx, batch=1, strideA=0, strideB=0, strideC=0):
    """Selected output elements (bidx[e], iidx[e], jidx[e]) as float64."""
    _check_operand(A, dtype)
    _check_operand(B, dtype)
    _check_c(C, dtype)
    bidx = np.ascontiguousarray(bidx, dtype=np.int64)
    iidx = np.ascontiguousarray(iidx, dtype=np.int64)
    jidx = np.ascontiguousarray(jidx, dtype=np.int64)
    if not (bidx.shape == iidx.shape == jidx.shape):
        raise ValueError("index arrays must have one shape")
    out = np.empty(bidx.shape, dtype=np.float64)
    rc = _load().oracle_gemm_elems(DTYPES[dtype], int(bool(transA)), int(bool(transB)),
                                   M, N, K, float(alpha), _ptr(A), lda, strideA,
                                   _ptr(B), ldb, strideB, float(beta), _ptr(C), ldc,
                                   strideC, batch, bidx.size, _ptr(bidx), _ptr(iidx),
                                   _ptr(jidx), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_gemm_elems rejected its arguments")
    return out


def f16_to_double(bits: int) -> float:
    """Exact value of one IEEE binary16 bit pattern."""
    return _load().oracle_f16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    """Exact value of one bfloat16 bit pattern."""
    return _load().oracle_bf16_to_double(bits)
