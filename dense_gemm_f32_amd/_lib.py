"""ctypes binding to libmgemm.so: argument marshalling only.

Every function here forwards to the C entry point of the same name declared
in include/mgemm.h.  Operands may be torch tensors (their ``data_ptr()`` is
passed, after checking that they live on the GPU and are large enough for the
sizes, leading dimensions and strides given) or raw integer device
addresses (no checks beyond the library's own).  The default stream is the
current torch stream of the operands' device.

There is no fallback: if libmgemm.so is missing, the first call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmgemm.so")
POISON_LIB_PATH = os.path.join(PKG, "libmgemm_poison.so")   # LDS race-check build
BUILD_LDS_POISON = 1   # MGEMM_BUILD_LDS_POISON

OP_N, OP_T = 0, 1
F32, F16, BF16, I8, I32, F64 = 0, 1, 2, 3, 4, 5
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "i8": I8, "i32": I32, "f64": F64}
ELEM_SIZE = {F32: 4, F16: 2, BF16: 2, I8: 1, I32: 4, F64: 8}

STATUS = {0: "MGEMM_OK", 1: "MGEMM_INVALID_ARG", 2: "MGEMM_HIP_ERROR", 3: "MGEMM_SCRATCH_TOO_SMALL"}
# fixed device scratch of gemm_splitk_noalloc (MGEMM_NOALLOC_SCRATCH_BYTES in include/mgemm.h)
NOALLOC_SCRATCH_BYTES = 64 << 20
# zeroed prefix of a gemm_streamk workspace and the workgroup cap
# (MGEMM_STREAMK_COUNTER_BYTES, MGEMM_STREAMK_MAX_WORKGROUPS in include/mgemm.h)
STREAMK_COUNTER_BYTES = 64 << 10
STREAMK_MAX_WORKGROUPS = 16384


class MgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class VariantInfo(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("dtype", ctypes.c_int), ("block_m", ctypes.c_int),
                ("block_n", ctypes.c_int), ("block_k", ctypes.c_int), ("waves_m", ctypes.c_int),
                ("waves_n", ctypes.c_int), ("threads", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("pipe", ctypes.c_int), ("name", ctypes.c_char * 64)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


class SplitkPlanInfo(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_int64), ("chunks", ctypes.c_int64),
                ("chunk_len", ctypes.c_int64), ("variant", VariantInfo), ("grid", ctypes.c_int64)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["variant"] = self.variant.as_dict()
        return d


class StreamkPlanInfo(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("tiles", ctypes.c_int64), ("iterations", ctypes.c_int64),
                ("k_per_iteration", ctypes.c_int64), ("variant", VariantInfo)]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["variant"] = self.variant.as_dict()
        return d


_lib = None
_override = None   # a library that using_library() routes every call to


def load():
    """The library the calls go to: libmgemm.so (raises if it has not been built), or
    the one a using_library() block selects."""
    global _lib
    if _override is not None:
        return _override
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Route every call of this module to another build of the same sources inside the
    block (e.g. POISON_LIB_PATH, the LDS race-check build); the product library is used
    again afterwards."""
    global _override
    prev = _override
    _override = _open(path)
    try:
        yield _override
    finally:
        _override = prev


def build_flags():
    """MGEMM_BUILD_* bits of the library in use (0: the product build)."""
    return load().mgemm_build_flags()


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()'). There is no fallback path.")
    lib = ctypes.CDLL(path)
    i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    single = [i32, i32, i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    for name in ("gemm_f32", "gemm_f16", "gemm_bf16"):
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = single
    lib.gemm_strided_batched.restype = i32
    lib.gemm_strided_batched.argtypes = [i32, i32, i32, i64, i64, i64, f32, vp, i64, i64, vp, i64,
                                         i64, f32, vp, i64, i64, i64, vp]
    f64 = ctypes.c_double
    lib.gemm_f64.restype = i32
    lib.gemm_f64.argtypes = [i32, i32, i64, i64, i64, f64, vp, i64, vp, i64, f64, vp, i64, vp]
    lib.gemm_f64_strided_batched.restype = i32
    lib.gemm_f64_strided_batched.argtypes = [i32, i32, i64, i64, i64, f64, vp, i64, i64, vp, i64,
                                             i64, f64, vp, i64, i64, i64, vp]
    lib.gemm_splitk.restype = i32
    lib.gemm_splitk.argtypes = [i32, i32, i32, i32, i64, i64, i64, f64, vp, i64, vp, i64, f64, vp,
                                i64, i64, vp, i64, vp]
    lib.gemm_splitk_noalloc.restype = i32
    lib.gemm_splitk_noalloc.argtypes = [i32, i32, i32, i32, i64, i64, i64, f64, vp, i64, vp, i64, f64,
                                        vp, i64, i64, vp]
    lib.mgemm_splitk_plan.restype = i32
    lib.mgemm_splitk_plan.argtypes = [i32, i32, i32, i64, i64, i64, vp, i64, vp, i64, i64,
                                      ctypes.POINTER(SplitkPlanInfo)]
    lib.gemm_streamk.restype = i32
    lib.gemm_streamk.argtypes = [i32, i32, i32, i32, i64, i64, i64, f64, vp, i64, vp, i64, f64, vp,
                                 i64, i64, vp, i64, vp]
    lib.mgemm_streamk_plan.restype = i32
    lib.mgemm_streamk_plan.argtypes = [i32, i32, i32, i64, i64, i64, vp, i64, vp, i64, i64,
                                       ctypes.POINTER(StreamkPlanInfo)]
    lib.gemm_strided_batched_ex.restype = i32
    lib.gemm_strided_batched_ex.argtypes = [i32, i32, i32, i32, i64, i64, i64, f32, vp, i64, i64, vp,
                                            i64, i64, f32, vp, i64, i64, i64, vp]
    lib.mgemm_status_string.restype = ctypes.c_char_p
    lib.mgemm_status_string.argtypes = [i32]
    lib.mgemm_num_variants.restype = i32
    lib.mgemm_num_variants.argtypes = []
    lib.mgemm_variant.restype = i32
    lib.mgemm_variant.argtypes = [i32, ctypes.POINTER(VariantInfo)]
    lib.mgemm_select.restype = i32
    lib.mgemm_select.argtypes = [i32, i32, i32, i64, i64, i64, f32, vp, i64, i64, vp, i64, i64,
                                 f32, vp, i64, i64, i64, ctypes.POINTER(VariantInfo),
                                 ctypes.POINTER(i64)]
    lib.mgemm_select_ex.restype = i32
    lib.mgemm_select_ex.argtypes = [i32, i32, i32, i32, i64, i64, i64, ctypes.c_double, vp, i64, i64,
                                    vp, i64, i64, ctypes.c_double, vp, i64, i64, i64,
                                    ctypes.POINTER(VariantInfo), ctypes.POINTER(i64)]
    lib.mgemm_force_variant.restype = i32
    lib.mgemm_force_variant.argtypes = [i32, i32]
    lib.mgemm_build_flags.restype = i32
    lib.mgemm_build_flags.argtypes = []
    return lib


# --------------------------------------------------------------------------- helpers

def _span(rows, cols, ld):
    return 0 if rows == 0 or cols == 0 else (rows - 1) * ld + cols


def _extent(rows, cols, ld, stride, batch):
    """Elements an operand covers: batch entries at `stride`, each rows x cols at `ld`."""
    if batch == 0:
        return 0
    return (batch - 1) * stride + _span(rows, cols, ld)


def _addr(x, need_elems: int, elem_size: int, what: str):
    """(device address, CUDA device index or None) of x; for tensors also checks the
    device, element size, layout and size."""
    if x is None:
        return None, None
    if type(x) is int:
        return x, None
    # the common case in one expression; anything else takes the checks below,
    # which name what is wrong
    try:
        if x.is_cuda and x.element_size() == elem_size and x.numel() >= need_elems and x.is_contiguous():
            return x.data_ptr(), x.get_device()
    except (AttributeError, TypeError):
        pass
    if isinstance(x, int):
        return x, None
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor or an int address")
    if not x.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if x.element_size() != elem_size:
        raise ValueError(f"{what}: element size {x.element_size()} != {elem_size}")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be a contiguous buffer (express strides with ld/stride)")
    if x.numel() < need_elems:
        raise ValueError(f"{what}: buffer holds {x.numel()} elements, sizes need {need_elems}")
    return x.data_ptr(), x.get_device()


_current_raw_stream = None   # device index -> handle of torch's current stream there


def _stream(stream, device):
    """Launch stream handle: `stream` itself, else torch's current stream on `device` (a
    CUDA device index), else None (the library's default, the null stream)."""
    if stream is not None:
        return int(stream)
    if device is None:
        return None
    global _current_raw_stream
    if _current_raw_stream is None:
        import torch
        # the raw handle without building a Stream object (about 0.06 against 1.9 us a
        # call, which matters for launches of a few microseconds); the public call
        # otherwise
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _current_raw_stream = raw if raw is not None else (
            lambda index: torch.cuda.current_stream(index).cuda_stream)
    return _current_raw_stream(device)


def _workspace_on(nbytes, device, stream, launch, zero=False):
    """A torch-allocated workspace for a call launched on stream handle `launch`.  It is
    allocated (and, with `zero`, zero-filled) on that stream, so that the fill precedes the
    call and torch's caching allocator, once the tensor is dropped, hands the block only to
    work ordered after the call's kernels (allocated on another stream, the block could be
    reused while they still write it)."""
    import torch
    make = torch.zeros if zero else torch.empty
    if stream is None:   # the launch stream is torch's current stream
        return make(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(torch.cuda.ExternalStream(launch, device=device)):
        return make(nbytes, dtype=torch.uint8, device=device)


def _check(status: int, what: str):
    if status != 0:
        raise MgemmError(status, what)


def _single(name, dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream):
    es = ELEM_SIZE[dtype]
    ces = 8 if dtype == F64 else 4
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0
    pa, _ = _addr(A, _span(a_rows, a_cols, lda) if reads else 0, es, "A")
    pb, _ = _addr(B, _span(b_rows, b_cols, ldb) if reads else 0, es, "B")
    pc, dev = _addr(C, _span(M, N, ldc), ces, "C")
    st = getattr(load(), name)(int(transA), int(transB), M, N, K, alpha, pa, lda, pb, ldb, beta,
                               pc, ldc, _stream(stream, dev))
    _check(st, name)


# --------------------------------------------------------------------------- entry points

def gemm_f32(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C = alpha*op(A)*op(B) + beta*C, fp32 operands (see include/mgemm.h)."""
    _single("gemm_f32", F32, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_f16(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """binary16 A/B, fp32 accumulate and fp32 C."""
    _single("gemm_f16", F16, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_bf16(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """bfloat16 A/B, fp32 accumulate and fp32 C."""
    _single("gemm_bf16", BF16, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
            stream)


def gemm_f64(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """double A, B, C, alpha and beta; fp64 matrix-core products."""
    _single("gemm_f64", F64, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)


def gemm_f64_strided_batched(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB,
                             beta, C, ldc, strideC, batch, stream=None):
    """Strided-batched fp64 GEMM (double alpha and beta)."""
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0 and batch > 0
    pa, _ = _addr(A, _extent(a_rows, a_cols, lda, strideA, batch) if reads else 0, 8, "A")
    pb, _ = _addr(B, _extent(b_rows, b_cols, ldb, strideB, batch) if reads else 0, 8, "B")
    pc, dev = _addr(C, _extent(M, N, ldc, strideC, batch), 8, "C")
    st = load().gemm_f64_strided_batched(int(transA), int(transB), M, N, K, alpha, pa, lda, strideA,
                                         pb, ldb, strideB, beta, pc, ldc, strideC, batch,
                                         _stream(stream, dev))
    _check(st, "gemm_f64_strided_batched")


def gemm_strided_batched(in_dtype, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb,
                         strideB, beta, C, ldc, strideC, batch, stream=None):
    """Strided-batched GEMM; in_dtype is 0/1/2 or "f32"/"f16"/"bf16"."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    es = ELEM_SIZE[dt]
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0 and batch > 0
    pa, _ = _addr(A, _extent(a_rows, a_cols, lda, strideA, batch) if reads else 0, es, "A")
    pb, _ = _addr(B, _extent(b_rows, b_cols, ldb, strideB, batch) if reads else 0, es, "B")
    pc, dev = _addr(C, _extent(M, N, ldc, strideC, batch), 4, "C")
    st = load().gemm_strided_batched(dt, int(transA), int(transB), M, N, K, alpha, pa, lda,
                                     strideA, pb, ldb, strideB, beta, pc, ldc, strideC, batch,
                                     _stream(stream, dev))
    _check(st, "gemm_strided_batched")


def gemm_strided_batched_ex(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, strideA, B,
                            ldb, strideB, beta, C, ldc, strideC, batch, stream=None):
    """Strided-batched GEMM with C of type c_dtype: fp32, or the inputs' 16-bit type."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    ct = DTYPE_CODES.get(c_dtype, c_dtype)
    es = ELEM_SIZE[dt]
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0 and batch > 0
    pa, _ = _addr(A, _extent(a_rows, a_cols, lda, strideA, batch) if reads else 0, es, "A")
    pb, _ = _addr(B, _extent(b_rows, b_cols, ldb, strideB, batch) if reads else 0, es, "B")
    pc, dev = _addr(C, _extent(M, N, ldc, strideC, batch), ELEM_SIZE.get(ct, 4), "C")
    st = load().gemm_strided_batched_ex(dt, ct, int(transA), int(transB), M, N, K, alpha, pa, lda,
                                        strideA, pb, ldb, strideB, beta, pc, ldc, strideC, batch,
                                        _stream(stream, dev))
    _check(st, "gemm_strided_batched_ex")


def splitk_plan(in_dtype, M, N, K, splits=0, transA=0, transB=0, A=1 << 20, lda=None, B=1 << 20,
                ldb=None):
    """What gemm_splitk will do (a dict: workspace_bytes, chunks, chunk_len, and the GEMM
    kernel's variant and grid).  A and B are addresses (ints) or tensors: only their
    alignment matters."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    lda = lda if lda is not None else (M if transA else K)
    ldb = ldb if ldb is not None else (K if transB else N)
    pa = A if isinstance(A, int) else A.data_ptr()
    pb = B if isinstance(B, int) else B.data_ptr()
    info = SplitkPlanInfo()
    _check(load().mgemm_splitk_plan(dt, int(transA), int(transB), M, N, K, pa, lda, pb, ldb, splits,
                                    ctypes.byref(info)), "mgemm_splitk_plan")
    return info.as_dict()


def splitk_chunks(in_dtype, M, N, K, splits=0, **operands):
    """K-chunks gemm_splitk runs (1: the plain kernel)."""
    return splitk_plan(in_dtype, M, N, K, splits, **operands)["chunks"]


def splitk_workspace_bytes(in_dtype, M, N, K, splits=0, **operands):
    """Workspace bytes gemm_splitk needs (0 when nothing is chunked)."""
    return splitk_plan(in_dtype, M, N, K, splits, **operands)["workspace_bytes"]


def gemm_splitk(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                splits=0, workspace=None, stream=None):
    """Split-K GEMM (single matrix).  `workspace` is a device tensor (or int address) of at
    least splitk_workspace_bytes(...) bytes; None allocates one with torch on C's device."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    ct = DTYPE_CODES.get(c_dtype, c_dtype)
    es = ELEM_SIZE[dt]
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0
    pa, _ = _addr(A, _span(a_rows, a_cols, lda) if reads else 0, es, "A")
    pb, _ = _addr(B, _span(b_rows, b_cols, ldb) if reads else 0, es, "B")
    pc, dev = _addr(C, _span(M, N, ldc), ELEM_SIZE.get(ct, 4), "C")
    need = (splitk_workspace_bytes(dt, M, N, K, splits, transA=transA, transB=transB,
                                   A=pa or 0, lda=lda, B=pb or 0, ldb=ldb) if splits >= 0 else 0)
    launch = _stream(stream, dev)
    if workspace is None and need > 0:
        workspace = _workspace_on(need, dev, stream, launch)
    if workspace is None:
        pw, wbytes = None, 0
    elif isinstance(workspace, int):
        pw, wbytes = workspace, need
    else:
        pw, _ = _addr(workspace, 0, workspace.element_size(), "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    st = load().gemm_splitk(dt, ct, int(transA), int(transB), M, N, K, alpha, pa, lda, pb, ldb, beta,
                            pc, ldc, splits, pw, wbytes, launch)
    _check(st, "gemm_splitk")


def gemm_splitk_noalloc(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta,
                        C, ldc, splits=0, stream=None):
    """Split-K GEMM whose partial sums go to the library's fixed per-GPU scratch
    (NOALLOC_SCRATCH_BYTES): nothing is allocated, here or in the library.  Calls that may
    overlap on one GPU race on that scratch; order them on one stream."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    ct = DTYPE_CODES.get(c_dtype, c_dtype)
    es = ELEM_SIZE[dt]
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0
    pa, _ = _addr(A, _span(a_rows, a_cols, lda) if reads else 0, es, "A")
    pb, _ = _addr(B, _span(b_rows, b_cols, ldb) if reads else 0, es, "B")
    pc, dev = _addr(C, _span(M, N, ldc), ELEM_SIZE.get(ct, 4), "C")
    st = load().gemm_splitk_noalloc(dt, ct, int(transA), int(transB), M, N, K, alpha, pa, lda, pb,
                                    ldb, beta, pc, ldc, splits, _stream(stream, dev))
    _check(st, "gemm_splitk_noalloc")


def streamk_plan(in_dtype, M, N, K, workgroups=0, transA=0, transB=0, A=1 << 20, lda=None,
                 B=1 << 20, ldb=None):
    """What gemm_streamk will do (a dict: workspace_bytes, workgroups, tiles, iterations,
    k_per_iteration and the tile build's variant).  A and B are addresses (ints) or tensors:
    only their alignment matters."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    lda = lda if lda is not None else (M if transA else K)
    ldb = ldb if ldb is not None else (K if transB else N)
    pa = A if isinstance(A, int) else A.data_ptr()
    pb = B if isinstance(B, int) else B.data_ptr()
    info = StreamkPlanInfo()
    _check(load().mgemm_streamk_plan(dt, int(transA), int(transB), M, N, K, pa, lda, pb, ldb,
                                     workgroups, ctypes.byref(info)), "mgemm_streamk_plan")
    return info.as_dict()


def gemm_streamk(in_dtype, c_dtype, transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                 workgroups=0, workspace=None, stream=None):
    """Stream-K GEMM (single matrix).  `workspace` is a device tensor (or int address) of at
    least streamk_plan(...)["workspace_bytes"] bytes whose first STREAMK_COUNTER_BYTES are
    zero (zero-fill it once; every call leaves them zero); None allocates a zero-filled one
    with torch on C's device."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    ct = DTYPE_CODES.get(c_dtype, c_dtype)
    es = ELEM_SIZE[dt]
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    reads = M > 0 and N > 0 and K > 0 and alpha != 0.0
    pa, _ = _addr(A, _span(a_rows, a_cols, lda) if reads else 0, es, "A")
    pb, _ = _addr(B, _span(b_rows, b_cols, ldb) if reads else 0, es, "B")
    pc, dev = _addr(C, _span(M, N, ldc), ELEM_SIZE.get(ct, 4), "C")
    need = (streamk_plan(dt, M, N, K, workgroups, transA=transA, transB=transB, A=pa or 0, lda=lda,
                         B=pb or 0, ldb=ldb)["workspace_bytes"] if workgroups >= 0 else 0)
    launch = _stream(stream, dev)
    if workspace is None and need > 0:
        workspace = _workspace_on(need, dev, stream, launch, zero=True)
    if workspace is None:
        pw, wbytes = None, 0
    elif isinstance(workspace, int):
        pw, wbytes = workspace, need
    else:
        pw, _ = _addr(workspace, 0, workspace.element_size(), "workspace")
        wbytes = workspace.numel() * workspace.element_size()
    st = load().gemm_streamk(dt, ct, int(transA), int(transB), M, N, K, alpha, pa, lda, pb, ldb, beta,
                             pc, ldc, workgroups, pw, wbytes, launch)
    _check(st, "gemm_streamk")


# --------------------------------------------------------------------------- introspection

def status_string(status: int) -> str:
    return load().mgemm_status_string(status).decode()


def variants():
    lib = load()
    out = []
    for i in range(lib.mgemm_num_variants()):
        info = VariantInfo()
        _check(lib.mgemm_variant(i, ctypes.byref(info)), "mgemm_variant")
        out.append(info.as_dict())
    return out


def select(in_dtype, transA, transB, M, N, K, alpha=1.0, A=0, lda=None, strideA=0, B=0,
           ldb=None, strideB=0, beta=0.0, C=0, ldc=None, strideC=0, batch=1, c_dtype=None):
    """(variant info dict, grid size) for a call with these arguments; raises on invalid ones.
    Pointers are plain integers here (alignment matters, contents do not).  c_dtype: C's type
    (mgemm_select_ex); None takes fp32 (int32 for int8, double for fp64 inputs)."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    lda = lda if lda is not None else (M if transA else K)
    ldb = ldb if ldb is not None else (K if transB else N)
    ldc = ldc if ldc is not None else N
    info = VariantInfo()
    grid = ctypes.c_int64()
    if c_dtype is None:
        st = load().mgemm_select(dt, int(transA), int(transB), M, N, K, alpha, A, lda, strideA, B,
                                 ldb, strideB, beta, C, ldc, strideC, batch, ctypes.byref(info),
                                 ctypes.byref(grid))
        _check(st, "mgemm_select")
    else:
        ct = DTYPE_CODES.get(c_dtype, c_dtype)
        st = load().mgemm_select_ex(dt, ct, int(transA), int(transB), M, N, K, alpha, A, lda,
                                    strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
                                    ctypes.byref(info), ctypes.byref(grid))
        _check(st, "mgemm_select_ex")
    return info.as_dict(), grid.value


def force_variant(in_dtype, variant_id: Optional[int]):
    """Pin every later call of this input type to one variant (None restores auto)."""
    dt = DTYPE_CODES.get(in_dtype, in_dtype)
    _check(load().mgemm_force_variant(dt, -1 if variant_id is None else int(variant_id)),
           "mgemm_force_variant")
