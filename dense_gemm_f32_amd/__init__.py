"""MI355X-native dense row-major GEMM.

    C = alpha * op(A) * op(B) + beta * C      (fp32, f16 or bf16 A/B; fp32 accumulate;
                                               fp32 C, or 16-bit C of the inputs' type;
                                               int8 A/B with int32 C; fp64 throughout)

Python binding over the C-ABI library libmgemm.so (include/mgemm.h): the
functions below forward to the C entry points of the same names.  All the
arithmetic runs in the library's HIP kernels for gfx950; PyTorch only
provides device memory and streams.  ``torch_ops`` maps torch tensors
(row-major or transposed views, batch strides) onto the same entry points:
mm, bmm, matmul and attention_scores.
"""
from ._lib import (BF16, F16, F32, F64, I8, I32, NOALLOC_SCRATCH_BYTES, STREAMK_COUNTER_BYTES,
                   STREAMK_MAX_WORKGROUPS, OP_N, OP_T, MgemmError,
                   force_variant, gemm_bf16, gemm_f16, gemm_f32, gemm_f64,
                   gemm_f64_strided_batched, gemm_splitk, gemm_splitk_noalloc, gemm_streamk, gemm_strided_batched, gemm_strided_batched_ex, load, select,
                   splitk_chunks, splitk_plan, splitk_workspace_bytes, status_string, streamk_plan,
                   variants)
from . import torch_ops

__all__ = ["gemm_f32", "gemm_f16", "gemm_bf16", "gemm_f64", "gemm_strided_batched",
           "gemm_strided_batched_ex", "gemm_f64_strided_batched", "gemm_splitk",
           "gemm_splitk_noalloc", "NOALLOC_SCRATCH_BYTES", "STREAMK_COUNTER_BYTES",
           "STREAMK_MAX_WORKGROUPS", "splitk_chunks",
           "splitk_plan", "splitk_workspace_bytes", "gemm_streamk", "streamk_plan", "select",
           "variants",
           "force_variant", "status_string", "load", "MgemmError", "OP_N", "OP_T", "F32", "F16",
           "BF16", "I8", "I32", "F64", "torch_ops"]
