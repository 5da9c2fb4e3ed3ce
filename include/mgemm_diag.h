/*
 * mgemm_diag -- measurement aids for the benchmark, built into
 * libmgemm_diag.so beside libmgemm.so.  Nothing here computes a GEMM.
 */
#ifndef MGEMM_DIAG_H
#define MGEMM_DIAG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Register-only matrix-core throughput on caller-supplied 16-bit operand
 * values: 256 workgroups x 4 wavefronts, each loading 32 16-byte-per-lane
 * fragments from `operands` once and then issuing iters x 64 independent
 * 32x32x16 MFMAs (bf16 != 0: bfloat16, else binary16), fp32 accumulate.
 * operands  device buffer of mgemm_diag_ceiling_operand_bytes() bytes, the
 *           16-bit values (read only).
 * out       device buffer of mgemm_diag_ceiling_out_floats() floats, written
 *           (one sum per lane, so the work is not optimised away).
 * The kernel is enqueued on `stream`; the caller times it (flop count:
 * mgemm_diag_ceiling_flop(iters)).  Returns 0, 1 for a NULL buffer or
 * iters <= 0 (nothing launched), 2 when the launch fails. */
int mgemm_diag_mfma_ceiling(int bf16, const void *operands, float *out, int iters, hipStream_t stream);
int64_t mgemm_diag_ceiling_operand_bytes(void);
int64_t mgemm_diag_ceiling_out_floats(void);
double mgemm_diag_ceiling_flop(int iters);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_DIAG_H */
