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

/* Operand kinds of mgemm_diag_mfma_ceiling. */
#define MGEMM_DIAG_F16 0   /* binary16, v_mfma_f32_32x32x16_f16 */
#define MGEMM_DIAG_BF16 1  /* bfloat16, v_mfma_f32_32x32x16_bf16 */
#define MGEMM_DIAG_I8 2    /* int8, v_mfma_i32_32x32x32_i8 (twice the operations) */

/* Register-only matrix-core throughput on caller-supplied operand values:
 * 256 workgroups x 4 wavefronts, each loading 32 16-byte-per-lane fragments
 * from `operands` once and then issuing iters x 64 independent MFMAs of the
 * given kind (MGEMM_DIAG_*), fp32 (int32 for int8) accumulate.
 * operands  device buffer of mgemm_diag_ceiling_operand_bytes() bytes, the
 *           16-bit or 8-bit values (read only).
 * out       device buffer of mgemm_diag_ceiling_out_floats() floats, written
 *           (one sum per lane, so the work is not optimised away).
 * The kernel is enqueued on `stream`; the caller times it (operation count:
 * mgemm_diag_ceiling_ops(kind, iters)).  Returns 0, 1 for a NULL buffer,
 * iters <= 0 or an unknown kind (nothing launched), 2 when the launch fails. */
int mgemm_diag_mfma_ceiling(int kind, const void *operands, float *out, int iters, hipStream_t stream);
int64_t mgemm_diag_ceiling_operand_bytes(void);
int64_t mgemm_diag_ceiling_out_floats(void);
double mgemm_diag_ceiling_flop(int iters);             /* 16-bit kinds */
double mgemm_diag_ceiling_ops(int kind, int iters);     /* any kind */

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_DIAG_H */
