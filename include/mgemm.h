/*
 * mgemm -- dense row-major GEMM for AMD Instinct MI355X (gfx950).
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * The operation is the one defined on the page "Sgemm [128,128,8]"
 * (jianshu): C = alpha*A*B + beta*C with every matrix stored row-major
 * (the kernel's design comment, and host_gemm, its CPU reference).  op(X) is
 * X or its transpose: the transposed-operand form is the one the
 * "cuda11/matmul" tutorial (dlog.com.cn) reaches through einsum
 * 'bhqd,bhkd->bhqk' (section "Pytorch"), and the strided-batched form is its
 * bmm.  16-bit inputs with a float accumulator are the mixed-precision types
 * of the WMMA API page (adg.csdn.net), "1. 概述", element-type table.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  All matrices are row-major: element (r, c) of a matrix with
 *   leading dimension ld sits at base[r*ld + c].
 *   op(A) is M x K.  transA == MGEMM_OP_N: A is stored M x K, lda >= max(1,K).
 *                    transA == MGEMM_OP_T: A is stored K x M, lda >= max(1,M).
 *   op(B) is K x N.  transB == MGEMM_OP_N: B is stored K x N, ldb >= max(1,N).
 *                    transB == MGEMM_OP_T: B is stored N x K, ldb >= max(1,K).
 *   C is M x N, fp32, ldc >= max(1,N).
 *   Leading dimensions and batch strides are in elements.
 * Arithmetic.  Products and sums are fp32 (16-bit inputs are converted
 *   exactly); the summation order over k is unspecified but fixed, so
 *   repeated calls give identical bits.  Out-of-range parts of edge tiles
 *   contribute exactly zero (the residual-tile rule of the CSDN tile-algorithm
 *   page, "使用CUDA和瓦片算法计算矩阵乘法").  No saturation: IEEE inf/NaN.
 * beta == 0: C is write-only; its old contents (NaN included) are never read.
 * alpha == 0 or K == 0: C = beta * C; A and B are not read.
 * M == 0, N == 0 or batch == 0: nothing is launched; MGEMM_OK.
 * Ownership.  The caller owns A, B and C (device memory, e.g. from PyTorch).
 *   The library allocates and frees nothing and needs no handle; it
 *   may be called from several host threads at once.  gemm_splitk and
 *   gemm_streamk also take a caller-owned device workspace for their partial
 *   sums (its size comes from mgemm_splitk_plan / mgemm_streamk_plan;
 *   gemm_streamk's starts with arrival counters that must be zero), and
 *   gemm_splitk_noalloc uses a fixed per-GPU scratch inside the library; no
 *   other entry point uses memory beyond A, B and C.
 * Asynchrony.  Each call validates its arguments on the host, enqueues its
 *   kernels on `stream` (NULL = the default stream) and returns: one kernel,
 *   except gemm_splitk and gemm_splitk_noalloc with more than one chunk
 *   (the chunk products, then a reduction kernel).  Results are ready after
 *   the stream is synchronised; a workspace must not be reused by another
 *   call until the first call's kernels have finished (same stream: always).
 * Errors.  Invalid arguments are reported synchronously and nothing is
 *   launched: negative sizes, a leading dimension or stride below its
 *   minimum, a NULL pointer for an operand that will be read or written,
 *   a pointer not aligned to its element size, an unknown op or dtype,
 *   sizes beyond 2^31-1.  A failed launch returns MGEMM_HIP_ERROR.  Faults
 *   inside a kernel surface at the caller's next synchronisation.
 * Aliasing.  C must not overlap A or B.
 * Alignment.  Only element alignment is required; wider (16-byte) accesses
 *   are used when pointers, leading dimensions and strides allow them
 *   (rows aligned to 4 bytes are enough for all but a tile's last K-slab).
 */
#ifndef MGEMM_H
#define MGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MGEMM_OK = 0,
    MGEMM_INVALID_ARG = 1,
    MGEMM_HIP_ERROR = 2,
    MGEMM_SCRATCH_TOO_SMALL = 3  /* gemm_splitk_noalloc: partial sums exceed its fixed scratch */
} mgemm_status;

typedef enum { MGEMM_OP_N = 0, MGEMM_OP_T = 1 } mgemm_op;

typedef enum {
    MGEMM_F32 = 0,
    MGEMM_F16 = 1,
    MGEMM_BF16 = 2,
    MGEMM_I8 = 3,   /* int8 inputs (gemm_strided_batched_ex only) */
    MGEMM_I32 = 4,  /* int32 C of int8 inputs */
    MGEMM_F64 = 5   /* double A, B and C (gemm_f64* only) */
} mgemm_dtype;

/* Raw 16-bit storage: IEEE 754 binary16 and bfloat16 bit patterns. */
typedef uint16_t mgemm_f16;
typedef uint16_t mgemm_bf16;

/*
 * SGEMM: fp32 A, B, C; fp32 matrix-core products and fp32 accumulation.
 * Defined by "Sgemm [128,128,8]" (jianshu), design comment and host_gemm.
 */
mgemm_status gemm_f32(mgemm_op transA, mgemm_op transB,
                      int64_t M, int64_t N, int64_t K, float alpha,
                      const float *A, int64_t lda,
                      const float *B, int64_t ldb,
                      float beta, float *C, int64_t ldc,
                      hipStream_t stream);

/*
 * binary16 A and B, fp32 accumulation and fp32 C.
 * Input/accumulator pairing from the WMMA API page, "1. 概述" type table
 * (__half inputs, float accumulator).
 */
mgemm_status gemm_f16(mgemm_op transA, mgemm_op transB,
                      int64_t M, int64_t N, int64_t K, float alpha,
                      const mgemm_f16 *A, int64_t lda,
                      const mgemm_f16 *B, int64_t ldb,
                      float beta, float *C, int64_t ldc,
                      hipStream_t stream);

/*
 * bfloat16 A and B, fp32 accumulation and fp32 C.
 * Same table (__nv_bfloat16 inputs, float accumulator).
 */
mgemm_status gemm_bf16(mgemm_op transA, mgemm_op transB,
                       int64_t M, int64_t N, int64_t K, float alpha,
                       const mgemm_bf16 *A, int64_t lda,
                       const mgemm_bf16 *B, int64_t ldb,
                       float beta, float *C, int64_t ldc,
                       hipStream_t stream);

/*
 * Strided-batched GEMM: for b in [0, batch)
 *     C_b = alpha * op(A_b) * op(B_b) + beta * C_b,
 *     X_b = X + b * strideX   (element offsets, int64).
 * The bmm / einsum 'bhqd,bhkd->bhqk' forms of the "cuda11/matmul" tutorial
 * (dlog.com.cn), section "Pytorch".  in_dtype selects A/B's type (C is
 * always fp32).  strideA or strideB may be 0 (the operand is shared by every
 * batch entry); otherwise each must cover one operand matrix.  strideC must
 * cover one M x N matrix (C entries may not overlap).
 */
mgemm_status gemm_strided_batched(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB,
                                  int64_t M, int64_t N, int64_t K, float alpha,
                                  const void *A, int64_t lda, int64_t strideA,
                                  const void *B, int64_t ldb, int64_t strideB,
                                  float beta, float *C, int64_t ldc, int64_t strideC,
                                  int64_t batch, hipStream_t stream);

/*
 * Strided-batched GEMM with a choice of C type: as gemm_strided_batched, but
 * C (read when beta != 0, and written) has type c_dtype, which is either
 * MGEMM_F32 or the inputs' own 16-bit type (f16 -> f16, bf16 -> bf16; fp32
 * inputs take fp32 C only).  Accumulation stays fp32; alpha*acc + beta*C is
 * formed in fp32 and rounded to c_dtype to nearest, ties to even.
 * The "cuda11/matmul" tutorial (dlog.com.cn), section "Triton", converts its
 * fp32 accumulator to C's element type when storing; the WMMA API page's
 * fragment description lets the C/D matrices be __half.  A 16-bit C halves
 * the output traffic of store-bound shapes (attention scores with K = 64).
 *   C      device pointer, aligned to c_dtype's size; ldc, strideC in
 *          elements of c_dtype.
 * Errors: as gemm_strided_batched, plus MGEMM_INVALID_ARG for any other
 * c_dtype.
 *
 * int8 inputs (in_dtype = MGEMM_I8, the other precision row of the WMMA
 * page's type table, "1. 概述": 8-bit integer A/B with an int
 * accumulator): c_dtype must be MGEMM_I32; products accumulate exactly in
 * int32 and alpha*acc + beta*C is formed in 32-bit two's-complement
 * arithmetic (wrapping on overflow).  alpha and beta must be integers that
 * fit int32 (else MGEMM_INVALID_ARG).  Every transpose is accepted; an
 * MN-contiguous operand is read with transposing LDS reads, on tiles of
 * 128x128 and up (the 64x64 tiles serve transA = N, transB = T only).
 * lda, ldb, strides in elements (bytes); C aligned to 4 bytes.
 */
mgemm_status gemm_strided_batched_ex(mgemm_dtype in_dtype, mgemm_dtype c_dtype,
                                     mgemm_op transA, mgemm_op transB,
                                     int64_t M, int64_t N, int64_t K, float alpha,
                                     const void *A, int64_t lda, int64_t strideA,
                                     const void *B, int64_t ldb, int64_t strideB,
                                     float beta, void *C, int64_t ldc, int64_t strideC,
                                     int64_t batch, hipStream_t stream);

/*
 * DGEMM: double A, B, C, alpha and beta; double products and accumulation
 * on the matrix cores (v_mfma_f64_16x16x4_f64).  The double x double ->
 * double row of the WMMA API page's type table ("1. 概述").  Arguments,
 * layouts, quick returns, ownership and errors as gemm_f32, with elements of
 * 8 bytes (A, B, C aligned to 8; lda, ldb, ldc in elements).  Any leading
 * dimension works; 16-byte aligned operand rows (A and B aligned to 16 and
 * even lda, ldb) take the 16-byte load build.  The sum order differs from a
 * sequential loop, so results match an exact evaluation to within rounding,
 * and exactly whenever every partial sum is an integer below 2^53.
 */
mgemm_status gemm_f64(mgemm_op transA, mgemm_op transB,
                      int64_t M, int64_t N, int64_t K, double alpha,
                      const double *A, int64_t lda,
                      const double *B, int64_t ldb,
                      double beta, double *C, int64_t ldc,
                      hipStream_t stream);

/*
 * Strided-batched DGEMM: gemm_strided_batched's batch rules (int64 element
 * strides; strideA or strideB may be 0 to share the operand; strideC covers
 * one M x N matrix) with gemm_f64's types.  gemm_strided_batched and
 * gemm_strided_batched_ex, whose alpha and beta are float, refuse MGEMM_F64
 * with MGEMM_INVALID_ARG.
 */
mgemm_status gemm_f64_strided_batched(mgemm_op transA, mgemm_op transB,
                                      int64_t M, int64_t N, int64_t K, double alpha,
                                      const double *A, int64_t lda, int64_t strideA,
                                      const double *B, int64_t ldb, int64_t strideB,
                                      double beta, double *C, int64_t ldc, int64_t strideC,
                                      int64_t batch, hipStream_t stream);

/*
 * Split-K GEMM for under-filled shapes: the same
 * C = alpha * op(A) * op(B) + beta * C as the entry points above (the form
 * of "Sgemm [128,128,8]" (jianshu), design comment and host_gemm), computed
 * as K-chunks whose partial products spread over more of the device and
 * are then summed.  The pages size their tiles per
 * kernel through template parameters ("cuda11/matmul" tutorial, sections
 * V1-V3); a tile grid that leaves most of the 256 CUs idle, or holds too
 * few workgroups per CU to hide its loads, is the case this entry point is
 * for.
 *   in_dtype, c_dtype  as gemm_strided_batched_ex (fp32/f16/bf16 inputs with
 *          fp32 or the inputs' 16-bit C; int8 with int32 C), or MGEMM_F64
 *          for both.
 *   alpha, beta  double; for every in_dtype but MGEMM_F64 they must be
 *          exactly representable as float (else MGEMM_INVALID_ARG).
 *   splits  n > 1: about n chunks (whole K-slabs, so possibly fewer);
 *          1: the plain kernel; 0: automatic, which chunks
 *            - deep-K shapes (K >= 2 max(M, N)) whose 128x128 tiles leave
 *              CUs idle: enough chunks for 256 workgroups, each >= 512 deep;
 *            - grids of at most two rounds of 256 workgroups of an
 *              unaligned build (operand rows not 16-byte aligned) whose
 *              tile holds at least 5 us of matrix-core work: 3 chunks;
 *          and runs the plain kernel otherwise.  mgemm_splitk_plan reports
 *          which.
 *   workspace, workspace_bytes  device scratch owned by the caller, 16-byte
 *          aligned, at least mgemm_splitk_plan(...).workspace_bytes (0 when
 *          nothing is chunked; then workspace may be NULL).  It holds the
 *          chunks' partial products ([chunks][M][N]: fp32; int32 for int8;
 *          double for fp64) and is overwritten.  Calls that share a
 *          workspace must be ordered on one stream.
 * With chunks, two kernels run on `stream`: the chunked products, then a
 * reduction that adds the chunks in ascending order (deterministic),
 * applies alpha and beta (C read only when beta != 0) and rounds to C's
 * type.  Results differ from the one-pass kernels
 * only by fp32 (fp64) summation order, and are identical for
 * integer-valued inputs whose partial sums are exact.
 * Errors: as gemm_strided_batched_ex, plus MGEMM_INVALID_ARG for splits < 0
 * or a missing, misaligned or short workspace.
 */
mgemm_status gemm_splitk(mgemm_dtype in_dtype, mgemm_dtype c_dtype,
                         mgemm_op transA, mgemm_op transB,
                         int64_t M, int64_t N, int64_t K, double alpha,
                         const void *A, int64_t lda,
                         const void *B, int64_t ldb,
                         double beta, void *C, int64_t ldc,
                         int64_t splits, void *workspace, int64_t workspace_bytes,
                         hipStream_t stream);

/* gemm_splitk_noalloc -- gemm_splitk for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments, plan, kernels and
 * results as gemm_splitk, minus the workspace: the partial products go to a
 * fixed scratch array of MGEMM_NOALLOC_SCRATCH_BYTES in the library's own
 * device memory, one per GPU, held from the first call on that GPU until the
 * process ends.  The first call on a GPU looks the array's address up
 * (hipGetSymbolAddress); no call allocates or frees anything.
 *   stream  must belong to the calling thread's current device
 *          (MGEMM_INVALID_ARG otherwise).
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's partial sums (each call overwrites what it reads; nothing needs to
 * start at zero).  Calls that may run at the same time on one GPU (other
 * streams, other host threads) race on it: order them on one stream.
 * Errors: as gemm_splitk, plus MGEMM_SCRATCH_TOO_SMALL, before any device
 * call, when the plan's workspace_bytes (mgemm_splitk_plan) exceeds
 * MGEMM_NOALLOC_SCRATCH_BYTES; MGEMM_HIP_ERROR when the address lookup
 * fails. */
#define MGEMM_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
mgemm_status gemm_splitk_noalloc(mgemm_dtype in_dtype, mgemm_dtype c_dtype,
                                 mgemm_op transA, mgemm_op transB,
                                 int64_t M, int64_t N, int64_t K, double alpha,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 double beta, void *C, int64_t ldc,
                                 int64_t splits, hipStream_t stream);

/* Human-readable text for a status code (static storage). */
const char *mgemm_status_string(mgemm_status s);

/* ---------------------------------------------------------------------------
 * Introspection and tuning.  Pure host functions: no device is touched, so
 * they work on machines without a GPU.
 * ------------------------------------------------------------------------- */

/* Description of one compiled kernel variant (a tile shape). */
typedef struct {
    int id;            /* index accepted by mgemm_force_variant */
    int dtype;         /* mgemm_dtype of the inputs */
    int block_m;       /* output tile rows per workgroup */
    int block_n;       /* output tile columns per workgroup */
    int block_k;       /* K elements staged in LDS per pipeline step */
    int waves_m;       /* wavefronts along M */
    int waves_n;       /* wavefronts along N */
    int threads;       /* workgroup size */
    int lds_bytes;     /* LDS per workgroup */
    int pipe;          /* DMA-path schedule: 1 = four LDS stages of
                          block_k/2, 2 = two stages of block_k, 3 = one
                          stage of block_k (K <= block_k only), 4 = rows
                          4-byte aligned, two stages of block_k, 16-byte
                          copies but 4-byte ones on a tile's last slab
                          (every tile);
                          6 = small-problem kernel: one 16x16 tile per
                          workgroup, its waves_n waves sharing K, operands
                          through registers, K <= block_k */
    char name[64];     /* kernel family name, e.g. "mgemm_f32_256x256x32_w2x2" */
} mgemm_variant_info;

/* Number of compiled variants (all dtypes). */
int mgemm_num_variants(void);

/* How this copy of the library was built: 0 for the product build, or a set
 * of MGEMM_BUILD_* bits for a debug build of the same sources. */
#define MGEMM_BUILD_LDS_POISON 1  /* every LDS stage is filled with 0xFF before
                                     its first copy and after its last read
                                     (race check; slower) */
int mgemm_build_flags(void);

/* Fill *out for variant `id`; MGEMM_INVALID_ARG if id is out of range. */
mgemm_status mgemm_variant(int id, mgemm_variant_info *out);

/*
 * The variant (and launch grid size) a call with these arguments would use,
 * after the same validation the entry points perform.  Returns the
 * validation status; *out and *grid are set on MGEMM_OK (id = -1 and grid = 0
 * when the call would launch no GEMM kernel).  C is taken as fp32 (int32
 * for MGEMM_I8 inputs, double for MGEMM_F64).
 */
mgemm_status mgemm_select(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB,
                          int64_t M, int64_t N, int64_t K, float alpha,
                          const void *A, int64_t lda, int64_t strideA,
                          const void *B, int64_t ldb, int64_t strideB,
                          float beta, const float *C, int64_t ldc, int64_t strideC,
                          int64_t batch, mgemm_variant_info *out, int64_t *grid);

/*
 * mgemm_select for a C of type c_dtype, validated exactly as the entry points
 * validate that call: the pairs gemm_strided_batched_ex accepts (fp32 or the
 * inputs' own 16-bit type for 16-bit inputs, int32 for MGEMM_I8, double for
 * MGEMM_F64), C aligned to its own element size, alpha and beta as doubles
 * (integral for int8).  The variant chosen does not depend on C's type.
 */
mgemm_status mgemm_select_ex(mgemm_dtype in_dtype, mgemm_dtype c_dtype, mgemm_op transA,
                             mgemm_op transB, int64_t M, int64_t N, int64_t K, double alpha,
                             const void *A, int64_t lda, int64_t strideA,
                             const void *B, int64_t ldb, int64_t strideB,
                             double beta, const void *C, int64_t ldc, int64_t strideC,
                             int64_t batch, mgemm_variant_info *out, int64_t *grid);

/*
 * Force every later call of dtype `dtype` onto variant `id` (-1 restores the
 * automatic choice).  Process-wide; meant for tests and tile sweeps.
 * MGEMM_INVALID_ARG if the variant does not exist or has another dtype.
 */
mgemm_status mgemm_force_variant(mgemm_dtype dtype, int id);

/* What gemm_splitk will do for these arguments. */
typedef struct {
    int64_t workspace_bytes;   /* workspace the call needs (0: nothing chunked) */
    int64_t chunks;            /* K-chunks (1: the plain kernel) */
    int64_t chunk_len;         /* K per chunk; the last chunk takes the rest */
    mgemm_variant_info variant;  /* GEMM kernel launched: the chunked products or the
                                    plain kernel (id -1: none) */
    int64_t grid;              /* its workgroups */
} mgemm_splitk_plan_info;

/* Fill *out with gemm_splitk's plan for these arguments (A and B stand for
 * the operand addresses: their alignment matters, their contents do not).
 * Pure host; MGEMM_INVALID_ARG for splits < 0 or out == NULL. */
mgemm_status mgemm_splitk_plan(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB,
                               int64_t M, int64_t N, int64_t K,
                               const void *A, int64_t lda, const void *B, int64_t ldb,
                               int64_t splits, mgemm_splitk_plan_info *out);

/*
 * Stream-K GEMM: the same C = alpha * op(A) * op(B) + beta * C ("Sgemm
 * [128,128,8]" (jianshu), design comment and host_gemm), with the work cut
 * so that every workgroup gets an equal share whatever the tile count.  The
 * pages fix a tile per kernel ("cuda11/matmul" tutorial, sections V1-V3);
 * on 256 CUs a tile grid that is not a multiple of the CU count leaves the
 * last round part-empty (1000x1027: 272 tiles of 64x64), which is the case
 * this entry point is for.  The product is the list of (output tile, K
 * iteration) pairs; one launch of `workgroups` workgroups takes equal
 * consecutive ranges of it, writing whole tiles straight to C and the tiles
 * it splits as partial sums to the workspace.  Each workgroup that wrote
 * part of a split tile counts itself in on an arrival counter in the
 * workspace; the last to arrive adds the tile's partials in ascending K
 * (deterministic, whichever arrives last), applies alpha and beta, writes
 * C and leaves the counter at zero.  One kernel; nothing waits on another
 * workgroup.  It pays where the last round of tiles is mostly empty
 * (1000x1027x999 fp32: 272 tiles of 64x64); on grids that fill the device
 * the one-pass entry points are faster, and the automatic plan of
 * gemm_splitk does not choose it.
 *   in_dtype  MGEMM_F32 (c_dtype MGEMM_F32), MGEMM_F16 or MGEMM_BF16
 *          (c_dtype MGEMM_F32 or the inputs' own type: the partial sums stay
 *          fp32 and C is rounded once), MGEMM_I8 (c_dtype MGEMM_I32) or
 *          MGEMM_F64 (c_dtype MGEMM_F64, fp64 partial sums); other pairs
 *          give MGEMM_INVALID_ARG.
 *   alpha, beta  double; for every in_dtype but MGEMM_F64 exactly
 *          representable as float (int8: integral, as
 *          gemm_strided_batched_ex).
 *   workgroups  n > 0: n workgroups, capped at MGEMM_STREAMK_MAX_WORKGROUPS
 *          and at the number of (tile, iteration) pairs; 0: 512 (two per
 *          CU), capped likewise.
 *   workspace, workspace_bytes  device memory owned by the caller, 16-byte
 *          aligned, at least mgemm_streamk_plan(...).workspace_bytes (0 when
 *          no product is formed: M, N or K zero, or alpha zero, where at
 *          most C = beta * C runs; then it may be NULL).  Its first
 *          MGEMM_STREAMK_COUNTER_BYTES are arrival counters and MUST BE ZERO
 *          when the call's kernel starts: zero-fill a new workspace once
 *          (hipMemset, torch.zeros); every call leaves them zero when its
 *          kernel ends, so a workspace is then reusable by calls of any
 *          size without clearing.  Non-zero counters give wrong C for split
 *          tiles (never a hang).  The rest holds two partial tiles per
 *          workgroup, fp32 (int32 for int8, fp64 for fp64), overwritten.  Calls that share
 *          a workspace must be ordered on one stream.
 * A and B are read, C is read only when beta != 0; layouts, leading
 * dimensions and quick returns are those of gemm_strided_batched_ex with
 * batch 1.  Results differ from the one-pass kernels only by the summation
 * order (fp32; fp64 for fp64) where a tile is split, and are identical for
 * integer-valued inputs whose sums are exact.
 * Errors: as gemm_strided_batched_ex, plus MGEMM_INVALID_ARG for
 * workgroups < 0 or a missing, misaligned or short workspace; nothing is
 * launched then.
 */
#define MGEMM_STREAMK_COUNTER_BYTES ((int64_t)64 << 10)  /* zeroed prefix of a stream-K workspace */
#define MGEMM_STREAMK_MAX_WORKGROUPS ((int64_t)16384)     /* one 32-bit counter each */

mgemm_status gemm_streamk(mgemm_dtype in_dtype, mgemm_dtype c_dtype,
                          mgemm_op transA, mgemm_op transB,
                          int64_t M, int64_t N, int64_t K, double alpha,
                          const void *A, int64_t lda,
                          const void *B, int64_t ldb,
                          double beta, void *C, int64_t ldc,
                          int64_t workgroups, void *workspace, int64_t workspace_bytes,
                          hipStream_t stream);

/* What gemm_streamk will do for these arguments. */
typedef struct {
    int64_t workspace_bytes;   /* workspace the call needs (0: no product formed) */
    int64_t workgroups;        /* workgroups of the stream-K launch */
    int64_t tiles;             /* output tiles */
    int64_t iterations;        /* K-iterations per tile */
    int64_t k_per_iteration;   /* K elements per iteration (the last may be shorter) */
    mgemm_variant_info variant;  /* tile build (id -1: none) */
} mgemm_streamk_plan_info;

/* Fill *out with gemm_streamk's plan (A and B stand for the operand
 * addresses: their alignment matters, their contents do not).  Pure host;
 * MGEMM_INVALID_ARG for workgroups < 0, an unknown in_dtype, or out ==
 * NULL. */
mgemm_status mgemm_streamk_plan(mgemm_dtype in_dtype, mgemm_op transA, mgemm_op transB,
                                int64_t M, int64_t N, int64_t K,
                                const void *A, int64_t lda, const void *B, int64_t ldb,
                                int64_t workgroups, mgemm_streamk_plan_info *out);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_H */
