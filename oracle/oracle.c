/*
 * Oracle for dense row-major GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product library (libmgemm) never
 * calls it, and the two share no source, header, table or helper.
 *
 * What it computes (plain definition, no blocking, no reordering):
 *
 *   for every batch b, row i < M, column j < N:
 *       acc      = sum_{k = 0 .. K-1, ascending}  (double) opA[i][k] * (double) opB[k][j]
 *       out[i,j] = alpha * acc + beta * C[i,j]      (the beta term is dropped when beta == 0)
 *
 * Sources on the pages:
 *   - the GEMM form C = alpha*A*B + beta*C with every matrix row-major:
 *     "Sgemm [128,128,8]" (jianshu), the kernel's design comment and the
 *     host_gemm CPU reference that checks it;
 *   - the triple loop with a scalar accumulator:
 *     "cuda11/matmul" tutorial (dlog.com.cn), section "什么是矩阵乘法"
 *     (what matrix multiplication is), the CPU sgemm;
 *   - op(A)/op(B) with an explicit stride per matrix ("matrices may be
 *     non-contiguous"): same tutorial, section "Triton", the wrapper that
 *     passes strides;
 *   - half and bfloat16 operands with a float accumulator, 8-bit integer
 *     operands with an int accumulator, and double operands with a double
 *     accumulator:
 *     WMMA API page (adg.csdn.net), "1. 概述", the element-type table.
 *
 * Readings taken where the pages are silent (each listed in the design doc):
 *   - accumulation is fp64 (the pages accumulate in the element type; the
 *     exact fp64 sum of fp32 products is the stricter reference);
 *   - C is not read when beta == 0 (so NaN in C does not leak);
 *   - alpha == 0 or K == 0 gives beta * C; M, N or batch == 0 does nothing;
 *   - 16-bit inputs are decoded exactly from their bit patterns.
 *
 * Floating-point determinism: every product of two fp32 (or 16-bit) values
 * is exact in fp64 (24 + 24 < 53 mantissa bits), and the sum runs over k in
 * ascending order.  The file must be built with -ffp-contract=off so that
 * the epilogue alpha*acc + beta*c is never fused.
 *
 * Double operands (ORACLE_F64) take the same loop one precision up: the
 * products and the sum are formed in IEEE binary128 (gcc's __float128, 113
 * significand bits, where a product of two doubles is exact as a product of
 * two floats is exact in fp64), then alpha*acc + beta*C in binary128, and
 * the result is rounded once to double.  C is then double as well.
 *
 * Parallelism: OpenMP over output rows only.  Each output element is still
 * computed by exactly the loop above, so the thread count cannot change a bit.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2
#define ORACLE_I8 3   /* int8 A/B; C (when read) is int32 */
#define ORACLE_F64 5  /* double A/B/C; accumulation in binary128 */

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 encodes zero and subnormals (fraction * 2^-24),
 * exponent 31 encodes infinities and NaNs. */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * Exponent 0 encodes zero and subnormals (fraction * 2^-133). */
double oracle_bf16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xff;
    int frac = h & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

/* Nearest value of a binary format with `fbits` fraction bits, minimum
 * normal exponent `emin` and maximum exponent `emax` (IEEE 754
 * roundTiesToEven), as its bit pattern.  Values past the largest finite
 * number by half an ulp or more become infinity; NaN becomes a quiet NaN.
 * Used for 16-bit C: the result alpha*acc + beta*C converted to C's element
 * type on store ("cuda11/matmul" tutorial, section "Triton"). */
static uint16_t round_to_format(double x, int fbits, int ebits, int emin, int emax)
{
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const uint16_t inf = (uint16_t)(((1u << ebits) - 1) << fbits);
    if (isnan(x)) return (uint16_t)(inf | (1u << (fbits - 1)));
    const double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                          /* a in [2^(e-1), 2^e) */
    const int q = (e - 1 < emin ? emin : e - 1) - fbits;  /* exponent of one ulp there */
    const double v = ldexp(rint(ldexp(a, -q)), q);        /* rint: nearest, ties to even */
    if (v >= ldexp(1.0, emax + 1)) return (uint16_t)(sign | inf);
    if (v < ldexp(1.0, emin))              /* subnormal: fraction = v / 2^(emin - fbits) */
        return (uint16_t)(sign | (uint16_t)ldexp(v, fbits - emin));
    frexp(v, &e);                          /* v = 1.f * 2^(e-1) */
    const uint16_t frac = (uint16_t)(ldexp(v, fbits - (e - 1)) - ldexp(1.0, fbits));
    return (uint16_t)(sign | (uint16_t)((e - 1 + emax) << fbits) | frac);  /* bias = emax */
}

uint16_t oracle_double_to_f16(double x) { return round_to_format(x, 10, 5, -14, 15); }

uint16_t oracle_double_to_bf16(double x) { return round_to_format(x, 7, 8, -126, 127); }

/* Element-wise rounding of n values to dtype (ORACLE_F16 or ORACLE_BF16). */
int oracle_round16(int dtype, const double *in, uint16_t *out, int64_t n)
{
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e)
        out[e] = dtype == ORACLE_F16 ? oracle_double_to_f16(in[e]) : oracle_double_to_bf16(in[e]);
    return ORACLE_OK;
}

/* Element (r, c) of a row-major matrix with leading dimension ld, widened. */
static double load_elem(int dtype, const void *base, int64_t r, int64_t c, int64_t ld)
{
    int64_t off = r * ld + c;
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[off];
    if (dtype == ORACLE_F16)
        return oracle_f16_to_double(((const uint16_t *)base)[off]);
    if (dtype == ORACLE_I8)
        return (double)((const int8_t *)base)[off];
    return oracle_bf16_to_double(((const uint16_t *)base)[off]);
}

/* Element of C (fp32, or int32 for int8 inputs); both are 4 bytes wide. */
static double load_c(int dtype, const void *C, int64_t off)
{
    if (dtype == ORACLE_I8) return (double)((const int32_t *)C)[off];
    return (double)((const float *)C)[off];
}

/* op(A)[i][k]: A is stored M x K (transA == 0) or K x M (transA == 1). */
static double op_a(int dtype, const void *A, int transA, int64_t i, int64_t k, int64_t lda)
{
    return transA ? load_elem(dtype, A, k, i, lda) : load_elem(dtype, A, i, k, lda);
}

/* op(B)[k][j]: B is stored K x N (transB == 0) or N x K (transB == 1). */
static double op_b(int dtype, const void *B, int transB, int64_t k, int64_t j, int64_t ldb)
{
    return transB ? load_elem(dtype, B, j, k, ldb) : load_elem(dtype, B, k, j, ldb);
}

static size_t elem_size(int dtype)
{
    return dtype == ORACLE_F64 ? 8 : dtype == ORACLE_F32 ? 4 : dtype == ORACLE_I8 ? 1 : 2;
}

/* C's element size: double for double inputs, otherwise 4 (fp32 or int32). */
static size_t c_elem_size(int dtype) { return dtype == ORACLE_F64 ? 8 : 4; }

/* Element (r, c) of a row-major double matrix, widened to binary128 (exact). */
static __float128 load_f64(const void *base, int64_t r, int64_t c, int64_t ld)
{
    return (__float128)((const double *)base)[r * ld + c];
}

/* One output element for double operands: the definition in binary128,
 * rounded to double at the end. */
static double one_element_f64(int transA, int transB, int64_t K, double alpha,
                              const void *A, int64_t lda, const void *B, int64_t ldb,
                              double beta, const void *C, int64_t ldc, int64_t i, int64_t j)
{
    __float128 acc = 0;
    for (int64_t k = 0; k < K; ++k) {
        const __float128 a = transA ? load_f64(A, k, i, lda) : load_f64(A, i, k, lda);
        const __float128 b = transB ? load_f64(B, j, k, ldb) : load_f64(B, k, j, ldb);
        acc += a * b;
    }
    __float128 out = (__float128)alpha * acc;
    if (beta != 0.0)
        out = out + (__float128)beta * (__float128)((const double *)C)[i * ldc + j];
    return (double)out;
}

/* One output element, exactly as the definition at the top of this file. */
static double one_element(int dtype, int transA, int transB, int64_t K, double alpha,
                          const void *A, int64_t lda, const void *B, int64_t ldb,
                          double beta, const void *C, int64_t ldc,
                          int64_t i, int64_t j)
{
    if (dtype == ORACLE_F64)
        return one_element_f64(transA, transB, K, alpha, A, lda, B, ldb, beta, C, ldc, i, j);
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += op_a(dtype, A, transA, i, k, lda) * op_b(dtype, B, transB, k, j, ldb);
    double out = alpha * acc;
    if (beta != 0.0)
        out = out + beta * load_c(dtype, C, i * ldc + j);
    return out;
}

static int check_args(int dtype, int transA, int transB, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, int64_t batch)
{
    if ((dtype < ORACLE_F32 || dtype > ORACLE_I8) && dtype != ORACLE_F64) return ORACLE_BAD_ARG;
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return ORACLE_BAD_ARG;
    if (M < 0 || N < 0 || K < 0 || batch < 0) return ORACLE_BAD_ARG;
    if (lda < (transA ? M : K) || ldb < (transB ? K : N) || ldc < N) return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

/*
 * Full output: out[b*strideO + i*ldo + j] for every b < batch, i < M, j < N.
 * A, B, C of batch b start at base + b*stride (in elements).
 * C may be NULL when beta == 0.
 */
int oracle_gemm(int dtype, int transA, int transB,
                int64_t M, int64_t N, int64_t K, double alpha,
                const void *A, int64_t lda, int64_t strideA,
                const void *B, int64_t ldb, int64_t strideB,
                double beta, const void *C, int64_t ldc, int64_t strideC,
                int64_t batch, double *out, int64_t ldo, int64_t strideO)
{
    if (check_args(dtype, transA, transB, M, N, K, lda, ldb, ldc, batch) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    if (ldo < N) return ORACLE_BAD_ARG;
    if (beta != 0.0 && C == NULL) return ORACLE_BAD_ARG;
    size_t es = elem_size(dtype);
    int64_t rows = batch * M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t b = row / M, i = row % M;
        const char *Ab = (const char *)A + (size_t)(b * strideA) * es;
        const char *Bb = (const char *)B + (size_t)(b * strideB) * es;
        const char *Cb = C ? (const char *)C + (size_t)(b * strideC) * c_elem_size(dtype) : NULL;
        for (int64_t j = 0; j < N; ++j)
            out[b * strideO + i * ldo + j] =
                one_element(dtype, transA, transB, K, alpha, Ab, lda, Bb, ldb,
                            beta, Cb, ldc, i, j);
    }
    return ORACLE_OK;
}

/*
 * Selected elements only: out[e] is element (bidx[e], iidx[e], jidx[e]),
 * computed by the same definition.  Used for full-size problems where the
 * whole output would take too long on the host.
 */
int oracle_gemm_elems(int dtype, int transA, int transB,
                      int64_t M, int64_t N, int64_t K, double alpha,
                      const void *A, int64_t lda, int64_t strideA,
                      const void *B, int64_t ldb, int64_t strideB,
                      double beta, const void *C, int64_t ldc, int64_t strideC,
                      int64_t batch, int64_t count,
                      const int64_t *bidx, const int64_t *iidx, const int64_t *jidx,
                      double *out)
{
    if (check_args(dtype, transA, transB, M, N, K, lda, ldb, ldc, batch) != ORACLE_OK)
        return ORACLE_BAD_ARG;
    if (beta != 0.0 && C == NULL) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < count; ++e)
        if (bidx[e] < 0 || bidx[e] >= batch || iidx[e] < 0 || iidx[e] >= M ||
            jidx[e] < 0 || jidx[e] >= N)
            return ORACLE_BAD_ARG;
    size_t es = elem_size(dtype);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t e = 0; e < count; ++e) {
        int64_t b = bidx[e];
        const char *Ab = (const char *)A + (size_t)(b * strideA) * es;
        const char *Bb = (const char *)B + (size_t)(b * strideB) * es;
        const char *Cb = C ? (const char *)C + (size_t)(b * strideC) * c_elem_size(dtype) : NULL;
        out[e] = one_element(dtype, transA, transB, K, alpha, Ab, lda, Bb, ldb,
                             beta, Cb, ldc, iidx[e], jidx[e]);
    }
    return ORACLE_OK;
}

/* int32 C of int8 inputs: the exact integer result taken modulo 2^32 into
 * [-2^31, 2^31) (two's-complement wrapping).  Each input must be an integer
 * of magnitude below 2^53 (exact in fp64); otherwise ORACLE_BAD_ARG. */
int oracle_wrap_i32(const double *in, int32_t *out, int64_t n)
{
    for (int64_t e = 0; e < n; ++e) {
        const double x = in[e];
        if (!(fabs(x) < 9007199254740992.0) || x != floor(x)) return ORACLE_BAD_ARG;
        const int64_t v = (int64_t)x;
        out[e] = (int32_t)(uint32_t)((uint64_t)v & 0xffffffffu);
    }
    return ORACLE_OK;
}

/* Thread count of the OpenMP loops above (timing only: results do not
 * depend on it, since threads split whole output elements). */
void oracle_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
