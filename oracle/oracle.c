/*
 * Oracle for dense GEMM, C = A.B -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load this
 * library.  It shares no code with the HIP path (no headers, helpers or tables) and
 * the HIP path never calls it.
 *
 * What it computes is the definition every page states: with A of size M x K and
 * B of size K x N, C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 * ("GEMM", Part 4 of How to make your models fast, opening formulas;
 *  "GEMM Optimization", section "The Problem").
 *
 * Precision.  Operands are fp32 values, bf16 bit patterns, IEEE binary16 (fp16) bit
 * patterns, or 8-bit floating-point bit patterns in one of the two OCP 8-bit formats
 * (E4M3 and E5M2; A and B may use different ones).  Each is widened exactly to double;
 * the product of two such values is exact in double (at most 24 + 24 significant bits),
 * and products are summed in double over k in ascending order.  fp16 is decoded from its fields as IEEE 754
 * defines binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction bits; exponent
 * 0 holds zero and the subnormals fraction * 2^-24, exponent 31 infinity and NaN);
 * the pages name fp16 only as another input type of the matrix cores, and fp8 likewise
 * ("A06 - Tiled Matrix Multiply (GEMM)", section "Matrix cores: MFMA and Tensor Cores": fp8 in,
 * fp32 accumulate) without fixing a format.  The 8-bit formats are decoded from their fields
 * as the OCP 8-bit floating point specification defines them: E4M3 has 1 sign, 4 exponent
 * bits with bias 7 and 3 fraction bits, no infinities, and only S.1111.111 is NaN (largest
 * value 448); E5M2 has 1 sign, 5 exponent bits with bias 15 and 2 fraction bits, with
 * infinities and NaNs at exponent 31 as in IEEE 754 (largest finite value 57344).  In both,
 * exponent 0 holds zero and the subnormals fraction * 2^(1 - bias - fraction bits).  The teaching module's lab does the same: its checker is a CPU
 * reference that accumulates in double ("A06 - Tiled Matrix Multiply (GEMM)",
 * section "Lab 1 - The optimization ladder", note on the tolerance).
 *
 * Alongside C the oracle returns D[i][j] = sum over k of |A[i][k] * B[k][j]|, the
 * scale the parity tolerance is normalised by: a result passes when
 * |C_gpu - C| / D <= tol element by element.
 *
 * Loop order i-k-j: one row of C is accumulated in double row buffers while k runs
 * ascending, so every C[i][j] sees its terms in the order k = 0, 1, ..., K-1.
 * OpenMP splits the rows i across threads; the per-element order does not depend on
 * the thread count.
 *
 * Layout.  Element (r, c) of a logical R x C operand with leading dimension ld sits
 * at r*ld + c (order 0, row-major) or at r + c*ld (order 1, column-major).
 * C and D are written dense row-major, M x N, as doubles.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2, ORACLE_E4M3 = 3, ORACLE_E5M2 = 4 };

static int valid_dtype(int dtype) { return dtype >= ORACLE_F32 && dtype <= ORACLE_E5M2; }

/* IEEE binary16 bit pattern -> its value */
static double f16_value(uint16_t h)
{
    const int sign = h >> 15, exp = (h >> 10) & 0x1f, frac = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)frac, -24);              /* zero and subnormals */
    else if (exp == 31)
        v = frac == 0 ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + frac), exp - 25); /* (1 + frac/1024) * 2^(exp-15) */
    return sign ? -v : v;
}

/* OCP E4M3 bit pattern -> its value */
static double e4m3_value(uint8_t b)
{
    const int sign = b >> 7, exp = (b >> 3) & 0xf, frac = b & 0x7;
    double v;
    if (exp == 15 && frac == 7)
        v = NAN;                                     /* the only NaN; no infinities */
    else if (exp == 0)
        v = ldexp((double)frac, -9);                 /* zero and subnormals */
    else
        v = ldexp((double)(8 + frac), exp - 10);     /* (1 + frac/8) * 2^(exp-7) */
    return sign ? -v : v;
}

/* OCP E5M2 bit pattern -> its value */
static double e5m2_value(uint8_t b)
{
    const int sign = b >> 7, exp = (b >> 2) & 0x1f, frac = b & 0x3;
    double v;
    if (exp == 31)
        v = frac == 0 ? INFINITY : NAN;
    else if (exp == 0)
        v = ldexp((double)frac, -16);                /* zero and subnormals */
    else
        v = ldexp((double)(4 + frac), exp - 17);     /* (1 + frac/4) * 2^(exp-15) */
    return sign ? -v : v;
}

/* one operand element, widened exactly to double */
static double element(const void *base, int dtype, int64_t r, int64_t c, int64_t ld, int order)
{
    int64_t at = (order == 0) ? r * ld + c : r + c * ld;
    if (dtype == ORACLE_F32) {
        return (double)((const float *)base)[at];
    } else if (dtype == ORACLE_F16) {
        return f16_value(((const uint16_t *)base)[at]);
    } else if (dtype == ORACLE_E4M3) {
        return e4m3_value(((const uint8_t *)base)[at]);
    } else if (dtype == ORACLE_E5M2) {
        return e5m2_value(((const uint8_t *)base)[at]);
    } else {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[at] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

/*
 * Full product.  Returns the number of multiply-adds performed in *macs
 * (M*N*K for a correct loop nest; FLOPs = 2*M*N*K, the count every page uses).
 * Returns 0 on success, -1 on a bad argument.
 */
int oracle_gemm_ab(int64_t M, int64_t N, int64_t K,
                   int dtype_a, const void *A, int64_t lda, int order_a,
                   int dtype_b, const void *B, int64_t ldb, int order_b,
                   double *C, double *D, int64_t *macs)
{
    if (M < 0 || N < 0 || K < 0 || !valid_dtype(dtype_a) || !valid_dtype(dtype_b))
        return -1;
    int64_t count = 0;
#pragma omp parallel reduction(+ : count)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *d = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) {
                s[j] = 0.0;
                d[j] = 0.0;
            }
            for (int64_t k = 0; k < K; ++k) {
                double a = element(A, dtype_a, i, k, lda, order_a);
                for (int64_t j = 0; j < N; ++j) {
                    double p = a * element(B, dtype_b, k, j, ldb, order_b);
                    s[j] += p;
                    d[j] += fabs(p);
                }
                count += N;
            }
            for (int64_t j = 0; j < N; ++j) {
                C[i * N + j] = s[j];
                D[i * N + j] = d[j];
            }
        }
        free(s);
        free(d);
    }
    if (macs)
        *macs = count;
    return 0;
}

/* Both operands of one type. */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int dtype,
                const void *A, int64_t lda, int order_a,
                const void *B, int64_t ldb, int order_b,
                double *C, double *D, int64_t *macs)
{
    return oracle_gemm_ab(M, N, K, dtype, A, lda, order_a, dtype, B, ldb, order_b, C, D, macs);
}

/*
 * Selected elements only: for each t < nsamp, C[t] and D[t] for the element
 * (rows[t], cols[t]).  Same arithmetic and order as the full product; used to check
 * outputs of problems too large for the full loop nest.
 */
int oracle_gemm_sampled_ab(int64_t M, int64_t N, int64_t K,
                           int dtype_a, const void *A, int64_t lda, int order_a,
                           int dtype_b, const void *B, int64_t ldb, int order_b,
                           const int64_t *rows, const int64_t *cols, int64_t nsamp,
                           double *C, double *D)
{
    if (M < 0 || N < 0 || K < 0 || nsamp < 0 || !valid_dtype(dtype_a) || !valid_dtype(dtype_b))
        return -1;
    for (int64_t t = 0; t < nsamp; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
            return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < nsamp; ++t) {
        double s = 0.0, d = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = element(A, dtype_a, rows[t], k, lda, order_a) *
                       element(B, dtype_b, k, cols[t], ldb, order_b);
            s += p;
            d += fabs(p);
        }
        C[t] = s;
        D[t] = d;
    }
    return 0;
}

int oracle_gemm_sampled(int64_t M, int64_t N, int64_t K, int dtype,
                        const void *A, int64_t lda, int order_a,
                        const void *B, int64_t ldb, int order_b,
                        const int64_t *rows, const int64_t *cols, int64_t nsamp,
                        double *C, double *D)
{
    return oracle_gemm_sampled_ab(M, N, K, dtype, A, lda, order_a, dtype, B, ldb, order_b, rows, cols, nsamp,
                                  C, D);
}

/* Threads OpenMP will use (reported with CPU timings). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
