/*
 * oracle_gemm.c -- the oracle: a plain, slow, obviously correct CPU GEMM in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * execute this file or the library built from it; only the tests, the smoke
 * check and the bench's CPU-baseline leg do.  It shares no code, header or
 * table with the HIP library.
 *
 * What it computes (the plain definition, nothing else):
 *
 *     C[m][n] = sum_{k=0}^{K-1} a(m,k) * b(k,n)        evaluated in fp64
 *
 *   - "An educational GEMM ladder for Helios GPUs", section "Educational GEMM
 *     Ladder": every rung computes C = AB with A in R^{MxK}, B in R^{KxN},
 *     C in R^{MxN}, BF16 inputs.
 *   - Same page, "Level 0 APIs" table: the matrix instruction accumulates the
 *     BF16 product into FP32 registers, and the store converts the FP32
 *     accumulator on its way to global memory.  The oracle keeps the sum in
 *     fp64 (every bf16*bf16 or fp16*fp16 product is exact in fp64) and rounds
 *     the exact result once, to nearest-even, when an fp16/bf16 output is
 *     asked for.
 *
 * Operand indexing (the pages speak of K-contiguous and N-contiguous operands,
 * "A Deep Dive into LDS Optimizations on AMD Instinct MI450 GPUs", Part I,
 * "Why Is It Important?"):
 *     layout 0 = K-contiguous :  a(m,k) = A[m*lda + k],  b(k,n) = B[n*ldb + k]
 *     layout 1 = MN-contiguous:  a(m,k) = A[k*lda + m],  b(k,n) = B[k*ldb + n]
 *     C is row-major:            C[m*ldc + n]
 * Leading dimensions count elements.
 *
 * Loop order m (OpenMP, static) -> k -> n, so the summation order over k is
 * fixed and the result is deterministic for any thread count.
 *
 * Element formats are decoded and encoded here from their IEEE-style
 * definitions (sign, biased exponent, stored fraction); no library conversion
 * is used:
 *     bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits
 *     fp16: 1 sign, 5 exponent (bias 15), 10 fraction bits
 *     e4m3: 1 sign, 4 exponent (bias 7), 3 fraction bits, one byte per
 *           element; the OCP 8-bit "E4M3" encoding, which has no infinities:
 *           exponent 15 with fraction 7 is NaN and every other pattern is
 *           finite (largest 448).  Only decoded: the oracle never produces
 *           fp8 outputs.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_E4M3 = 2 };
enum { ORACLE_K_CONTIG = 0, ORACLE_MN_CONTIG = 1 };

/* Decode a binary16-family pattern with `fbits` fraction bits and `ebits`
 * exponent bits into an exact double. */
static double decode_small_float(uint16_t bits, int ebits, int fbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int sign = (bits >> (ebits + fbits)) & 1;
    const int e = (bits >> fbits) & ((1 << ebits) - 1);
    const int f = bits & ((1 << fbits) - 1);
    double v;
    if (e == 0) {
        /* zero or subnormal: f * 2^(1 - bias - fbits) */
        v = ldexp((double)f, 1 - bias - fbits);
    } else if (e == (1 << ebits) - 1) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        /* normal: (2^fbits + f) * 2^(e - bias - fbits) */
        v = ldexp((double)((1 << fbits) + f), e - bias - fbits);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest binary16-family value, ties to even, and
 * return its bit pattern.  Overflow goes to infinity, tiny values to
 * subnormals or signed zero, NaN to the canonical quiet NaN. */
static uint16_t encode_small_float(double x, int ebits, int fbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias, emax = bias;
    const uint16_t sign = signbit(x) ? (uint16_t)(1u << (ebits + fbits)) : 0;
    const uint16_t exp_ones = (uint16_t)(((1u << ebits) - 1) << fbits);
    if (isnan(x))
        return (uint16_t)(exp_ones | (1u << (fbits - 1)));
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | exp_ones);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                  /* a = m' * 2^e, m' in [1, 2) */
    if (e < emin)
        e = emin;            /* subnormal range keeps the minimum spacing */
    const double q = ldexp(1.0, e - fbits);   /* spacing of representable values */
    const double r = rint(a / q);             /* a / q is exact; rint rounds half to even */
    const double v = r * q;
    if (v >= ldexp(1.0, emax + 1))
        return (uint16_t)(sign | exp_ones);   /* overflow */
    if (v < ldexp(1.0, emin)) {
        const uint32_t mant = (uint32_t)(v / ldexp(1.0, emin - fbits));
        return (uint16_t)(sign | mant);       /* subnormal or zero */
    }
    int e2;
    frexp(v, &e2);
    e2 -= 1;
    const uint32_t mant = (uint32_t)(v / ldexp(1.0, e2 - fbits)) - (1u << fbits);
    return (uint16_t)(sign | ((uint32_t)(e2 + bias) << fbits) | mant);
}

/* OCP E4M3: as the binary16 family for e < 15; e == 15 is a normal binade too,
 * except the all-ones pattern, which is NaN. */
double oracle_decode_e4m3(uint8_t bits)
{
    const int sign = (bits >> 7) & 1;
    const int e = (bits >> 3) & 15;
    const int f = bits & 7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, 1 - 7 - 3);             /* subnormal: f * 2^-9 */
    else
        v = ldexp((double)(8 + f), e - 7 - 3);       /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

double oracle_decode_bf16(uint16_t bits) { return decode_small_float(bits, 8, 7); }
double oracle_decode_f16(uint16_t bits) { return decode_small_float(bits, 5, 10); }
uint16_t oracle_encode_bf16(double x) { return encode_small_float(x, 8, 7); }
uint16_t oracle_encode_f16(double x) { return encode_small_float(x, 5, 10); }

/* Element i of a bf16/fp16 (two bytes each) or e4m3 (one byte) array. */
static double element(const void *p, int64_t i, int dtype)
{
    if (dtype == ORACLE_E4M3)
        return oracle_decode_e4m3(((const uint8_t *)p)[i]);
    const uint16_t bits = ((const uint16_t *)p)[i];
    return dtype == ORACLE_F16 ? oracle_decode_f16(bits) : oracle_decode_bf16(bits);
}

void oracle_decode_array(const void *in, double *out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = element(in, i, dtype);
}

void oracle_encode_array(const double *in, uint16_t *out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = dtype == ORACLE_F16 ? oracle_encode_f16(in[i]) : oracle_encode_bf16(in[i]);
}

static int check_args(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                      int layoutA, int layoutB, int dtype)
{
    if (M < 0 || N < 0 || K < 0)
        return 1;
    if ((layoutA != ORACLE_K_CONTIG && layoutA != ORACLE_MN_CONTIG) ||
        (layoutB != ORACLE_K_CONTIG && layoutB != ORACLE_MN_CONTIG))
        return 1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16 && dtype != ORACLE_E4M3)
        return 1;
    if (lda < (layoutA == ORACLE_K_CONTIG ? K : M))
        return 1;
    if (ldb < (layoutB == ORACLE_MN_CONTIG ? N : K))
        return 1;
    return 0;
}

static inline int64_t a_index(int64_t m, int64_t k, int64_t lda, int layoutA)
{
    return layoutA == ORACLE_K_CONTIG ? m * lda + k : k * lda + m;
}

static inline int64_t b_index(int64_t k, int64_t n, int64_t ldb, int layoutB)
{
    return layoutB == ORACLE_MN_CONTIG ? k * ldb + n : n * ldb + k;
}

/* Rows [row_begin, row_end) of C = A*B, written to C (row row_begin at C[0]).
 * nthreads <= 0 uses every available thread.  Returns 0 on success. */
int oracle_gemm_rows(const void *A, const void *B, double *C,
                     int64_t M, int64_t N, int64_t K,
                     int64_t lda, int64_t ldb, int64_t ldc,
                     int layoutA, int layoutB, int dtype,
                     int64_t row_begin, int64_t row_end, int nthreads)
{
    if (check_args(M, N, K, lda, ldb, layoutA, layoutB, dtype) || ldc < N ||
        row_begin < 0 || row_end > M || row_begin > row_end)
        return 1;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t m = row_begin; m < row_end; m++) {
        double *crow = C + (m - row_begin) * ldc;
        for (int64_t n = 0; n < N; n++)
            crow[n] = 0.0;
        for (int64_t k = 0; k < K; k++) {
            const double a = element(A, a_index(m, k, lda, layoutA), dtype);
            for (int64_t n = 0; n < N; n++)
                crow[n] += a * element(B, b_index(k, n, ldb, layoutB), dtype);
        }
    }
    return 0;
}

int oracle_gemm(const void *A, const void *B, double *C,
                int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                int layoutA, int layoutB, int dtype, int nthreads)
{
    return oracle_gemm_rows(A, B, C, M, N, K, lda, ldb, ldc, layoutA, layoutB, dtype,
                            0, M, nthreads);
}

/* Individual entries C[rows[i]][cols[i]], each the k-ordered fp64 dot product;
 * used to check outputs of problems too large for the full loop. */
int oracle_gemm_entries(const void *A, const void *B,
                        int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                        int layoutA, int layoutB, int dtype,
                        const int64_t *rows, const int64_t *cols, int64_t count,
                        double *out, int nthreads)
{
    if (check_args(M, N, K, lda, ldb, layoutA, layoutB, dtype))
        return 1;
    for (int64_t i = 0; i < count; i++)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N)
            return 1;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t i = 0; i < count; i++) {
        const int64_t m = rows[i], n = cols[i];
        double s = 0.0;
        for (int64_t k = 0; k < K; k++)
            s += element(A, a_index(m, k, lda, layoutA), dtype) *
                 element(B, b_index(k, n, ldb, layoutB), dtype);
        out[i] = s;
    }
    return 0;
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
