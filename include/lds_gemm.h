/*
 * lds_gemm.h -- C ABI of the LDS-staged BF16/FP16 GEMM for AMD Instinct
 * MI355X (gfx950, CDNA4).
 *
 * Operation (all entry points): C <- A * B, with
 *     C[m][n] = sum_{k<K} a(m,k) * b(k,n)
 * accumulated in fp32 by the matrix cores and converted once when stored.
 *   - "An educational GEMM ladder for Helios GPUs", section "Educational GEMM
 *     Ladder": each rung computes C = AB, A in R^{MxK}, B in R^{KxN},
 *     C in R^{MxN}, BF16 inputs.
 *   - Same page, "Level 0 APIs" table: the matrix instruction accumulates the
 *     16-bit product into FP32 registers; the store converts the FP32
 *     accumulator and writes it to global memory.
 *   - Operand contiguity: "A Deep Dive into LDS Optimizations on AMD Instinct
 *     MI450 GPUs", Part I, "Why Is It Important?" (a K-contiguous or an
 *     N-contiguous operand reaches the matrix cores through LDS).
 *
 * Layout of operands (leading dimensions count ELEMENTS, not bytes):
 *     layoutA == GEMM_K_CONTIG : a(m,k) = A[m*lda + k]   (row-major M x K)
 *     layoutA == GEMM_MN_CONTIG: a(m,k) = A[k*lda + m]   (column-major M x K)
 *     layoutB == GEMM_MN_CONTIG: b(k,n) = B[k*ldb + n]   (row-major K x N)
 *     layoutB == GEMM_K_CONTIG : b(k,n) = B[n*ldb + k]   (column-major K x N)
 *     C is row-major:            C[m*ldc + n]
 * Only the M x N entries of C are written; C memory between N and ldc is
 * left untouched.  Inputs beyond M, N or K are never read.
 *
 * Ownership and asynchrony: the caller owns A, B and C (device memory of the
 * handle's device) and keeps them alive until the work queued on `stream`
 * has finished.  The library never allocates, frees or retains caller
 * memory and allocates no workspace.  gemm_run only enqueues work on
 * `stream` and returns without synchronising the host; it launches kernels
 * and nothing else (no allocation, memset or copy), so a call made while
 * `stream` is being captured into a HIP graph is captured and replays.
 *
 * Errors: every function returns a gemm_status.  Arguments are validated
 * before anything is launched; on an error nothing is enqueued and C is
 * untouched.  No C++ exception crosses this interface.  Handles are
 * immutable after creation, so one handle may be used from several host
 * threads and streams at once.
 */
#ifndef LDS_GEMM_H
#define LDS_GEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_ctx *gemm_handle_t;

/* Which index of an operand is unit-stride in memory. */
enum gemm_layout {
    GEMM_K_CONTIG = 0,   /* K is contiguous (A row-major, B column-major)  */
    GEMM_MN_CONTIG = 1   /* M (for A) or N (for B) is contiguous           */
};

/* Element types, named input_output; accumulation is always fp32.
 * E4M3 is the OCP 8-bit floating-point format with 4 exponent bits (bias 7),
 * 3 fraction bits and no infinities, one byte per element; its products run
 * on the gfx950 fp8 matrix instruction ("Lds Optimization", "MFMA Transpose
 * Load from LDS (gfx950 only)": DS_READ_B64_TR_B8 feeds 8-bit MFMA
 * operands). */
enum gemm_dtype {
    GEMM_BF16_F32 = 0,   /* bf16 A, B;  fp32 C                             */
    GEMM_BF16_BF16 = 1,  /* bf16 A, B;  bf16 C (round to nearest even)     */
    GEMM_F16_F16 = 2,    /* fp16 A, B;  fp16 C (round to nearest even)     */
    GEMM_F16_F32 = 3,    /* fp16 A, B;  fp32 C                             */
    GEMM_E4M3_F32 = 4,   /* fp8 E4M3 A, B;  fp32 C                         */
    GEMM_E4M3_BF16 = 5   /* fp8 E4M3 A, B;  bf16 C (round to nearest even) */
};

enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,   /* bad enum, negative size, NULL pointer, ld too small, C overlaps A/B */
    GEMM_ERR_UNSUPPORTED = 2,   /* valid request the kernels cannot serve: misaligned pointer or ld, size of 2^30 or more, an operand spanning 2^63 bytes or more */
    GEMM_ERR_DEVICE = 3,        /* no device, not a gfx950 device, or the current device is not the handle's */
    GEMM_ERR_LAUNCH = 4         /* the HIP runtime rejected the kernel launch */
};

/* Create a handle bound to the calling thread's current HIP device.
 * Fails with GEMM_ERR_DEVICE unless that device is gfx950.  *out receives
 * the handle (NULL on failure); release it with gemm_destroy. */
int gemm_create(gemm_handle_t *out);

/* Enqueue C <- A*B on `stream` (0 = the device's null stream).
 *   A, B       device pointers to bf16/fp16 (2-byte) or E4M3 (1-byte)
 *              elements, 16-byte aligned; lda/ldb must be multiples of 16
 *              bytes (8 bf16/fp16 or 16 E4M3 elements).  E4M3 inputs further
 *              need the contiguous extents (K or M of A, N or K of B) to be
 *              multiples of 16 elements, else GEMM_ERR_UNSUPPORTED.
 *   C          device pointer to fp32 (4-byte aligned) or bf16/fp16
 *              (2-byte aligned) elements; must not overlap A or B.
 *   M, N, K    sizes, 0 <= size < 2^30; lda, ldb, ldc < 2^40; no operand may span 2^63 bytes
 *              or more ((rows - 1) * ld + row length, in bytes).  M == 0 or N == 0 is a no-op;
 *              K == 0 writes zeros (the empty sum) to the M x N block of C.
 *   lda        >= K (layoutA K-contig) or >= M (MN-contig)
 *   ldb        >= N (layoutB MN-contig) or >= K (K-contig)
 *   ldc        >= N
 *   layoutA/B  enum gemm_layout;  dtype  enum gemm_dtype.
 * Must be called with the handle's device current. */
int gemm_run(gemm_handle_t h, const void *A, const void *B, void *C,
             int64_t M, int64_t N, int64_t K,
             int64_t lda, int64_t ldb, int64_t ldc,
             int layoutA, int layoutB, int dtype, hipStream_t stream);

/* Release a handle.  NULL is accepted and returns GEMM_OK. */
int gemm_destroy(gemm_handle_t h);

/* Static English text for a gemm_status value ("unknown status" otherwise). */
const char *gemm_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* LDS_GEMM_H */
