/* The C ABI used from plain C (C11, no C++): create a handle, run
 * C = A*B for all-ones bf16 operands (every entry of C is exactly K, the
 * closed form of an all-ones product), check the status codes of a few
 * invalid calls, destroy the handle.  Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "lds_gemm.h"

#define CHECK_HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
    fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); return 2; } } while (0)

int main(void) {
  const int64_t M = 200, N = 136, K = 264;
  gemm_handle_t h = NULL;
  int st = gemm_create(&h);
  if (st != GEMM_OK) {
    fprintf(stderr, "gemm_create: %s\n", gemm_status_str(st));
    return 1;
  }
  const size_t na = (size_t)(M * K), nb = (size_t)(K * N), nc = (size_t)(M * N);
  uint16_t *ha = malloc(na * 2), *hb = malloc(nb * 2);
  float *hc = malloc(nc * 4);
  if (!ha || !hb || !hc) return 2;
  for (size_t i = 0; i < na; i++) ha[i] = 0x3F80; /* bf16 1.0 */
  for (size_t i = 0; i < nb; i++) hb[i] = 0x3F80;
  void *da, *db, *dc;
  CHECK_HIP(hipMalloc(&da, na * 2));
  CHECK_HIP(hipMalloc(&db, nb * 2));
  CHECK_HIP(hipMalloc(&dc, nc * 4));
  CHECK_HIP(hipMemcpy(da, ha, na * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(db, hb, nb * 2, hipMemcpyHostToDevice));
  st = gemm_run(h, da, db, dc, M, N, K, K, N, N, GEMM_K_CONTIG, GEMM_MN_CONTIG, GEMM_BF16_F32, 0);
  if (st != GEMM_OK) {
    fprintf(stderr, "gemm_run: %s\n", gemm_status_str(st));
    return 1;
  }
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(hc, dc, nc * 4, hipMemcpyDeviceToHost));
  size_t bad = 0;
  for (size_t i = 0; i < nc; i++) bad += hc[i] != (float)K;
  /* invalid calls: rejected before any launch */
  int e1 = gemm_run(h, da, db, dc, -1, N, K, K, N, N, 0, 1, 0, 0);
  int e2 = gemm_run(h, da, db, dc, M, N, K, K, N, N, 0, 1, 99, 0);
  int e3 = gemm_run(NULL, da, db, dc, M, N, K, K, N, N, 0, 1, 0, 0);
  st = gemm_destroy(h);
  hipFree(da);
  hipFree(db);
  hipFree(dc);
  free(ha);
  free(hb);
  free(hc);
  printf("C ABI from C: %zu of %zu entries differ from K; invalid calls -> %d %d %d; destroy -> %d\n",
         bad, nc, e1, e2, e3, st);
  return (bad == 0 && e1 == GEMM_ERR_INVALID_ARG && e2 == GEMM_ERR_INVALID_ARG &&
          e3 == GEMM_ERR_INVALID_ARG && st == GEMM_OK) ? 0 : 1;
}
