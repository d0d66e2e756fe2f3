// Host-side driver for the UBSan run of gemm_run's argument validation.
// Reads one request per line from stdin -- A B C M N K lda ldb ldc layoutA
// layoutB dtype, integers, pointers as plain addresses that are never
// dereferenced -- calls gemm_run with a stand-in handle on a device that
// does not exist, and prints the returned status, one per line.  Built with
// undefined-behaviour checks that abort on the first report.
#include <cstdint>
#include <cstdio>

#include "lds_gemm.h"

struct stand_in_handle {
  int device;   // no such device: requests that pass validation stop at the device check
};

int main() {
  stand_in_handle h{1 << 20};
  long long v[12];
  while (std::scanf("%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", &v[0], &v[1],
                    &v[2], &v[3], &v[4], &v[5], &v[6], &v[7], &v[8], &v[9], &v[10], &v[11]) == 12) {
    const int st = gemm_run(reinterpret_cast<gemm_handle_t>(&h), reinterpret_cast<const void *>(v[0]),
                            reinterpret_cast<const void *>(v[1]), reinterpret_cast<void *>(v[2]),
                            v[3], v[4], v[5], v[6], v[7], v[8], (int)v[9], (int)v[10], (int)v[11],
                            nullptr);
    std::printf("%d\n", st);
  }
  return 0;
}
