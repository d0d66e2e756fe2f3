// gemm_api.hip -- the C ABI declared in include/lds_gemm.h: argument
// validation, choice of kernel and tile shape, and the launch on the
// caller's stream.  The kernels: the ping-pong kernel (gemm_kernel_pingpong.h,
// shapes with at least 256 tiles of 256 x 256), the direct-to-LDS kernel
// (gemm_kernel_dma.h, 128 and 64 tiles), the split-K ring kernel
// (gemm_kernel_skinny.h, M <= 32) and the register-staged kernel
// (gemm_kernel.h, shapes the 16-byte direct-to-LDS loads cannot take).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "gemm_kernel.h"
#include "gemm_kernel_dma.h"
#include "gemm_kernel_pingpong.h"
#include "gemm_kernel_skinny.h"
#include "lds_gemm.h"

struct gemm_ctx {
  int device;
};

namespace lsm {

// Tile shapes.  GROUP_M is the number of tile rows walked together so that
// workgroups resident on one XCD share A and B panels in its L2.
//   Big:    256 x 256 x 64, 8 waves (2 per SIMD), each wave 128 x 64.
//           LDS 2 stages x 64 KiB = 128 KiB.
//   Mid:    128 x 128 x 64, 4 waves of 64 x 64.  LDS 64 KiB.
//   Small:  64 x 64 x 64, 4 waves of 32 x 32.  LDS 32 KiB.
//   Skinny: 32 x 64 x 64, 2 waves of 32 x 32 for M <= 32.  LDS 24 KiB.
using Big = Tile<256, 256, 64, 2, 4, 8>;
using Mid = Tile<128, 128, 64, 2, 2, 8>;
using Small = Tile<64, 64, 64, 2, 2, 4>;
using Skinny = Tile<32, 64, 64, 1, 2, 8>;
// Direct-to-LDS kernel shapes: 4 waves (one per SIMD).
//   DmaMid: 128 x 128 x 64, wave tile 64 x 64, LDS 2 x 32 KiB.
using DmaMid = Tile<128, 128, 64, 2, 2, 8>;
//   DmaSmall: 64 x 64 x 64, wave tile 32 x 32, LDS 2 x 16 KiB.
using DmaSmall = Tile<64, 64, 64, 2, 2, 8>;
// Ping-pong kernel: 256 x 256 x 64, 8 waves in two groups, wave tile 128 x 64.
using PingPong = Tile<256, 256, 64, 2, 4, 8>;
// Split-K ring kernel, M <= 32: 32 x 64 column slabs, K stages of 128, a
// ring of 6 stages (144 KiB), 4 waves splitting each stage's K range.
// LSM_RING_STAGES overrides the ring depth only for the A/B build that
// measures what the depth buys; the library is built with 6.
#ifndef LSM_RING_STAGES
#define LSM_RING_STAGES 6
#endif
using SkinnyStream = SkinnyTile<32, 64, 128, LSM_RING_STAGES>;
// 8-bit (E4M3) inputs: the same tiles in bytes, so BK doubles in elements.
using PingPong8 = Tile<256, 256, 128, 2, 4, 8>;
using DmaMid8 = Tile<128, 128, 128, 2, 2, 8>;
using DmaSmall8 = Tile<64, 64, 128, 2, 2, 8>;
using SkinnyStream8 = SkinnyTile<32, 64, 256, LSM_RING_STAGES>;

struct Args {
  const uint16_t *A;
  const uint16_t *B;
  void *C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  uint32_t a_bytes, b_bytes;   // operand footprints (used by the direct-to-LDS kernel)
};

// DMA4: the direct-to-LDS kernel with four LDS stages (operand panels beyond the L2).
enum Kind { REG = 0, DMA = 1, PINGPONG = 2, SKINNY = 3, DMA4 = 4 };

// The ping-pong kernel's 16-bit instances run on v_mfma_f32_16x16x32 and its
// E4M3 instances on v_mfma_scale_f32_16x16x128_f8f6f4.  LSM_PP_MFMA = 32 and
// LSM_PP_MFMA8 = 32 build them with the 32 x 32 forms instead (32x32x16,
// 32x32x64); they exist only for the A/B build that measures the MFMA shape.
// The library is built with 16.
#ifndef LSM_PP_MFMA
#define LSM_PP_MFMA 16
#endif
#ifndef LSM_PP_MFMA8
#define LSM_PP_MFMA8 16
#endif

template <class T, int KIND, int LA, int LB, int IN, int OUT>
static hipError_t launch_dma(const Args &a, hipStream_t stream) {
  int tiles_m = (a.M + T::BM - 1) / T::BM;
  int tiles_n = (a.N + T::BN - 1) / T::BN;
  const uint16_t *A = a.A, *B = a.B;
  void *C = a.C;
  int M = a.M, N = a.N, K = a.K;
  int64_t lda = a.lda, ldb = a.ldb, ldc = a.ldc;
  uint32_t ab = a.a_bytes, bb = a.b_bytes;
  // 16-byte C stores (LDS-staged epilogue) need C and every row start aligned
  constexpr int64_t esz = OUT == OUT_F32 ? 4 : 2;
  int c_vec = ((uintptr_t)C % 16 == 0) && ((ldc * esz) % 16 == 0);
  void *params[] = {&A, &B, &C, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &ab, &bb, &c_vec};
  const void *fn;
  if constexpr (KIND == PINGPONG)
    fn = (const void *)lds_gemm_pingpong_kernel<T, LA, LB, IN, OUT,
                                                IN == IN_E4M3 ? LSM_PP_MFMA8 : LSM_PP_MFMA>;
  else if constexpr (KIND == DMA4)
    fn = (const void *)lds_gemm_dma_kernel<T, LA, LB, IN, OUT, 4>;
  else
    fn = (const void *)lds_gemm_dma_kernel<T, LA, LB, IN, OUT>;
  return hipLaunchKernel(fn, dim3((unsigned)(tiles_m * tiles_n)), dim3(T::NT), params, 0, stream);
}

template <class T, int LA, int LB, int IN, int OUT>
static hipError_t launch_skinny(const Args &a, hipStream_t stream) {
  int tiles_m = (a.M + T::BM - 1) / T::BM;
  int tiles_n = (a.N + T::BN - 1) / T::BN;
  const uint16_t *A = a.A, *B = a.B;
  void *C = a.C;
  int M = a.M, N = a.N, K = a.K;
  int64_t lda = a.lda, ldb = a.ldb, ldc = a.ldc;
  uint32_t ab = a.a_bytes, bb = a.b_bytes;
  void *params[] = {&A, &B, &C, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n, &ab, &bb};
  return hipLaunchKernel((const void *)lds_gemm_skinny_kernel<T, LA, LB, IN, OUT>,
                         dim3((unsigned)(tiles_m * tiles_n)), dim3(T::NT), params, 0, stream);
}

template <class T, int LA, int LB, int IN, int OUT>
static hipError_t launch(const Args &a, hipStream_t stream) {
  int tiles_m = (a.M + T::BM - 1) / T::BM;
  int tiles_n = (a.N + T::BN - 1) / T::BN;
  const uint16_t *A = a.A, *B = a.B;
  void *C = a.C;
  int M = a.M, N = a.N, K = a.K;
  int64_t lda = a.lda, ldb = a.ldb, ldc = a.ldc;
  void *params[] = {&A, &B, &C, &M, &N, &K, &lda, &ldb, &ldc, &tiles_m, &tiles_n};
  return hipLaunchKernel((const void *)lds_gemm_kernel<T, LA, LB, IN, OUT>,
                         dim3((unsigned)(tiles_m * tiles_n)), dim3(T::NT), params, 0, stream);
}

template <class T, int KIND, int LA, int LB, int IN, int OUT>
static hipError_t launch_kind(const Args &a, hipStream_t s) {
  if constexpr (KIND == REG)
    return launch<T, LA, LB, IN, OUT>(a, s);
  else if constexpr (KIND == SKINNY)
    return launch_skinny<T, LA, LB, IN, OUT>(a, s);
  else
    return launch_dma<T, KIND, LA, LB, IN, OUT>(a, s);
}

template <class T, int DMA, int IN, int OUT>
static hipError_t launch_layout(const Args &a, int la, int lb, hipStream_t s) {
  if (la == KC && lb == KC) return launch_kind<T, DMA, KC, KC, IN, OUT>(a, s);
  if (la == KC && lb == MNC) return launch_kind<T, DMA, KC, MNC, IN, OUT>(a, s);
  if (la == MNC && lb == KC) return launch_kind<T, DMA, MNC, KC, IN, OUT>(a, s);
  return launch_kind<T, DMA, MNC, MNC, IN, OUT>(a, s);
}

template <class T, int DMA = REG>
static hipError_t launch_dtype(const Args &a, int la, int lb, int dtype, hipStream_t s) {
  switch (dtype) {
    case GEMM_BF16_F32: return launch_layout<T, DMA, IN_BF16, OUT_F32>(a, la, lb, s);
    case GEMM_BF16_BF16: return launch_layout<T, DMA, IN_BF16, OUT_BF16>(a, la, lb, s);
    case GEMM_F16_F16: return launch_layout<T, DMA, IN_F16, OUT_F16>(a, la, lb, s);
    default: return launch_layout<T, DMA, IN_F16, OUT_F32>(a, la, lb, s);
  }
}

template <class T, int DMA>
static hipError_t launch_fp8(const Args &a, int la, int lb, int dtype, hipStream_t s) {
  if (dtype == GEMM_E4M3_F32) return launch_layout<T, DMA, IN_E4M3, OUT_F32>(a, la, lb, s);
  return launch_layout<T, DMA, IN_E4M3, OUT_BF16>(a, la, lb, s);
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static bool is_fp8(int dtype) { return dtype == GEMM_E4M3_F32 || dtype == GEMM_E4M3_BF16; }

// The direct-to-LDS kernels need whole 16-byte chunks along each operand's
// contiguous dimension, and byte offsets (footprint plus one tile of rows of
// overhang, plus a K advance) below 2^31 for their 32-bit buffer offsets.
static bool offsets_fit_31_bits(int64_t outer, int64_t ld, int64_t es, int64_t K) {
  int64_t r;
  return !__builtin_mul_overflow(outer + 512, ld, &r) && !__builtin_mul_overflow(r, es, &r) &&
         !__builtin_add_overflow(r, es * K, &r) && r < ((int64_t)1 << 31);
}

static bool dma_ok(const Args &a, int la, int lb, int64_t es) {
  const int64_t a_inner = la == KC ? a.K : a.M, a_outer = la == KC ? a.M : a.K;
  const int64_t b_inner = lb == MNC ? a.N : a.K, b_outer = lb == MNC ? a.K : a.N;
  return (a_inner * es) % 16 == 0 && (b_inner * es) % 16 == 0 &&
         offsets_fit_31_bits(a_outer, a.lda, es, a.K) &&
         offsets_fit_31_bits(b_outer, a.ldb, es, a.K);
}

// One XCD's L2 on MI355X.
constexpr int64_t kL2BytesPerXcd = (int64_t)4 << 20;

// The 64 x 64 tile takes four LDS stages when the operand panels that one
// XCD's workgroups read over the whole K range do not fit in its L2: its K
// steps are short (four MFMAs per wave and K tile, two for 8-bit inputs), so
// with the loads only one tile ahead it waits on the longer latency of loads
// the L2 misses.  Measured on MI355X (kernel traces): 512 x 512 x 4096 and
// 1024 x 1024 x 4096 take 22 us with four stages against 31 us with two;
// while the panels fit, four stages are 11-16% slower.
// LSM_SMALL_FOUR_STAGES = 0 (an A/B build only) keeps the double buffer for
// every shape; the library is built with 1.
#ifndef LSM_SMALL_FOUR_STAGES
#define LSM_SMALL_FOUR_STAGES 1
#endif
static bool small_tile_four_stages(const Args &a, int64_t es) {
  if (!LSM_SMALL_FOUR_STAGES) return false;
  const long long panel = 64LL * a.K * es;
  return xcd_max_panel_bytes((int)ceil_div(a.M, 64), (int)ceil_div(a.N, 64), 8, panel, panel) >
         kL2BytesPerXcd;
}

// Shape classes.  M <= 32 takes the split-K ring kernel (HBM-bound).
// Otherwise the big tile when it still gives every CU at least one
// workgroup, else the 128 tile when that does, else the 64 tile (a short,
// latency-bound K loop per workgroup; more workgroups hide more of it),
// with four LDS stages when its operand panels overflow the L2.
// Shapes whose contiguous extents are not whole 16-byte chunks (dma_ok()
// false) take the register-staged kernel of the same class.
// 8-bit inputs run on the direct-to-LDS kernels only (gemm_run rejects fp8
// shapes those cannot take).
static hipError_t dispatch(const Args &a, int la, int lb, int dtype, hipStream_t s) {
  const int64_t t256 = ceil_div(a.M, 256) * ceil_div(a.N, 256);
  const int64_t t128 = ceil_div(a.M, 128) * ceil_div(a.N, 128);
  if (is_fp8(dtype)) {
    if (a.M <= 32) return launch_fp8<SkinnyStream8, SKINNY>(a, la, lb, dtype, s);
    if (t256 >= 256) return launch_fp8<PingPong8, PINGPONG>(a, la, lb, dtype, s);
    if (t128 >= 256) return launch_fp8<DmaMid8, DMA>(a, la, lb, dtype, s);
    if (small_tile_four_stages(a, 1)) return launch_fp8<DmaSmall8, DMA4>(a, la, lb, dtype, s);
    return launch_fp8<DmaSmall8, DMA>(a, la, lb, dtype, s);
  }
  const bool dma = dma_ok(a, la, lb, 2);
  if (dma) {
    if (a.M <= 32) return launch_dtype<SkinnyStream, SKINNY>(a, la, lb, dtype, s);
    if (t256 >= 256) return launch_dtype<PingPong, PINGPONG>(a, la, lb, dtype, s);
    if (t128 >= 256) return launch_dtype<DmaMid, DMA>(a, la, lb, dtype, s);
    if (small_tile_four_stages(a, 2)) return launch_dtype<DmaSmall, DMA4>(a, la, lb, dtype, s);
    return launch_dtype<DmaSmall, DMA>(a, la, lb, dtype, s);
  }
  if (a.M <= 32) return launch_dtype<Skinny>(a, la, lb, dtype, s);
  if (t256 >= 256) return launch_dtype<Big>(a, la, lb, dtype, s);
  if (t128 >= 64) return launch_dtype<Mid>(a, la, lb, dtype, s);
  return launch_dtype<Small>(a, la, lb, dtype, s);
}

// Bytes spanned by `outer` rows of `inner` elements of `es` bytes at leading
// dimension `ld`, i.e. ((outer - 1) * ld + inner) * es, or -1 when that does
// not fit in 63 bits (no such buffer can exist).
static int64_t footprint_bytes(int64_t outer, int64_t ld, int64_t inner, int64_t es) {
  int64_t r;
  if (__builtin_mul_overflow(outer - 1, ld, &r) || __builtin_add_overflow(r, inner, &r) ||
      __builtin_mul_overflow(r, es, &r))
    return -1;
  return r;
}

static bool ranges_overlap(const void *p, int64_t pbytes, const void *q, int64_t qbytes) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)pbytes;
}

}  // namespace lsm

extern "C" {

#if LSM_PP_TIMELINE
// Measurement builds only: install (or, with NULL, remove) the buffer the
// ping-pong kernel writes its per-wave phase cycles to, 64 counts per
// workgroup of the launch.  0 on success, -1 on a HIP error.
int lsm_pp_timeline_set(void *buf) {
  return hipMemcpyToSymbol(HIP_SYMBOL(lsm::pp_timeline_buf), &buf, sizeof(buf)) == hipSuccess ? 0 : -1;
}
#endif

int gemm_create(gemm_handle_t *out) {
  if (!out) return GEMM_ERR_INVALID_ARG;
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_DEVICE;
  gemm_ctx *h = new (std::nothrow) gemm_ctx{dev};
  if (!h) return GEMM_ERR_DEVICE;
  *out = h;
  return GEMM_OK;
}

int gemm_destroy(gemm_handle_t h) {
  delete h;
  return GEMM_OK;
}

const char *gemm_status_str(int status) {
  switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "unsupported argument (alignment or size)";
    case GEMM_ERR_DEVICE: return "device is not a usable gfx950 device";
    case GEMM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int gemm_run(gemm_handle_t h, const void *A, const void *B, void *C, int64_t M, int64_t N,
             int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int layoutA, int layoutB,
             int dtype, hipStream_t stream) {
  using namespace lsm;
  if (!h) return GEMM_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
  if ((layoutA != GEMM_K_CONTIG && layoutA != GEMM_MN_CONTIG) ||
      (layoutB != GEMM_K_CONTIG && layoutB != GEMM_MN_CONTIG))
    return GEMM_ERR_INVALID_ARG;
  if (dtype < GEMM_BF16_F32 || dtype > GEMM_E4M3_BF16) return GEMM_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return GEMM_OK;
  if (!C || (K > 0 && (!A || !B))) return GEMM_ERR_INVALID_ARG;

  const int64_t a_outer = layoutA == GEMM_K_CONTIG ? M : K;
  const int64_t a_inner = layoutA == GEMM_K_CONTIG ? K : M;
  const int64_t b_outer = layoutB == GEMM_MN_CONTIG ? K : N;
  const int64_t b_inner = layoutB == GEMM_MN_CONTIG ? N : K;
  if (lda < a_inner || ldb < b_inner || ldc < N || lda < 1 || ldb < 1)
    return GEMM_ERR_INVALID_ARG;

  const int64_t kMaxDim = (int64_t)1 << 30;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return GEMM_ERR_UNSUPPORTED;
  // the grid of the smallest tile (32 x 64) must fit a 31-bit workgroup count
  if (ceil_div(M, 32) * ceil_div(N, 64) >= ((int64_t)1 << 31)) return GEMM_ERR_UNSUPPORTED;
  if (lda >= ((int64_t)1 << 40) || ldb >= ((int64_t)1 << 40) || ldc >= ((int64_t)1 << 40))
    return GEMM_ERR_UNSUPPORTED;
  const int64_t out_size =
      (dtype == GEMM_BF16_F32 || dtype == GEMM_F16_F32 || dtype == GEMM_E4M3_F32) ? 4 : 2;
  const int64_t es = is_fp8(dtype) ? 1 : 2;             // input element bytes
  if (K > 0) {
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((lda * es) & 15) || ((ldb * es) & 15))
      return GEMM_ERR_UNSUPPORTED;
  }
  if ((uintptr_t)C & (uintptr_t)(out_size - 1)) return GEMM_ERR_UNSUPPORTED;

  const int64_t c_bytes = footprint_bytes(M, ldc, N, out_size);
  const int64_t a_fp = K > 0 ? footprint_bytes(a_outer, lda, a_inner, es) : 0;
  const int64_t b_fp = K > 0 ? footprint_bytes(b_outer, ldb, b_inner, es) : 0;
  if (c_bytes < 0 || a_fp < 0 || b_fp < 0) return GEMM_ERR_UNSUPPORTED;
  if (K > 0 && (ranges_overlap(C, c_bytes, A, a_fp) || ranges_overlap(C, c_bytes, B, b_fp)))
    return GEMM_ERR_INVALID_ARG;

  const Args args{(const uint16_t *)A, (const uint16_t *)B, C, (int)M, (int)N, (int)K,
                  lda, ldb, ldc, (uint32_t)(a_fp < ((int64_t)1 << 31) ? a_fp : 0),
                  (uint32_t)(b_fp < ((int64_t)1 << 31) ? b_fp : 0)};
  // 8-bit inputs need the direct-to-LDS kernels: whole 16-element chunks
  // along both contiguous extents and 32-bit buffer offsets.
  if (is_fp8(dtype) && !dma_ok(args, layoutA, layoutB, 1)) return GEMM_ERR_UNSUPPORTED;

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) return GEMM_ERR_DEVICE;
  if (dispatch(args, layoutA, layoutB, dtype, stream) != hipSuccess) return GEMM_ERR_LAUNCH;
  return GEMM_OK;
}

}  // extern "C"
