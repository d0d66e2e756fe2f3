// gemm_kernel.h -- the register-staged LDS GEMM kernel for gfx950: the
// general path, valid for every shape, layout and alignment the C ABI accepts.
//
// One workgroup computes a BM x BN tile of C.  Per K step of BK:
//   1. every thread issues 128-bit global loads of its chunks of the next
//      A and B tiles into registers, coalesced along each operand's
//      unit-stride dimension;
//   2. each wave reads its MFMA fragments of the current tile from LDS --
//      ds_read_b128 for a K-contiguous operand, two ds_read_b64_tr_b16 for an
//      M/N-contiguous operand -- and issues v_mfma_f32_32x32x16_{bf16,f16};
//   3. the registers of step 1 are written with ds_write_b128 into the other
//      LDS stage at XOR-swizzled addresses;
//   4. one workgroup barrier hands the stages over.
// Two LDS stages let the fill of K step t+1 overlap the matrix work of step t
// ("An educational GEMM ladder for Helios GPUs", "Level 1: Double-Buffered in
// LDS": prologue, fill the inactive buffer while the matrix cores consume the
// current one, one barrier per K step).  The global loads are issued first
// and the LDS writes last, so the loads' latency is covered by the matrix
// work ("Lds Optimization", "Optimization Method 3: Increase Write-Read
// Distance": global loads for the next phase are the first thing to place
// between a write and its wait).  The epilogue converts the fp32 accumulators
// to the output type (round to nearest even) and masks the ragged edges of
// the tile in the same pass ("An educational GEMM ladder for Helios GPUs",
// "Level 0 APIs", store()).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"

namespace lsm {

// Load this thread's chunks of one operand tile into registers.  `p` points at
// the thread's first chunk.  When the tile is not wholly inside the matrix,
// rows at or beyond `outer_rem` read as zero and inner indices at or beyond
// `inner_rem` read as zero; nothing outside the matrix is touched.
template <class OT>
__device__ __forceinline__ void load_tile(u32x4 (&reg)[OT::LOADS], const uint16_t *p, int64_t ld,
                                          int outer0, int inner0, int outer_rem, int inner_rem) {
  const bool full = outer_rem >= OT::ROWS && inner_rem >= OT::INNER;   // uniform
  if (full) {
#pragma unroll
    for (int i = 0; i < OT::LOADS; i++)
      reg[i] = *(const u32x4 *)(p + (int64_t)(i * OT::ROW_STEP) * ld);
  } else {
#pragma unroll
    for (int i = 0; i < OT::LOADS; i++) {
      const int outer = outer0 + i * OT::ROW_STEP;
      const int nv = outer < outer_rem ? inner_rem - inner0 : 0;   // valid elements of the chunk
      const uint16_t *q = p + (int64_t)(i * OT::ROW_STEP) * ld;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (nv >= 8) {
        v = *(const u32x4 *)q;
      } else if (nv > 0) {
        unsigned short e[8];
#pragma unroll
        for (int j = 0; j < 8; j++) e[j] = j < nv ? q[j] : (unsigned short)0;
#pragma unroll
        for (int j = 0; j < 4; j++) v[j] = (unsigned)e[2 * j] | ((unsigned)e[2 * j + 1] << 16);
      }
      reg[i] = v;
    }
  }
}

template <class OT>
__device__ __forceinline__ void store_tile(char *lds, int off0, const u32x4 (&reg)[OT::LOADS]) {
#pragma unroll
  for (int i = 0; i < OT::LOADS; i++)
    *(u32x4 *)(lds + off0 + i * OT::ROW_STEP * OT::ROW_BYTES) = reg[i];
}

template <class T, int LA, int LB, int IN, int OUT>
__global__ __launch_bounds__(T::NT) void lds_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n) {
  using OA = OperandTile<T::BM, T::BK, LA, T::NT>;
  using OB = OperandTile<T::BN, T::BK, LB, T::NT>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if constexpr (LSM_LDS_POISON) {   // poison build: all of LDS, before any load or write
    lds_poison(smem, 2 * STAGE, tid, blockDim.x);
    __syncthreads();
  }
  const int wave = tid >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;

  int tm, tn;
  tile_coords(xcd_logical_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, T::GROUP_M, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int m_rem = M - m0, n_rem = N - n0;

  // This thread's first chunk of each operand tile (outer row, inner element).
  const int a_outer = loader_row(tid, OA::ROW_BYTES), a_inner = 8 * loader_chunk(tid, OA::ROW_BYTES);
  const int b_outer = loader_row(tid, OB::ROW_BYTES), b_inner = 8 * loader_chunk(tid, OB::ROW_BYTES);
  const int a_lds = loader_lds_offset(tid, OA::ROW_BYTES, OA::kcontig);
  const int b_lds = loader_lds_offset(tid, OB::ROW_BYTES, OB::kcontig);
  // Panel origins: K-contiguous A starts at row m0, M-contiguous A at column m0.
  const uint16_t *pa = (LA == KC ? A + (int64_t)m0 * lda : A + m0) + (int64_t)a_outer * lda + a_inner;
  const uint16_t *pb = (LB == KC ? B + (int64_t)n0 * ldb : B + n0) + (int64_t)b_outer * ldb + b_inner;
  // Moving one K tile: along the inner dimension (K-contig) or down BK rows (MN-contig).
  const int64_t a_kstep = LA == KC ? T::BK : (int64_t)T::BK * lda;
  const int64_t b_kstep = LB == KC ? T::BK : (int64_t)T::BK * ldb;

  u32x4 ra[OA::LOADS], rb[OB::LOADS];
  auto load_k_tile = [&](int kt) {
    const int k0 = kt * T::BK;
    if constexpr (LA == KC)
      load_tile<OA>(ra, pa + kt * a_kstep, lda, a_outer, a_inner, m_rem, K - k0);
    else
      load_tile<OA>(ra, pa + kt * a_kstep, lda, a_outer, a_inner, K - k0, m_rem);
    if constexpr (LB == KC)
      load_tile<OB>(rb, pb + kt * b_kstep, ldb, b_outer, b_inner, n_rem, K - k0);
    else
      load_tile<OB>(rb, pb + kt * b_kstep, ldb, b_outer, b_inner, K - k0, n_rem);
  };

  v16f32 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; i++)
#pragma unroll
    for (int j = 0; j < T::FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  const int KT = (K + T::BK - 1) / T::BK;
  if (KT > 0) {
    load_k_tile(0);
    store_tile<OA>(smem, a_lds, ra);
    store_tile<OB>(smem + OA::BYTES, b_lds, rb);
    __syncthreads();
  }

  for (int kt = 0; kt < KT; ++kt) {
    const char *sA = smem + (kt & 1) * STAGE;
    const char *sB = sA + OA::BYTES;
    const bool more = kt + 1 < KT;
    if (more) load_k_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < T::KSTEPS; ++kk) {
      v8i16 af[T::FM], bf[T::FN];
#pragma unroll
      for (int i = 0; i < T::FM; i++) af[i] = read_frag<OA>(sA, lane, wm * T::TM + 32 * i, kk);
#pragma unroll
      for (int j = 0; j < T::FN; j++) bf[j] = read_frag<OB>(sB, lane, wn * T::TN + 32 * j, kk);
#pragma unroll
      for (int i = 0; i < T::FM; i++)
#pragma unroll
        for (int j = 0; j < T::FN; j++) acc[i][j] = mfma_32x32x16<IN>(af[i], bf[j], acc[i][j]);
    }
    if (more) {
      char *dst = smem + ((kt + 1) & 1) * STAGE;
      store_tile<OA>(dst, a_lds, ra);
      store_tile<OB>(dst + OA::BYTES, b_lds, rb);
    }
    __syncthreads();
  }

  epilogue<T, OUT>(C, acc, M, N, ldc, m0, n0, wm, wn, lane);
}

}  // namespace lsm
