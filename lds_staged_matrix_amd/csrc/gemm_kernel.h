// gemm_kernel.h -- the LDS-staged BF16/FP16 GEMM kernel for gfx950.
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

#include "lds_layout.h"

namespace lsm {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef _Float16 v8f16 __attribute__((ext_vector_type(8)));
typedef float v16f32 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

enum { KC = 0, MNC = 1 };                       // operand contiguity, values of enum gemm_layout
enum { IN_BF16 = 0, IN_F16 = 1 };
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

template <int BM_, int BN_, int BK_, int WM_, int WN_, int GROUP_M_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WM = WM_, WN = WN_;                // wave grid inside the workgroup
  static constexpr int GROUP_M = GROUP_M_;                // tile rows per L2 group
  static constexpr int NT = WM * WN * 64;                  // threads per workgroup
  static constexpr int TM = BM / WM, TN = BN / WN;         // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;         // 32x32 fragments per wave
  static constexpr int KSTEPS = BK / 16;                   // MFMA k steps per K tile
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
};

// Geometry of one operand's LDS tile.  MN is the tile's M (for A) or N (for
// B) extent.  K-contiguous: MN rows of BK elements.  MN-contiguous: BK rows of
// MN elements.  "outer" is the strided dimension of the operand in memory,
// "inner" its unit-stride dimension.
template <int MN, int BK, int LAYOUT, int NT>
struct OperandTile {
  static constexpr bool kcontig = LAYOUT == KC;
  static constexpr int ROWS = kcontig ? MN : BK;                 // outer extent
  static constexpr int INNER = kcontig ? BK : MN;                // inner extent (elements)
  static constexpr int ROW_BYTES = 2 * INNER;
  static constexpr int CPR = ROW_BYTES / 16;                     // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROW_BYTES;
  static constexpr int CHUNKS = BYTES / 16;
  static constexpr int LOADS = CHUNKS / NT;                      // 16-byte loads per thread
  static constexpr int ROW_STEP = NT / CPR;                      // rows between a thread's loads
  static constexpr int SWZ_PERIOD = kcontig ? 16 : 4;            // rows after which the swizzle repeats
  static_assert(CHUNKS % NT == 0, "tile must split evenly into 16-byte loads");
  static_assert(NT % CPR == 0 && ROW_STEP % SWZ_PERIOD == 0,
                "a thread's chunks must share one swizzle phase");
};

template <int IN>
__device__ __forceinline__ v16f32 mfma_32x32x16(v8i16 a, v8i16 b, v16f32 c) {
  if constexpr (IN == IN_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf16, a),
                                                   __builtin_bit_cast(v8bf16, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8f16, a),
                                                  __builtin_bit_cast(v8f16, b), c, 0, 0, 0);
}

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

// One 32x32x16 operand fragment: lane l gets row/column (l & 31) of the
// fragment starting at `base`, k = 16*kk + 8*(l >> 5) + 0..7.
template <class OT>
__device__ __forceinline__ v8i16 read_frag(const char *lds, int lane, int base, int kk) {
  if constexpr (OT::kcontig) {
    return *(const v8i16 *)(lds + frag_kc_offset(lane, base, kk, OT::ROW_BYTES));
  } else {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(lds + frag_tr_offset(lane, base, kk, 0, OT::ROW_BYTES)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(lds + frag_tr_offset(lane, base, kk, 1, OT::ROW_BYTES)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <int OUT>
__device__ __forceinline__ void store_out(void *C, int64_t idx, float v) {
  if constexpr (OUT == OUT_F32) {
    ((float *)C)[idx] = v;
  } else if constexpr (OUT == OUT_BF16) {
    ((__bf16 *)C)[idx] = (__bf16)v;          // v_cvt_pk_bf16_f32: round to nearest even
  } else {
    ((_Float16 *)C)[idx] = (_Float16)v;      // v_cvt_f16_f32: round to nearest even
  }
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

  // Epilogue.  Accumulator register r of lane l holds row
  // 8*(r >> 2) + 4*(l >> 5) + (r & 3) and column (l & 31) of its 32x32 block
  // (layout checked with a probe).
  const bool interior = m_rem >= T::BM && n_rem >= T::BN;
  const int row0 = m0 + wm * T::TM + 4 * (lane >> 5);
  const int col0 = n0 + wn * T::TN + (lane & 31);
#pragma unroll
  for (int i = 0; i < T::FM; i++)
#pragma unroll
    for (int j = 0; j < T::FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
        const int col = col0 + 32 * j;
        if (interior || (row < M && col < N)) store_out<OUT>(C, (int64_t)row * ldc + col, acc[i][j][r]);
      }
}

}  // namespace lsm
