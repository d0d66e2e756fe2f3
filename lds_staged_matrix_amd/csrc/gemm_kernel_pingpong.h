// gemm_kernel_pingpong.h -- LDS-staged GEMM with direct-to-LDS loads and a
// two-group ping-pong schedule, for gfx950.
//
// Eight waves, two per SIMD, in two groups of four (waves 0-3 and 4-7; wave
// w runs on SIMD w mod 4).  Each wave owns a 128 x 64 block of the 256 x 256
// workgroup tile.  The groups alternate between two kinds of phase,
// separated by workgroup barriers:
//   memory phase  M(t): read every MFMA fragment of K tile t from LDS into
//                       registers (group 0 also starts the direct-to-LDS
//                       loads of tile t+1);
//   compute phase C(t): the 32 MFMAs of tile t, from registers only.
// Group 1 starts one phase late, so while one wave of a SIMD issues MFMAs the
// other wave of that SIMD moves data.  On gfx950 an MFMA stream and LDS->VGPR
// returns overlap when they come from different waves of a SIMD, and mostly
// serialize when one wave interleaves both (measured on MI355X with a
// microbenchmark; the pages report the same scheduling family -- four-wave
// interleave and eight- or sixteen-wave ping-pong -- working on MI355X,
// "An educational GEMM ladder for Helios GPUs", Summary).
//
// Barrier b (0-based, all eight waves):
//   b = 0          after the prologue loads of tiles 0 and 1 (tile 0 landed)
//   group 0: M(t) ... b = 2t+1 ... C(t) ... b = 2t+2
//   group 1: idle ... b = 1; then M(t) ... b = 2t+2 ... C(t) ... b = 2t+3
// Group 1 skips the barrier after its last compute phase, so both groups
// pass 2*KT + 1 barriers.
// LDS hazards (tile t lives in stage t & 1):
//  * stage t&1 is read between barriers 2t and 2t+2; the loads of tile t+2
//    into it start after barrier 2t+2 (group 0, during M(t+1));
//  * every wave waits for its own LDS reads before the barrier that ends its
//    memory phase, and group 0 waits for its loads (vmcnt(0)) before the
//    barrier that ends its compute phase, so tile t+1 is complete at barrier
//    2t+2, before any wave reads it.
// Loads of tile t+1 therefore have two phases (64 MFMAs per SIMD) to land.
//
// The LDS layout, the swizzle on the global side of the loads, the edge
// handling through buffer range checks and the inline-assembly loads are
// those of gemm_kernel_dma.h.
//
// MF selects the MFMA shape: 16 (the library: v_mfma_f32_16x16x32 for 16-bit
// and v_mfma_scale_f32_16x16x128_f8f6f4 for E4M3 inputs, each wave's 128 x 64
// block as 8 x 4 blocks of 16 x 16) or 32 (v_mfma_f32_32x32x16 and
// v_mfma_scale_f32_32x32x64_f8f6f4, an A/B build).  Both read the same LDS
// bytes per K tile.  On MI355X, at its 1400 W socket limit on random
// operands, the 16 x 16 instructions spend less energy per flop (a quarter of
// the accumulator register traffic per instruction for half the work), so the
// chip holds a higher clock: 8192^3 bf16 runs about 5% faster with them.
// Their transposed reads need their own swizzles (mn16_swizzle and
// mn16_swizzle8 in lds_layout.h), which take two lane offsets per loader.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"
#include "gemm_kernel_dma.h"

namespace lsm {

// The library stages C through LDS for the whole workgroup at once
// (epilogue_lds_rows); LSM_PP_ROW_EPI = 0, an A/B build only, stages it per
// wave (epilogue_lds) instead.
#ifndef LSM_PP_ROW_EPI
#define LSM_PP_ROW_EPI 1
#endif

__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Ping-pong tile: 256 x 256 x 64, waves 2 (M) x 4 (N), wave tile 128 x 64.
template <class T, int LA, int LB, int IN, int OUT, int MF = 32>
__global__ __launch_bounds__(T::NT, 1) void lds_gemm_pingpong_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n,
    uint32_t a_bytes, uint32_t b_bytes, int c_vec) {
  static_assert(T::WM == 2 && T::NT == 512, "two groups of four waves");
  static_assert(MF == 32 || MF == 16, "32 x 32 or 16 x 16 MFMAs");
  using L = AccLayout<MF>;
  constexpr int LOADERS = T::NT / 2;                     // group 0 issues every load
  constexpr int ES = InT<IN>::ES;
  // MFMA k-steps per K tile (a 16 x 16 MFMA is twice as deep as a 32 x 32 one)
  constexpr int KSTEPS = T::BK / (MF == 32 ? InT<IN>::KSTEP : 2 * InT<IN>::KSTEP);
  constexpr int FM = T::TM / MF, FN = T::TN / MF;        // MFMA blocks per wave
  // With 16 x 16 MFMAs an MN-contiguous tile takes the layout of those
  // fragments' transposed reads, with two lane offsets per loader.
  using OA = OperandTile<T::BM, T::BK, LA, LOADERS, ES, MF == 16>;
  using OB = OperandTile<T::BN, T::BK, LB, LOADERS, ES, MF == 16>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int LOADS_PER_TILE = OA::LOADS + OB::LOADS;  // per group-0 wave
  constexpr int FRAGS = KSTEPS * (FM + FN);               // fragment reads per memory phase
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if constexpr (LSM_LDS_POISON) {   // poison build: all of LDS, before any load or write
    lds_poison(smem, 2 * STAGE, tid, blockDim.x);
    __syncthreads();
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;                           // 0: waves 0-3, 1: waves 4-7
  const int wm = group, wn = wave & 3;

  int tm, tn;
  tile_coords(xcd_logical_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, T::GROUP_M, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  const i32x4 rsA = buffer_rsrc(A, a_bytes);
  const i32x4 rsB = buffer_rsrc(B, b_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

  // Loader geometry for group 0 (tid < LOADERS).
  int a_inner, b_inner, unused;
  const uint32_t a_voff = dma_lane_offset<OA>(tid & (LOADERS - 1), m0, M, lda, a_bytes, a_inner);
  const uint32_t b_voff = dma_lane_offset<OB>(tid & (LOADERS - 1), n0, N, ldb, b_bytes, b_inner);
  // offsets of the load rounds of the second swizzle phase (the same as the
  // first unless the tile takes two lane offsets)
  const uint32_t a_voff1 = OA::LANE_OFFSETS == 2
      ? dma_lane_offset<OA>(tid & (LOADERS - 1), m0, M, lda, a_bytes, unused, 1) : a_voff;
  const uint32_t b_voff1 = OB::LANE_OFFSETS == 2
      ? dma_lane_offset<OB>(tid & (LOADERS - 1), n0, N, ldb, b_bytes, unused, 1) : b_voff;
  const uint32_t a_round = (uint32_t)(OA::ROW_STEP * lda * ES);
  const uint32_t b_round = (uint32_t)(OB::ROW_STEP * ldb * ES);
  const uint32_t a_kstep = (uint32_t)(LA == KC ? ES * T::BK : ES * T::BK * lda);
  const uint32_t b_kstep = (uint32_t)(LB == KC ? ES * T::BK : ES * T::BK * ldb);
  const int lwave = wave & 3;

  // Load d of K tile kt is round d of A (d < OA::LOADS) or round
  // d - OA::LOADS of B.  Per K tile, the lane offsets of each operand's two
  // swizzle phases (a K-contiguous tile has one phase, and its chunks at
  // k >= K in the last, partial K tile read as zero through kOutOfRange).
  struct Voffs { uint32_t a[2], b[2]; };
  auto voffs = [&](int kt) {
    const int k0 = kt * T::BK;
    Voffs v{{a_voff, a_voff1}, {b_voff, b_voff1}};
    if (k0 + T::BK > K) {
      if constexpr (LA == KC) v.a[0] = v.a[1] = k0 + a_inner < K ? a_voff : kOutOfRange;
      if constexpr (LB == KC) v.b[0] = v.b[1] = k0 + b_inner < K ? b_voff : kOutOfRange;
    }
    return v;
  };
  auto issue_one = [&](int kt, int d, const Voffs &v) {
    const uint32_t st = lds0 + (uint32_t)((kt & 1) * STAGE);
    if (d < OA::LOADS)
      dma16(rsA, st + (uint32_t)((d * LOADERS + 64 * lwave) * 16), v.a[OA::round_phase(d)],
            (uint32_t)kt * a_kstep + d * a_round);
    else
      dma16(rsB, st + OA::BYTES + (uint32_t)(((d - OA::LOADS) * LOADERS + 64 * lwave) * 16),
            v.b[OB::round_phase(d - OA::LOADS)], (uint32_t)kt * b_kstep + (d - OA::LOADS) * b_round);
  };
  auto issue = [&](int kt) {
    const Voffs v = voffs(kt);
#pragma unroll
    for (int d = 0; d < LOADS_PER_TILE; d++) issue_one(kt, d, v);
  };

  typename L::type acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int r = 0; r < L::R; r++) acc[i][j][r] = 0.f;

  const int KT = (K + T::BK - 1) / T::BK;
  if (KT > 0) {
    if (group == 0) {
      issue(0);
      if (KT > 1) {
        issue(1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS_PER_TILE) : "memory");   // tile 0 landed
      } else {
        wait_dma();
      }
    }
    wg_barrier();                                        // b = 0
    if (group == 1) wg_barrier();                        // b = 1: group 1 idles through M(0) of group 0

    typename InT<IN>::frag fa[KSTEPS][FM], fb[KSTEPS][FN];
    for (int kt = 0; kt < KT; ++kt) {
      // ---- memory phase M(kt)
      // Group 0 also starts the loads of tile kt+1 (their stage was freed at
      // the last barrier; they have until the end of C(kt) to land).  The
      // load issue blocks while the CU's load queue drains, so it is
      // interleaved with the fragment reads, whose issue blocks on a
      // different counter: two loads after each of the first frag reads.
      const char *sA = smem + (kt & 1) * STAGE;
      const char *sB = sA + OA::BYTES;
      // `with_loads` compiles the load issue in; `load` then decides at run time.
      auto m_phase = [&](auto with_loads, bool load) {
        constexpr bool LOAD = decltype(with_loads)::value;
        Voffs v{};
        if constexpr (LOAD) v = voffs(kt + 1);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
          for (int i = 0; i < FM + FN; i++) {
            if constexpr (MF == 32) {
              if (i < FM)
                fa[kk][i] = read_frag_in<OA, IN>(sA, lane, wm * T::TM + 32 * i, kk);
              else
                fb[kk][i - FM] = read_frag_in<OB, IN>(sB, lane, wn * T::TN + 32 * (i - FM), kk);
            } else {
              if (i < FM)
                fa[kk][i] = read_frag16_in<OA, IN>(sA, lane, wm * T::TM + 16 * i, kk);
              else
                fb[kk][i - FM] = read_frag16_in<OB, IN>(sB, lane, wn * T::TN + 16 * (i - FM), kk);
            }
            if constexpr (LOAD) {
              // spread LOADS_PER_TILE loads evenly over the FRAGS fragment reads
              const int q = kk * (FM + FN) + i;
              if (load) {
#pragma unroll
                for (int d = q * LOADS_PER_TILE / FRAGS; d < (q + 1) * LOADS_PER_TILE / FRAGS; d++)
                  issue_one(kt + 1, d, v);
              }
            }
          }
        }
      };
      // Two copies of the phase, with and without the loads: a run-time
      // branch around each load would make the compiler wait for every
      // outstanding fragment read at each branch.
      const bool load_next = group == 0 && kt >= 1 && kt + 1 < KT;
      if (load_next)
        m_phase(std::true_type{}, true);
      else
        m_phase(std::false_type{}, false);
      wait_lds_reads();
      wg_barrier();                                      // end of M(kt)

      // ---- compute phase C(kt)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
          for (int j = 0; j < FN; j++) {
            if constexpr (MF == 32)
              acc[i][j] = mfma_step<IN>(fa[kk][i], fb[kk][j], acc[i][j]);
            else
              acc[i][j] = mfma16_step<IN>(fa[kk][i], fb[kk][j], acc[i][j]);
          }
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) pin_acc(acc[i][j]);
      __builtin_amdgcn_s_setprio(0);
      if (group == 0) {
        wait_dma();                                      // tile kt+1 landed
        wg_barrier();                                    // end of C(kt)
      } else if (kt + 1 < KT) {
        wg_barrier();
      }
    }
  }

  // The LDS is free once every wave is past its last fragment read.
  if (c_vec) {
    __syncthreads();
    if constexpr (LSM_PP_ROW_EPI)
      epilogue_lds_rows<T, OUT, 2 * STAGE, MF>(C, acc, smem, M, N, ldc, m0, n0, wm, wn, wave, lane);
    else
      epilogue_lds<T, OUT, 2 * STAGE, MF>(C, acc, smem, M, N, ldc, m0, n0, wm, wn, wave, lane);
  } else {
    epilogue<T, OUT, MF>(C, acc, M, N, ldc, m0, n0, wm, wn, lane);
  }
}

}  // namespace lsm
