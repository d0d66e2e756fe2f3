// gemm_kernel_skinny.h -- LDS-staged GEMM for latency- and bandwidth-bound
// shapes on gfx950: a deep direct-to-LDS ring and a K split over the waves
// of a workgroup.
//
// Two kinds of shape use it.  With M <= 32 the product does 2*32 flops per B
// element, far below the ~315 flop/byte ridge of MI355X, so the kernel's only
// job is to keep enough bytes of B in flight to run HBM at full rate.  Small
// and mid-size problems (a few hundred workgroups of 64 x 64) are bound by
// the latency of their short K loop rather than by MFMA or HBM throughput.
// Both want many loads in flight per workgroup and little work per wave.
// Each workgroup owns a BM x BN tile of C and walks all of K:
//  * K is cut into stages of BK.  A stage holds A[BM x BK] and B[BK x BN] in
//    their stored contiguity, with the same swizzled layouts, global-side
//    swizzle and buffer range checks as gemm_kernel_dma.h.
//  * NS stages form a ring; the direct-to-LDS loads of stage s + NS - 1 are
//    issued as soon as stage s - 1 has been consumed, so NS - 1 stages are in
//    flight per workgroup.
//  * The four waves split each stage's K range: wave w runs MFMA k-steps
//    w*KSTEPS .. (w+1)*KSTEPS - 1 of the stage (32 x 32 x 16 MFMAs over the
//    whole BM x BN tile) into its own accumulators.  One barrier per stage.
//  * At the end the four partial BM x BN tiles are summed through LDS in a
//    fixed order (wave 0 + 1 + 2 + 3) and stored by the fused, edge-masked
//    epilogue.
// This is the "skinny" variant of the hot path: the same loader, layout,
// transposed reads, MFMA and epilogue, with B streamed exactly once
// ("An educational GEMM ladder for Helios GPUs": asynchronous loads into a
// multi-stage LDS ring, "Level 1" and "Level 2"; the wave-level K split and
// LDS reduction are this kernel's own choice for a tile too small to give
// every wave its own output block).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_kernel_dma.h"

namespace lsm {

template <int BM_, int BN_, int BK_, int NS_, int GROUP_M_ = 8>
struct SkinnyTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_, GROUP_M = GROUP_M_;
  static constexpr int NT = 256, WAVES = 4;
  static constexpr int FM = BM / 32, FN = BN / 32;       // 32 x 32 accumulators per wave
  static_assert(BM % 32 == 0 && BN % 32 == 0, "split-K tile geometry");
};

template <class T, int LA, int LB, int IN, int OUT>
__global__ __launch_bounds__(T::NT, 1) void lds_gemm_skinny_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n,
    uint32_t a_bytes, uint32_t b_bytes) {
  constexpr int ES = InT<IN>::ES;
  constexpr int KSTEPS = T::BK / InT<IN>::KSTEP / T::WAVES;   // MFMA k-steps per wave per stage
  static_assert(KSTEPS >= 1 && KSTEPS * InT<IN>::KSTEP * T::WAVES == T::BK, "stage splits over the waves");
  using OA = OperandTile<T::BM, T::BK, LA, T::NT, ES>;
  using OB = OperandTile<T::BN, T::BK, LB, T::NT, ES>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int LPS = OA::LOADS + OB::LOADS;             // loads per thread per stage
  constexpr int L = T::NS - 1;                           // load lead, in stages
  constexpr int RED = T::WAVES * T::FM * T::FN * 16 * 64 * 4;   // bytes of the partial-sum exchange
  static_assert(RED <= T::NS * STAGE, "the reduction reuses the ring");
  __shared__ __attribute__((aligned(1024))) char smem[T::NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if constexpr (LSM_LDS_POISON) {   // poison build: all of LDS, before any load or write
    lds_poison(smem, T::NS * STAGE, tid, blockDim.x);
    __syncthreads();
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_coords(xcd_logical_id(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, T::GROUP_M, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  const i32x4 rsA = buffer_rsrc(A, a_bytes);
  const i32x4 rsB = buffer_rsrc(B, b_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

  int a_inner, b_inner;
  const uint32_t a_voff = dma_lane_offset<OA>(tid, m0, M, lda, a_bytes, a_inner);
  const uint32_t b_voff = dma_lane_offset<OB>(tid, n0, N, ldb, b_bytes, b_inner);
  const uint32_t a_round = (uint32_t)(OA::ROW_STEP * lda * ES);
  const uint32_t b_round = (uint32_t)(OB::ROW_STEP * ldb * ES);
  const uint32_t a_kstep = (uint32_t)(LA == KC ? ES * T::BK : ES * T::BK * lda);
  const uint32_t b_kstep = (uint32_t)(LB == KC ? ES * T::BK : ES * T::BK * ldb);
  const int KT = (K + T::BK - 1) / T::BK;

  // Loads of stage kt into ring slot `slot`.  Stages past the end of K are
  // loaded with every lane out of range (zeros into a dead slot) so that the
  // number of outstanding loads per stage stays constant.
  auto issue = [&](int kt, int slot) {
    const int k0 = kt * T::BK;
    uint32_t av = a_voff, bv = b_voff;
    uint32_t as = (uint32_t)kt * a_kstep, bs = (uint32_t)kt * b_kstep;
    if (kt >= KT) {
      av = bv = kOutOfRange;
      as = bs = 0;
    } else if (k0 + T::BK > K) {   // last, partial stage: chunks at k >= K read as zero
      if constexpr (LA == KC) av = k0 + a_inner < K ? a_voff : kOutOfRange;
      if constexpr (LB == KC) bv = k0 + b_inner < K ? b_voff : kOutOfRange;
    }
    const uint32_t st = lds0 + (uint32_t)(slot * STAGE);
    dma_tile<OA, T::NT>(rsA, st, wave, av, as, a_round);
    dma_tile<OB, T::NT>(rsB, st + OA::BYTES, wave, bv, bs, b_round);
  };

  v16f32 acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; i++)
#pragma unroll
    for (int j = 0; j < T::FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  if (KT > 0) {
#pragma unroll
    for (int p = 0; p < L; p++) issue(p, p);
    int slot = 0, ld_slot = L;
    for (int kt = 0; kt < KT; ++kt) {
      // Own loads of stage kt have landed once at most the loads of the L-1
      // later stages are outstanding; the barrier then publishes the whole
      // stage and tells every wave that stage kt-1 (slot ld_slot) is free.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((L - 1) * LPS) : "memory");
      __syncthreads();
      issue(kt + L, ld_slot);
      const char *sA = smem + slot * STAGE;
      const char *sB = sA + OA::BYTES;
      typename InT<IN>::frag fa[KSTEPS][T::FM], fb[KSTEPS][T::FN];
#pragma unroll
      for (int s = 0; s < KSTEPS; s++) {
        const int kk = wave * KSTEPS + s;
#pragma unroll
        for (int i = 0; i < T::FM; i++) fa[s][i] = read_frag_in<OA, IN>(sA, lane, 32 * i, kk);
#pragma unroll
        for (int j = 0; j < T::FN; j++) fb[s][j] = read_frag_in<OB, IN>(sB, lane, 32 * j, kk);
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; s++)
#pragma unroll
        for (int i = 0; i < T::FM; i++)
#pragma unroll
          for (int j = 0; j < T::FN; j++) acc[i][j] = mfma_step<IN>(fa[s][i], fb[s][j], acc[i][j]);
      slot = slot + 1 == T::NS ? 0 : slot + 1;
      ld_slot = ld_slot + 1 == T::NS ? 0 : ld_slot + 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS
  }

  // Sum the four waves' partial tiles through LDS, in wave order.
  __syncthreads();                                       // every wave is done with the ring
  if constexpr (LSM_LDS_POISON) {   // poison build: the reduction region, before its writes
    lds_poison(smem, RED, tid, T::NT);
    __syncthreads();
  }
  // Slot of accumulator register r of block (i, j) of wave w, lane l.
  auto red_at = [&](int w, int i, int j, int r) { return (((w * T::FM + i) * T::FN + j) * 16 + r) * 64 + lane; };
  float *red = (float *)smem;
#pragma unroll
  for (int i = 0; i < T::FM; i++)
#pragma unroll
    for (int j = 0; j < T::FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) red[red_at(wave, i, j, r)] = acc[i][j][r];
  __syncthreads();
  // Wave w finalises accumulator registers r = 4w .. 4w+3 of every 32 x 32
  // block: rows 8w + 4*(l >> 5) + 0..3 (32 x 32 MFMA accumulator layout).
#pragma unroll
  for (int i = 0; i < T::FM; i++) {
    const int row0 = m0 + 32 * i + 8 * wave + 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < T::FN; j++) {
      const int col = n0 + 32 * j + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r = 4 * wave + q;
        float v = red[red_at(0, i, j, r)];
#pragma unroll
        for (int w = 1; w < T::WAVES; w++) v += red[red_at(w, i, j, r)];
        const int row = row0 + q;
        if (row < M && col < N) store_out<OUT>(C, (int64_t)row * ldc + col, v);
      }
    }
  }
}

}  // namespace lsm
