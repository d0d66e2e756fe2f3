// gemm_kernel_skinny.h -- LDS-staged GEMM for small M (M <= 32) on gfx950:
// bandwidth-bound, B streamed from HBM once through a deep LDS ring.
//
// With M <= 32 the product does 2*32 flops per B element, far below the
// ~315 flop/byte ridge of MI355X, so the kernel's only job is to keep enough
// bytes of B in flight to run HBM at full rate.  Each workgroup owns a
// 32 x BN column slab of C and walks all of K:
//  * K is cut into stages of BK = 128.  A stage holds A[32 x 128] and
//    B[128 x BN] in their stored contiguity, with the same swizzled layouts,
//    global-side swizzle and buffer range checks as gemm_kernel_dma.h.
//  * NS stages form a ring; the direct-to-LDS loads of stage s + NS - 1 are
//    issued as soon as stage s - 1 has been consumed, so NS - 1 stages
//    (NS - 1 times 24 KiB for BN = 64) are in flight per workgroup.
//  * The four waves split each stage's K range: wave w runs the two MFMA
//    k-steps 2w, 2w + 1 (32 x 32 x 16 MFMAs, BN / 32 of them per k-step) into
//    its own accumulators.  One barrier per stage.
//  * At the end the four partial 32 x BN tiles are summed through LDS in a
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

template <int BN_, int NS_>
struct SkinnyTile {
  static constexpr int BM = 32, BN = BN_, BK = 128, NS = NS_;
  static constexpr int NT = 256, WAVES = 4;
  static constexpr int FN = BN / 32;                     // 32 x 32 accumulators per wave
  static constexpr int KSTEPS = BK / 16 / WAVES;         // MFMA k-steps per wave per stage
  static_assert(BN % 32 == 0 && KSTEPS >= 1, "skinny tile geometry");
};

template <class T, int LA, int LB, int IN, int OUT>
__global__ __launch_bounds__(T::NT, 1) void lds_gemm_skinny_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, void *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, uint32_t a_bytes,
    uint32_t b_bytes) {
  using OA = OperandTile<T::BM, T::BK, LA, T::NT>;
  using OB = OperandTile<T::BN, T::BK, LB, T::NT>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int LPS = OA::LOADS + OB::LOADS;             // loads per thread per stage
  constexpr int L = T::NS - 1;                           // load lead, in stages
  constexpr int RED = T::WAVES * T::FN * 16 * 64 * 4;    // bytes of the partial-sum exchange
  static_assert(RED <= T::NS * STAGE, "the reduction reuses the ring");
  __shared__ __attribute__((aligned(1024))) char smem[T::NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * T::BN;

  const i32x4 rsA = buffer_rsrc(A, a_bytes);
  const i32x4 rsB = buffer_rsrc(B, b_bytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

  int a_inner, b_inner;
  const uint32_t a_voff = dma_lane_offset<OA>(tid, 0, M, lda, a_bytes, a_inner);
  const uint32_t b_voff = dma_lane_offset<OB>(tid, n0, N, ldb, b_bytes, b_inner);
  const uint32_t a_round = (uint32_t)(OA::ROW_STEP * lda * 2);
  const uint32_t b_round = (uint32_t)(OB::ROW_STEP * ldb * 2);
  const uint32_t a_kstep = (uint32_t)(LA == KC ? 2 * T::BK : 2 * T::BK * lda);
  const uint32_t b_kstep = (uint32_t)(LB == KC ? 2 * T::BK : 2 * T::BK * ldb);
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

  v16f32 acc[T::FN];
#pragma unroll
  for (int j = 0; j < T::FN; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[j][r] = 0.f;

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
      v8i16 fa[T::KSTEPS], fb[T::KSTEPS][T::FN];
#pragma unroll
      for (int s = 0; s < T::KSTEPS; s++) {
        const int kk = wave * T::KSTEPS + s;
        fa[s] = read_frag<OA>(sA, lane, 0, kk);
#pragma unroll
        for (int j = 0; j < T::FN; j++) fb[s][j] = read_frag<OB>(sB, lane, 32 * j, kk);
      }
#pragma unroll
      for (int s = 0; s < T::KSTEPS; s++)
#pragma unroll
        for (int j = 0; j < T::FN; j++) acc[j] = mfma_32x32x16<IN>(fa[s], fb[s][j], acc[j]);
      slot = slot + 1 == T::NS ? 0 : slot + 1;
      ld_slot = ld_slot + 1 == T::NS ? 0 : ld_slot + 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may still target LDS
  }

  // Sum the four waves' partial tiles through LDS, in wave order.
  __syncthreads();                                       // every wave is done with the ring
  float *red = (float *)smem;
#pragma unroll
  for (int j = 0; j < T::FN; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) red[((wave * T::FN + j) * 16 + r) * 64 + lane] = acc[j][r];
  __syncthreads();
  // Wave w finalises accumulator registers r = 4w .. 4w+3 of every 32 x 32
  // block: rows 8w + 4*(l >> 5) + 0..3 (32 x 32 MFMA accumulator layout).
  const int row0 = 8 * wave + 4 * (lane >> 5);
#pragma unroll
  for (int j = 0; j < T::FN; j++) {
    const int col = n0 + 32 * j + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 4 * wave + i;
      float v = red[((0 * T::FN + j) * 16 + r) * 64 + lane];
#pragma unroll
      for (int w = 1; w < T::WAVES; w++) v += red[((w * T::FN + j) * 16 + r) * 64 + lane];
      const int row = row0 + i;
      if (row < M && col < N) store_out<OUT>(C, (int64_t)row * ldc + col, v);
    }
  }
}

}  // namespace lsm
