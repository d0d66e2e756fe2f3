// gemm_kernel_pingpong.h -- LDS-staged GEMM with direct-to-LDS loads and a
// two-group ping-pong schedule, for gfx950.
//
// Eight waves, two per SIMD, in two groups of four (waves 0-3 and 4-7; wave
// w runs on SIMD w mod 4).  Each wave owns a 128 x 64 block of the 256 x 256
// workgroup tile.  The groups alternate between two kinds of phase,
// separated by workgroup barriers:
//   memory phase  M(t): read every MFMA fragment of K tile t from LDS into
//                       registers, and issue this group's direct-to-LDS
//                       loads of a later tile (below);
//   compute phase C(t): the MFMAs of tile t, from registers only.
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
// pass 2*KT + 1 barriers.  Tile t is read between barriers 2t and 2t+2.
//
// Who loads what.  A tile of either operand is 32 KiB: 8 rounds of 16-byte
// loads by the 256 lanes of one group.
//  * split loads (A K-contiguous, the library's NN and NT): group 0 loads A
//    of tile t+1 in M(t), group 1 loads B of tile t+2 in its M(t).  A takes
//    two LDS stages (tile t in stage t & 1), B three (stage t mod 3): 160 KiB.
//    A of tile t+1 goes into the stage of tile t-1, whose last reads ended at
//    barrier 2t; group 0 waits for it (vmcnt(0)) before barrier 2t+2, the
//    end of C(t).  B of tile t+2 goes into the stage of tile t-1 as well and
//    is issued after barrier 2t+1; group 1 waits for it at the end of its
//    next memory phase, before barrier 2t+4, when tile t+2 is first read.
//    So each group issues half of the 64 KiB of loads per tile, in its own
//    memory phase, and the B loads have three phases to land.
//  * one loader (A MN-contiguous, TN and TT, where splitting measured
//    slower; and the A/B builds that change the fragment reads): group 0
//    loads all of tile t+1 in M(t), into two stages of 64 KiB; it waits for
//    them before barrier 2t+2.  The loads have two phases to land, and
//    group 0's memory phase carries all of them.
// Tiles 0 and 1 come with the prologue (split: each group its operand).
// Every wave waits for its own LDS reads before the barrier that ends its
// memory phase, and a tile is complete at the barrier before its first read.
// A wave's vmcnt covers only its own quarter of its group's loads, so even
// the loading group reads a tile only after a barrier that follows all four
// waits: group 0's wait stays at the end of C(t), before barrier 2t+2.
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

// The library splits the loads between the groups when A is K-contiguous;
// LSM_PP_SPLIT_LOADS = 0, an A/B build only, keeps one loader group for every
// layout.
#ifndef LSM_PP_SPLIT_LOADS
#define LSM_PP_SPLIT_LOADS 1
#endif

// LSM_PP_TIMELINE = 1 (measurement builds only, A/B builds timeline and
// timeline1): each wave adds up the shader-clock cycles (s_memtime) of its
// phases and writes 8 counts to the buffer that lsm_pp_timeline_set
// installs: memory-phase work, wait at the barrier after it, MFMA issue, wait
// for its own loads, wait at the barrier after the MFMAs (each summed over
// the K loop), then prologue, K loop and epilogue.  Nothing is written while
// no buffer is installed.  The library is built with 0.
#ifndef LSM_PP_TIMELINE
#define LSM_PP_TIMELINE 0
#endif
#if LSM_PP_TIMELINE
__device__ unsigned long long *pp_timeline_buf;
#define PP_CLOCK() __builtin_amdgcn_s_memtime()
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
#if LSM_PP_TIMELINE
  const unsigned long long t_start = PP_CLOCK();
  unsigned long long t_first = 0, ph[5] = {0, 0, 0, 0, 0};
#endif
  using L = AccLayout<MF>;
  constexpr int LOADERS = T::NT / 2;                     // lanes of the group loading an operand
  constexpr int ES = InT<IN>::ES;
  // MFMA k-steps per K tile (a 16 x 16 MFMA is twice as deep as a 32 x 32 one)
  constexpr int KSTEPS = T::BK / (MF == 32 ? InT<IN>::KSTEP : 2 * InT<IN>::KSTEP);
  constexpr int FM = T::TM / MF, FN = T::TN / MF;        // MFMA blocks per wave
  // With 16 x 16 MFMAs an MN-contiguous tile takes the layout of those
  // fragments' transposed reads, with two lane offsets per loader.
  using OA = OperandTile<T::BM, T::BK, LA, LOADERS, ES, MF == 16>;
  using OB = OperandTile<T::BN, T::BK, LB, LOADERS, ES, MF == 16>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int LOADS_PER_TILE = OA::LOADS + OB::LOADS;  // per wave of a lone loader group
  constexpr int FRAGS = KSTEPS * (FM + FN);               // fragment reads per memory phase
  // Load schedule (see the head of this file): one loader group, or the
  // loads split between the groups -- compiled per group, or in one memory
  // phase whose operand each wave selects (B K-contiguous: the per-group
  // form needs more than 256 VGPRs there).  The A/B builds that change the
  // fragment reads (32 x 32 MFMAs, no swizzle, scalar 16-bit reads) keep one
  // loader group: with them both split forms need more.
  enum { ONE_LOADER, SPLIT_SELECT, SPLIT_PER_GROUP };
  constexpr bool SPLIT_FITS = MF == 16 && LSM_LDS_SWIZZLE && LSM_TR_READ;
  constexpr int SCHED = !LSM_PP_SPLIT_LOADS || LA != KC || !SPLIT_FITS ? ONE_LOADER
                        : LB == MNC                                    ? SPLIT_PER_GROUP
                                                                       : SPLIT_SELECT;
  constexpr bool SPLIT = SCHED != ONE_LOADER;
  // A stages, then B stages (two each, or three of B when the loads are split)
  constexpr int A_STAGE = SPLIT ? OA::BYTES : STAGE;
  constexpr int B_BASE = SPLIT ? 2 * OA::BYTES : OA::BYTES;
  constexpr int B_STAGE = SPLIT ? OB::BYTES : STAGE;
  constexpr int LDS_BYTES = SPLIT ? 2 * OA::BYTES + 3 * OB::BYTES : 2 * STAGE;
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if constexpr (LSM_LDS_POISON) {   // poison build: all of LDS, before any load or write
    lds_poison(smem, LDS_BYTES, tid, blockDim.x);
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

  // Loader geometry.  Each loading wave covers its operand's tile in
  // LOADERS-thread rounds; lane offsets from the wave's index in its group.
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

  // LDS offsets of tile kt's A and B stages
  auto a_stage = [&](int kt) { return (uint32_t)((kt & 1) * A_STAGE); };
  auto b_stage = [&](int kt) { return (uint32_t)(B_BASE + (SPLIT ? kt % 3 : kt & 1) * B_STAGE); };
  // An operand's lane offsets for K tile kt, one per swizzle phase (a
  // K-contiguous tile has one phase, and its chunks at k >= K in the last,
  // partial K tile read as zero through kOutOfRange).
  struct Pair { uint32_t v[2]; };
  auto tail = [&](int kt, uint32_t voff, int inner, Pair p) {
    const int k0 = kt * T::BK;
    if (k0 + T::BK > K) p.v[0] = p.v[1] = k0 + inner < K ? voff : kOutOfRange;
    return p;
  };
  auto voffs_a = [&](int kt) {
    Pair p{{a_voff, a_voff1}};
    if constexpr (LA == KC) p = tail(kt, a_voff, a_inner, p);
    return p;
  };
  auto voffs_b = [&](int kt) {
    Pair p{{b_voff, b_voff1}};
    if constexpr (LB == KC) p = tail(kt, b_voff, b_inner, p);
    return p;
  };
  // load round d of A (B) of K tile kt
  auto issue_a = [&](int kt, int d, const Pair &p) {
    dma16(rsA, lds0 + a_stage(kt) + (uint32_t)((d * LOADERS + 64 * lwave) * 16), p.v[OA::round_phase(d)],
          (uint32_t)kt * a_kstep + d * a_round);
  };
  auto issue_b = [&](int kt, int d, const Pair &p) {
    dma16(rsB, lds0 + b_stage(kt) + (uint32_t)((d * LOADERS + 64 * lwave) * 16), p.v[OB::round_phase(d)],
          (uint32_t)kt * b_kstep + d * b_round);
  };
  // One loader group: load d of tile kt is round d of A (d < OA::LOADS) or
  // round d - OA::LOADS of B.
  auto issue_one = [&](int kt, int d, const Pair &pa, const Pair &pb) {
    if (d < OA::LOADS)
      issue_a(kt, d, pa);
    else
      issue_b(kt, d - OA::LOADS, pb);
  };

  // Split loads, selecting form: the wave-uniform choice of operand.
  static_assert(!SPLIT || OA::LOADS == OB::LOADS, "equal load rounds per operand");
  static_assert(SCHED != SPLIT_SELECT || OA::LANE_OFFSETS == 1 || OB::LANE_OFFSETS == 1 ||
                (OA::ROW_STEP == OB::ROW_STEP && OA::PHASE_ROWS == OB::PHASE_ROWS),
                "one round-to-lane-offset map serves both operands");
  using OP = std::conditional_t<OB::LANE_OFFSETS == 2, OB, OA>;   // its round phases
  const bool loads_b = SPLIT && group == 1;
  const i32x4 o_rs = loads_b ? rsB : rsA;
  const uint32_t o_voff0 = loads_b ? b_voff : a_voff, o_voff1 = loads_b ? b_voff1 : a_voff1;
  const int o_inner = loads_b ? b_inner : a_inner;
  const bool o_kc = loads_b ? LB == KC : LA == KC;
  const uint32_t o_kstep = loads_b ? b_kstep : a_kstep, o_round = loads_b ? b_round : a_round;
  auto voffs_own = [&](int kt) {
    const Pair p{{o_voff0, o_voff1}};
    return o_kc ? tail(kt, o_voff0, o_inner, p) : p;
  };
  auto issue_own = [&](int kt, int d, const Pair &p) {
    const uint32_t st = loads_b ? b_stage(kt) : a_stage(kt);
    dma16(o_rs, lds0 + st + (uint32_t)((d * LOADERS + 64 * lwave) * 16), p.v[OP::round_phase(d)],
          (uint32_t)kt * o_kstep + d * o_round);
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
    if constexpr (SPLIT) {
      // group 0 loads A of tiles 0 and 1, group 1 B of tiles 0 and 1
#pragma unroll
      for (int t = 0; t < 2; t++) {
        if (t < KT) {
          const Pair p = voffs_own(t);
#pragma unroll
          for (int d = 0; d < OA::LOADS; d++) issue_own(t, d, p);
        }
      }
      if (KT > 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OA::LOADS) : "memory");       // tile 0's part landed
      else
        wait_dma();
    } else if (group == 0) {
#pragma unroll
      for (int t = 0; t < 2; t++) {
        if (t < KT) {
          const Pair pa = voffs_a(t), pb = voffs_b(t);
#pragma unroll
          for (int d = 0; d < LOADS_PER_TILE; d++) issue_one(t, d, pa, pb);
        }
      }
      if (KT > 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS_PER_TILE) : "memory");   // tile 0 landed
      else
        wait_dma();
    }
    wg_barrier();                                        // b = 0
    if (group == 1) wg_barrier();                        // b = 1: group 1 idles through M(0) of group 0

    typename InT<IN>::frag fa[KSTEPS][FM], fb[KSTEPS][FN];
    for (int kt = 0; kt < KT; ++kt) {
#if LSM_PP_TIMELINE
      const unsigned long long ta = PP_CLOCK();
      if (kt == 0) t_first = ta;
#endif
      // ---- memory phase M(kt)
      // The loads of this phase (none, or those the schedule gives the wave's
      // group) go into stages freed at the last barrier.  The load issue
      // blocks while the CU's load queue drains, so it is interleaved with
      // the fragment reads, whose issue blocks on a different counter.
      const char *sA = smem + a_stage(kt);
      const char *sB = smem + b_stage(kt);
      // LOAD compiles the load issue in: 0 none, 1 both operands of tile
      // kt+1 (one loader group), 2 the wave's own operand (A of tile kt+1 or
      // B of tile kt+2), 3 A of tile kt+1, 4 B of tile kt+2.
      auto m_phase = [&](auto load_kind) {
        constexpr int LOAD = decltype(load_kind)::value;
        constexpr int NL = LOAD == 1 ? LOADS_PER_TILE : OA::LOADS;
        const int lt = kt + (LOAD == 4 || (LOAD == 2 && loads_b) ? 2 : 1);   // the tile loaded
        Pair pa{}, pb{};
        if constexpr (LOAD == 1 || LOAD == 3) pa = voffs_a(lt);
        if constexpr (LOAD == 1 || LOAD == 4) pb = voffs_b(lt);
        if constexpr (LOAD == 2) pa = voffs_own(lt);
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
            // spread the NL loads evenly over the FRAGS fragment reads
            const int q = kk * (FM + FN) + i;
#pragma unroll
            for (int d = q * NL / FRAGS; LOAD != 0 && d < (q + 1) * NL / FRAGS; d++) {
              if constexpr (LOAD == 1) issue_one(lt, d, pa, pb);
              if constexpr (LOAD == 2) issue_own(lt, d, pa);
              if constexpr (LOAD == 3) issue_a(lt, d, pa);
              if constexpr (LOAD == 4) issue_b(lt, d, pb);
            }
          }
        }
      };
      using None = std::integral_constant<int, 0>;
      // Separate copies of the phase with and without loads: a run-time
      // branch around each load would make the compiler wait for every
      // outstanding fragment read at each branch.
      if constexpr (SCHED == ONE_LOADER) {
        if (group == 0 && kt >= 1 && kt + 1 < KT)
          m_phase(std::integral_constant<int, 1>{});
        else
          m_phase(None{});
      } else {
        // group 0 loads A of tile kt+1 from kt = 1 on (tile 1 came with the
        // prologue), group 1 B of tile kt+2
        const bool load = loads_b ? kt + 2 < KT : kt >= 1 && kt + 1 < KT;
        if constexpr (SCHED == SPLIT_PER_GROUP) {
          if (load && !loads_b)
            m_phase(std::integral_constant<int, 3>{});
          else if (load)
            m_phase(std::integral_constant<int, 4>{});
          else
            m_phase(None{});
        } else {
          if (load)
            m_phase(std::integral_constant<int, 2>{});
          else
            m_phase(None{});
        }
        // group 1 waits here for its loads of the previous memory phase (B
        // of tile kt+1), which every wave reads after the next barrier
        if (loads_b) {
          if (load)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OB::LOADS) : "memory");
          else
            wait_dma();
        }
      }
      wait_lds_reads();
#if LSM_PP_TIMELINE
      const unsigned long long tb = PP_CLOCK();
#endif
      wg_barrier();                                      // end of M(kt)
#if LSM_PP_TIMELINE
      const unsigned long long tc = PP_CLOCK();
#endif

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
#if LSM_PP_TIMELINE
      const unsigned long long td = PP_CLOCK();
      unsigned long long te = td;
#endif
      if (group == 0) {
        wait_dma();                                      // tile kt+1 landed
#if LSM_PP_TIMELINE
        te = PP_CLOCK();
#endif
        wg_barrier();                                    // end of C(kt)
      } else if (kt + 1 < KT) {
        wg_barrier();
      }
#if LSM_PP_TIMELINE
      const unsigned long long tf = PP_CLOCK();
      ph[0] += tb - ta, ph[1] += tc - tb, ph[2] += td - tc, ph[3] += te - td, ph[4] += tf - te;
#endif
    }
  }
#if LSM_PP_TIMELINE
  const unsigned long long t_loop = PP_CLOCK();
#endif

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
#if LSM_PP_TIMELINE
  const unsigned long long t_end = PP_CLOCK();
  if (pp_timeline_buf != nullptr && lane == 0) {
    unsigned long long *o = pp_timeline_buf + ((size_t)blockIdx.x * 8 + wave) * 8;
    for (int i = 0; i < 5; i++) o[i] = ph[i];
    o[5] = t_first - t_start, o[6] = t_loop - t_first, o[7] = t_end - t_loop;
  }
#endif
}

}  // namespace lsm
