// gemm_common.h -- pieces shared by the GEMM kernels: vector types, tile
// geometry, the MFMA micro-kernel, LDS fragment reads and the epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_layout.h"

// LSM_TR_READ = 0 builds the kernels with the MN-contiguous operand read by
// eight 16-bit LDS loads per fragment instead of two ds_read_b64_tr_b16; it
// exists only for the A/B build that measures what the transposed read buys.
// The library is built with the default, 1.
#ifndef LSM_TR_READ
#define LSM_TR_READ 1
#endif

// LSM_LDS_POISON = 1 builds the kernels so that they fill their LDS with NaN
// bits (all-ones bytes: NaN as bf16, fp16 and E4M3) before its first use, and
// fill the epilogue's staging region and the split-K reduction region the
// same way before those are written.  A read of a slot that no load or write
// has filled then turns the products it reaches into NaN, which a bit-exact
// comparison on integer inputs reports ("Lds Optimization", "LDS Instruction
// Model" and "Verification Checklist": every read must follow the write it
// needs).  It exists only for the A/B build that checks this; the library is
// built with 0.
#ifndef LSM_LDS_POISON
#define LSM_LDS_POISON 0
#endif

namespace lsm {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef _Float16 v8f16 __attribute__((ext_vector_type(8)));
typedef float v16f32 __attribute__((ext_vector_type(16)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
typedef __attribute__((address_space(3))) void lds_void;

enum { KC = 0, MNC = 1 };                       // operand contiguity, values of enum gemm_layout
enum { IN_BF16 = 0, IN_F16 = 1, IN_E4M3 = 2 };
enum { OUT_F32 = 0, OUT_BF16 = 1, OUT_F16 = 2 };

// Input element types: bytes per element, k per 32 x 32 MFMA and the per-lane
// operand fragment.  16-bit inputs use v_mfma_f32_32x32x16_{bf16,f16} or
// v_mfma_f32_16x16x32_{bf16,f16} (8 elements, 16 bytes per lane; k = KSTEP or
// 2*KSTEP); OCP fp8 E4M3 inputs use v_mfma_scale_f32_32x32x64_f8f6f4 or
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (32 elements, 32 bytes).
template <int IN>
struct InT {
  static constexpr int ES = 2, KSTEP = 16;
  typedef v8i16 frag;
};
template <>
struct InT<IN_E4M3> {
  static constexpr int ES = 1, KSTEP = 64;
  typedef v8i32 frag;
};

template <int BM_, int BN_, int BK_, int WM_, int WN_, int GROUP_M_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WM = WM_, WN = WN_;                // wave grid inside the workgroup
  static constexpr int GROUP_M = GROUP_M_;                // tile rows per L2 group
  static constexpr int NT = WM * WN * 64;                  // threads per workgroup
  static constexpr int TM = BM / WM, TN = BN / WN;         // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;         // 32x32 fragments per wave
  static constexpr int KSTEPS = BK / 16;                   // MFMA k steps per K tile, 16-bit inputs
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
};

// Geometry of one operand's LDS tile.  MN is the tile's M (for A) or N (for
// B) extent.  K-contiguous: MN rows of BK elements.  MN-contiguous: BK rows of
// MN elements.  "outer" is the strided dimension of the operand in memory,
// "inner" its unit-stride dimension; ES is the element size in bytes.  The
// tile is filled in rounds of NT 16-byte chunks: chunk id = thread + round *
// NT, numbered row-major.  MF16 = 1 lays an MN-contiguous tile out for the
// transposed fragments of the 16 x 16 MFMAs (mn16_chunk_offset: 16 x 16 x 32
// for 16-bit, 16 x 16 x 128 for 8-bit elements); otherwise, and for
// K-contiguous tiles, the layout is the one the 32 x 32 fragments read
// (kc_chunk_offset, mn_chunk_offset).
template <int MN, int BK, int LAYOUT, int NT, int ES_ = 2, int MF16_ = 0>
struct OperandTile {
  static constexpr bool kcontig = LAYOUT == KC;
  static constexpr int ES = ES_;
  static constexpr bool mf16 = MF16_ != 0 && !kcontig;          // 16 x 16 MN layout
  static constexpr int ROWS = kcontig ? MN : BK;                 // outer extent
  static constexpr int INNER = kcontig ? BK : MN;                // inner extent (elements)
  static constexpr int ROW_BYTES = ES * INNER;
  static constexpr int EPC = 16 / ES;                            // elements per 16-byte chunk
  static constexpr int CPR = ROW_BYTES / 16;                     // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROW_BYTES;
  static constexpr int CHUNKS = BYTES / 16;
  static constexpr int LOADS = CHUNKS / NT;                      // 16-byte loads per thread
  static constexpr int ROW_STEP = NT / CPR;                      // rows between a thread's loads
  // rows per swizzle period
  static constexpr int SWZ_PERIOD = kcontig ? 16 : mf16 ? (ES == 2 ? 16 : 32) : (ES == 2 ? 4 : 8);
  // A thread's chunks of every load round share one swizzle phase when the
  // round step is a multiple of the period (one lane offset for all rounds).
  // The 16 x 16 MN layouts depend on the row only through the row inside a
  // round and one more bit, that of PHASE_ROWS (8 for 16-bit elements, rounds
  // of 8 rows; 16 for 8-bit elements, rounds of 16 rows): one lane offset for
  // the rounds with that bit clear and one for those with it set.
  static constexpr int PHASE_ROWS = SWZ_PERIOD / 2;
  static constexpr int LANE_OFFSETS = ROW_STEP % SWZ_PERIOD == 0 ? 1 : 2;
  static_assert(CHUNKS % NT == 0, "tile must split evenly into 16-byte loads");
  static_assert(NT % CPR == 0 && (ROW_STEP % SWZ_PERIOD == 0 ||
                                  (mf16 && ROW_STEP >= (ES == 2 ? 8 : 16) && PHASE_ROWS % ROW_STEP == 0)),
                "a thread's chunks must take one or two swizzle phases");
  // Which of the lane offsets load round d uses.
  __host__ __device__ static constexpr int round_phase(int d) {
    return LANE_OFFSETS == 1 ? 0 : ((d * ROW_STEP) / PHASE_ROWS) & 1;
  }
  // XOR applied to the chunk index of row `row` of this tile.
  __host__ __device__ static constexpr int swizzle(int row) {
    return kcontig ? kc_swizzle(row, ROW_BYTES)
                   : mf16 ? (ES == 2 ? mn16_swizzle(row, ROW_BYTES) : mn16_swizzle8(row, ROW_BYTES))
                          : mn_swizzle(row, ROW_BYTES, ES);
  }
};

// Poison build: `n` threads (thread index `t`) fill `bytes` bytes of LDS at
// `lds` (16-byte aligned, a multiple of 16) with all-ones bytes.  No-op in the
// library.  The caller orders it before the region's first use.
__device__ __forceinline__ void lds_poison(char *lds, int bytes, int t, int n) {
  if constexpr (LSM_LDS_POISON) {
    for (int i = t; i < bytes / 16; i += n) ((u32x4 *)lds)[i] = u32x4{~0u, ~0u, ~0u, ~0u};
  }
}

template <int IN>
__device__ __forceinline__ v16f32 mfma_32x32x16(v8i16 a, v8i16 b, v16f32 c) {
  if constexpr (IN == IN_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf16, a),
                                                   __builtin_bit_cast(v8bf16, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8f16, a),
                                                  __builtin_bit_cast(v8f16, b), c, 0, 0, 0);
}

// One 32 x 32 MFMA step of the input type: k = 16 (bf16/fp16) or k = 64
// (E4M3: format code 0 for both operands, E8M0 scales 127 = 2^0).
template <int IN>
__device__ __forceinline__ v16f32 mfma_step(typename InT<IN>::frag a, typename InT<IN>::frag b,
                                            v16f32 c) {
  if constexpr (IN == IN_E4M3)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  else
    return mfma_32x32x16<IN>(a, b, c);
}

// One 16 x 16 MFMA step (k = 32) on 16-bit inputs ("Lds Optimization",
// "Optimization Method 3: Increase Write-Read Distance", names
// v_mfma_f32_16x16x32 as the MFMA it overlaps).
template <int IN>
__device__ __forceinline__ v4f32 mfma_16x16x32(v8i16 a, v8i16 b, v4f32 c) {
  static_assert(IN != IN_E4M3, "16-bit inputs only");
  if constexpr (IN == IN_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf16, a),
                                                   __builtin_bit_cast(v8bf16, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8f16, a),
                                                  __builtin_bit_cast(v8f16, b), c, 0, 0, 0);
}

// One 16 x 16 MFMA step on E4M3 inputs (k = 128; format code 0 for both
// operands, E8M0 scales 127 = 2^0, as for the 32 x 32 x 64 form).
__device__ __forceinline__ v4f32 mfma_16x16x128_e4m3(v8i32 a, v8i32 b, v4f32 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// One 16 x 16 MFMA step of the input type.
template <int IN>
__device__ __forceinline__ v4f32 mfma16_step(typename InT<IN>::frag a, typename InT<IN>::frag b,
                                             v4f32 c) {
  if constexpr (IN == IN_E4M3)
    return mfma_16x16x128_e4m3(a, b, c);
  else
    return mfma_16x16x32<IN>(a, b, c);
}

// Accumulator layouts of the two MFMA shapes.  Register r of lane l holds
//   32 x 32 block (16 registers): row 8*(r >> 2) + 4*(l >> 5) + (r & 3), column l & 31;
//   16 x 16 block (4 registers):  row 4*(l >> 4) + r, column l & 15.
// Both are checked on the GPU, one MFMA at a time on random and one-hot
// integers, by the probe kernels of hw_probe.hip (tests/test_gpu_hw_maps.py).
// row() is the whole row; lane_row() + reg_row() splits it into its lane and register parts.
template <int MF>
struct AccLayout;
template <>
struct AccLayout<32> {
  static constexpr int F = 32, R = 16;
  typedef v16f32 type;
  __device__ static constexpr int lane_row(int lane) { return 4 * (lane >> 5); }
  __device__ static constexpr int reg_row(int r) { return 8 * (r >> 2) + (r & 3); }
  __device__ static constexpr int row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
  __device__ static constexpr int col(int lane) { return lane & 31; }
};
template <>
struct AccLayout<16> {
  static constexpr int F = 16, R = 4;
  typedef v4f32 type;
  __device__ static constexpr int lane_row(int lane) { return 4 * (lane >> 4); }
  __device__ static constexpr int reg_row(int r) { return r; }
  __device__ static constexpr int row(int r, int lane) { return 4 * (lane >> 4) + r; }
  __device__ static constexpr int col(int lane) { return lane & 15; }
};

// Keeps an accumulator's MFMAs ahead of this point: the compiler may otherwise
// sink register-only MFMAs past a following barrier into the next phase.
__device__ __forceinline__ void pin_acc(v16f32 &c) { asm volatile("" : "+v"(c)); }
__device__ __forceinline__ void pin_acc(v4f32 &c) { asm volatile("" : "+v"(c)); }

// One 32x32x16 operand fragment: lane l gets row/column (l & 31) of the
// fragment starting at `base`, k = 16*kk + 8*(l >> 5) + 0..7.
// One 32 x 64 operand fragment of 8-bit elements (k-step kk of the tile).
template <class OT>
__device__ __forceinline__ v8i32 read_frag8(const char *lds, int lane, int base, int kk) {
  if constexpr (OT::kcontig) {
    const u32x4 lo = *(const u32x4 *)(lds + frag_kc8_offset(lane, base, kk, 0, OT::ROW_BYTES));
    const u32x4 hi = *(const u32x4 *)(lds + frag_kc8_offset(lane, base, kk, 1, OT::ROW_BYTES));
    return __builtin_bit_cast(v8i32, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    v2i32 p[4];
#pragma unroll
    for (int q = 0; q < 4; q++)
      p[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i32 *)(lds + frag_tr8_offset(lane, base, kk, q, OT::ROW_BYTES)));
    const auto lo = __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3);
    const auto hi = __builtin_shufflevector(p[2], p[3], 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <class OT>
__device__ __forceinline__ v8i16 read_frag(const char *lds, int lane, int base, int kk) {
  if constexpr (OT::kcontig) {
    return *(const v8i16 *)(lds + frag_kc_offset(lane, base, kk, OT::ROW_BYTES));
  } else if constexpr (!LSM_TR_READ) {
    // element i of lane l: column base + (l & 31), k-row 16*kk + 8*(l >> 5) + i
    const int col = base + (lane & 31);
    v8i16 f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      f[i] = *(const short *)(lds + mn_chunk_offset(16 * kk + 8 * (lane >> 5) + i, col / 8,
                                                    OT::ROW_BYTES) + 2 * (col & 7));
    return f;
  } else {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(lds + frag_tr_offset(lane, base, kk, 0, OT::ROW_BYTES)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(lds + frag_tr_offset(lane, base, kk, 1, OT::ROW_BYTES)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// One 16 x 32 operand fragment of v_mfma_f32_16x16x32 (k-step kk of 32):
// lane l gets row/column (l & 15) of the fragment starting at `base`,
// k = 32*kk + 8*(l >> 4) + 0..7.
template <class OT>
__device__ __forceinline__ v8i16 read_frag16(const char *lds, int lane, int base, int kk) {
  if constexpr (OT::kcontig) {
    return *(const v8i16 *)(lds + frag16_kc_offset(lane, base, kk, OT::ROW_BYTES));
  } else if constexpr (!LSM_TR_READ) {
    static_assert(OT::mf16, "16 x 16 x 32 MN layout");
    const int col = base + (lane & 15);
    v8i16 f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      f[i] = *(const short *)(lds + mn16_chunk_offset(32 * kk + 8 * (lane >> 4) + i, col / 8,
                                                      OT::ROW_BYTES) + 2 * (col & 7));
    return f;
  } else {
    // lds + frag16_tr_offset(lane, base, kk, h, ROW_BYTES), computed as
    // ((tile + 256*(base >> 7) + lane part) XOR 32*((base >> 4) & 7)) + the
    // k-step and half, which equals it because the tile base (a multiple of
    // 1 KiB: every stage and operand tile is) has bits 5-7 clear.  The tile
    // base changes with the LDS stage, so the XOR is evaluated per read
    // instead of one loop-invariant address register per fragment.
    static_assert(OT::mf16 && OT::ROW_BYTES >= 256 && OT::BYTES % 1024 == 0,
                  "16 x 16 x 32 MN layout, rows of 256 bytes or more");
    const uint32_t tile = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)lds;
    const uint32_t a = ((tile + 256 * (base >> 7) + (uint32_t)frag16_tr_lane(lane, OT::ROW_BYTES)) ^
                        (uint32_t)(32 * ((base >> 4) & 7))) +
                       (uint32_t)(32 * kk * OT::ROW_BYTES);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(uintptr_t)a);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(uintptr_t)(a + 4 * OT::ROW_BYTES));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// One 16 x 128 operand fragment of v_mfma_scale_f32_16x16x128_f8f6f4 on
// 8-bit elements (k-step kk of 128): lane l gets row/column (l & 15) of the
// fragment starting at `base`, byte b standing for
// k = 128*kk + 16*((l >> 4) + 4*(b >> 4)) + (b & 15) (frag16_kc8_offset).
template <class OT>
__device__ __forceinline__ v8i32 read_frag16_8(const char *lds, int lane, int base, int kk) {
  static_assert(OT::ES == 1, "8-bit tile");
  if constexpr (OT::kcontig) {
    const u32x4 lo = *(const u32x4 *)(lds + frag16_kc8_offset(lane, base, kk, 0, OT::ROW_BYTES));
    const u32x4 hi = *(const u32x4 *)(lds + frag16_kc8_offset(lane, base, kk, 1, OT::ROW_BYTES));
    return __builtin_bit_cast(v8i32, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else if constexpr (!LSM_TR_READ) {
    static_assert(OT::mf16, "16 x 16 x 128 MN layout");
    const int col = base + (lane & 15);
    v8i32 f;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; b++)
        v |= (uint32_t)*(const unsigned char *)(lds + mn16_chunk_offset(128 * kk + 16 * ((lane >> 4) + 4 * (w >> 2)) +
                                                                              4 * (w & 3) + b,
                                                                          col / 16, OT::ROW_BYTES, 1) +
                                                 (col & 15))
             << (8 * b);
      f[w] = (int)v;
    }
    return f;
  } else {
    // lds + frag16_tr8_offset(lane, base, kk, q, ROW_BYTES), computed as
    // ((tile + 256*(base >> 8) + lane part) XOR 16*((base >> 4) & 15)) + the
    // k-step and q rows, which equals it because the tile base (a multiple of
    // 1 KiB) has bits 4-7 clear.
    static_assert(OT::mf16 && OT::ROW_BYTES >= 256 && OT::ROW_BYTES % 256 == 0 && OT::BYTES % 1024 == 0,
                  "16 x 16 x 128 MN layout, rows a multiple of 256 bytes");
    const uint32_t tile = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)lds;
    const uint32_t a = ((tile + 256 * (base >> 8) + (uint32_t)frag16_tr8_lane(lane, OT::ROW_BYTES)) ^
                        (uint32_t)(16 * ((base >> 4) & 15))) +
                       (uint32_t)(128 * kk * OT::ROW_BYTES);
    v2i32 p[4];
#pragma unroll
    for (int q = 0; q < 4; q++)
      p[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i32 *)(uintptr_t)(a + (uint32_t)(frag16_tr8_rows(0, q) * OT::ROW_BYTES)));
    const auto lo = __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3);
    const auto hi = __builtin_shufflevector(p[2], p[3], 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// 16 x 16 fragment of the input type.
template <class OT, int IN>
__device__ __forceinline__ typename InT<IN>::frag read_frag16_in(const char *lds, int lane, int base, int kk) {
  if constexpr (IN == IN_E4M3)
    return read_frag16_8<OT>(lds, lane, base, kk);
  else
    return read_frag16<OT>(lds, lane, base, kk);
}

// C is written with non-temporal stores: nothing in the kernel reads it back,
// and on MI355X streaming it past the caches gave the fp32 8192^3 case 3-5%.
template <int OUT>
__device__ __forceinline__ void store_out(void *C, int64_t idx, float v) {
  if constexpr (OUT == OUT_F32) {
    __builtin_nontemporal_store(v, (float *)C + idx);
  } else if constexpr (OUT == OUT_BF16) {
    // v_cvt_pk_bf16_f32: round to nearest even
    __builtin_nontemporal_store((__bf16)v, (__bf16 *)C + idx);
  } else {
    // v_cvt_f16_f32: round to nearest even
    __builtin_nontemporal_store((_Float16)v, (_Float16 *)C + idx);
  }
}

template <int OUT>
struct OutElem;
template <>
struct OutElem<OUT_F32> { typedef float type; };
template <>
struct OutElem<OUT_BF16> { typedef __bf16 type; };
template <>
struct OutElem<OUT_F16> { typedef _Float16 type; };

// Epilogue: each wave stores its accumulator blocks (layout AccLayout<MF>)
// straight from registers.  Interior tiles store unmasked; edge tiles mask
// rows >= M and columns >= N.
template <class T, int OUT, int MF = 32>
__device__ __forceinline__ void epilogue(void *C,
                                         const typename AccLayout<MF>::type (&acc)[T::TM / MF][T::TN / MF],
                                         int M, int N, int64_t ldc, int m0, int n0, int wm, int wn,
                                         int lane) {
  using L = AccLayout<MF>;
  const bool interior = M - m0 >= T::BM && N - n0 >= T::BN;
  const int row0 = m0 + wm * T::TM + L::lane_row(lane);
  const int col0 = n0 + wn * T::TN + L::col(lane);
  if (interior) {
#pragma unroll
    for (int i = 0; i < T::TM / MF; i++)
#pragma unroll
      for (int j = 0; j < T::TN / MF; j++)
#pragma unroll
        for (int r = 0; r < L::R; r++)
          store_out<OUT>(C, (int64_t)(row0 + MF * i + L::reg_row(r)) * ldc + col0 + MF * j,
                         acc[i][j][r]);
  } else {
#pragma unroll
    for (int i = 0; i < T::TM / MF; i++)
#pragma unroll
      for (int j = 0; j < T::TN / MF; j++)
#pragma unroll
        for (int r = 0; r < L::R; r++) {
          const int row = row0 + MF * i + L::reg_row(r);
          const int col = col0 + MF * j;
          if (row < M && col < N) store_out<OUT>(C, (int64_t)row * ldc + col, acc[i][j][r]);
        }
  }
}

// LDS-staged epilogue ("An educational GEMM ladder for Helios GPUs",
// "Level 10"): each wave converts its accumulators to the output type into a
// private LDS region laid out row-major, then reads it back 16 bytes per lane
// and stores whole 16-byte pieces of C rows, so every store instruction
// covers full 128-byte lines (4 rows of 64 fp32, 8 rows of 64 bf16/fp16)
// instead of 32-lane half rows.  Needs the wave tile 64 columns wide, C
// 16-byte aligned with ldc*sizeof(out) a multiple of 16, and the LDS free
// (every wave past its last LDS read of the main loop).  `lds_bytes` is the
// LDS the kernel owns; the wave tile is staged in passes of as many rows as
// fit.
// Region layout: row-major, 64 elements per row, 16-byte chunks swizzled per
// accumulator layout (epi_stage_offset in lds_layout.h) so that every
// accumulator write and every 16-byte read is conflict-free.
template <class T, int OUT, int LDS_BYTES, int MF = 32>
__device__ __forceinline__ void epilogue_lds(void *C,
                                             const typename AccLayout<MF>::type (&acc)[T::TM / MF][T::TN / MF],
                                             char *lds, int M, int N, int64_t ldc, int m0, int n0,
                                             int wm, int wn, int wave, int lane) {
  using L = AccLayout<MF>;
  static_assert(T::TN == 64, "wave tile 64 columns wide");
  typedef typename OutElem<OUT>::type E;
  constexpr int ESZ = sizeof(E);
  constexpr int ROWB = T::TN * ESZ;                          // 256 (fp32) or 128 bytes
  constexpr int CPR = ROWB / 16;                             // 16-byte chunks per row
  constexpr int WAVES = T::WM * T::WN;
  constexpr int FIT = LDS_BYTES / (WAVES * ROWB);            // rows per wave that fit
  constexpr int PR = FIT >= T::TM ? T::TM : (FIT >= 64 ? 64 : 32);   // rows per pass
  static_assert(PR % 32 == 0 && T::TM % PR == 0 && WAVES * PR * ROWB <= LDS_BYTES, "staging fits");
  constexpr int RPI = 64 * 16 / ROWB;                        // rows per 64-lane read
  char *mine = lds + wave * PR * ROWB;
  auto off = [&](int row, int chunk) { return epi_stage_offset(row, chunk, ROWB, MF); };
  lds_poison(mine, PR * ROWB, lane, 64);   // poison build: the wave's region, before its writes
  const int grow0 = m0 + wm * T::TM;
  const int gcol0 = n0 + wn * T::TN;
#pragma unroll
  for (int pass = 0; pass < T::TM / PR; pass++) {
    // accumulator blocks i of this pass: rows MF*i .. MF*i + MF - 1 of the wave tile
#pragma unroll
    for (int i = pass * PR / MF; i < (pass + 1) * PR / MF; i++)
#pragma unroll
      for (int j = 0; j < T::TN / MF; j++)
#pragma unroll
        for (int r = 0; r < L::R; r++) {
          const int row = MF * i - pass * PR + L::row(r, lane);
          const int col = MF * j + L::col(lane);
          *(E *)(mine + off(row, col * ESZ / 16) + (col * ESZ) % 16) = (E)acc[i][j][r];
        }
    // The reads below return rows written by other lanes of this wave: LDS
    // executes a wave's instructions in order, so no barrier is needed.
#pragma unroll
    for (int it = 0; it < PR / RPI; it++) {
      const int row = it * RPI + lane / CPR;
      const int chunk = lane % CPR;
      const u32x4 v = *(const u32x4 *)(mine + off(row, chunk));
      const int grow = grow0 + pass * PR + row;
      const int gcol = gcol0 + chunk * (16 / ESZ);
      if (grow < M) {
        E *dst = (E *)C + (int64_t)grow * ldc + gcol;
        if (gcol + 16 / ESZ <= N) {
          __builtin_nontemporal_store(v, (u32x4 *)dst);
        } else {
          const E *e = (const E *)&v;
#pragma unroll
          for (int q = 0; q < 16 / ESZ; q++)
            if (gcol + q < N) __builtin_nontemporal_store(e[q], dst + q);
        }
      }
    }
  }
}

// Workgroup-row epilogue (the ping-pong kernel's): the whole workgroup
// stages C through LDS, RP = LDS_BYTES / (BN * sizeof(out)) rows at a time,
// so that each 64-lane store writes whole rows of the workgroup tile (1 KiB
// of fp32, or two 512-byte rows of bf16/fp16) instead of the 256- or
// 128-byte pieces of one wave's tile that epilogue_lds stores.  The waves
// whose rows a pass holds write their accumulators (epi_row_stage_offset in
// lds_layout.h: every write and every 16-byte read conflict-free); after a
// barrier every wave reads and stores RP / waves rows; a barrier ends the
// pass.  Called by every wave of the workgroup, with the LDS free.  On MI355X
// it measured 0.2-0.8% faster than epilogue_lds in the ping-pong kernel
// (bf16 8192^3, 4096^3 with bf16 output, E4M3 8192^3; bit-exact).
template <class T, int OUT, int LDS_BYTES, int MF>
__device__ __forceinline__ void epilogue_lds_rows(void *C,
                                                  const typename AccLayout<MF>::type (&acc)[T::TM / MF][T::TN / MF],
                                                  char *lds, int M, int N, int64_t ldc, int m0, int n0,
                                                  int wm, int wn, int wave, int lane) {
  using L = AccLayout<MF>;
  typedef typename OutElem<OUT>::type E;
  constexpr int ESZ = sizeof(E);
  constexpr int WROWB = T::BN * ESZ;                      // bytes of one workgroup-tile row
  constexpr int CPR = WROWB / 16;                         // 16-byte chunks per row
  constexpr int RP = LDS_BYTES / WROWB < T::BM ? LDS_BYTES / WROWB : T::BM;   // rows per pass
  constexpr int WAVES = T::WM * T::WN;
  constexpr int RPW = RP / WAVES;                         // rows each wave stores per pass
  constexpr int RPI = 64 / CPR >= 1 ? 64 / CPR : 1;       // rows per 64-lane read
  static_assert(RP % T::TM == 0 && RP * WROWB <= LDS_BYTES && CPR <= 64 && 64 % CPR == 0 &&
                RPW % RPI == 0, "workgroup-row staging geometry");
  auto off = [&](int row, int chunk) { return epi_row_stage_offset(row, chunk, WROWB, MF, ESZ); };
  if constexpr (LSM_LDS_POISON) {   // poison build: the staging region, before its writes
    lds_poison(lds, RP * WROWB, wave * 64 + lane, WAVES * 64);
    __syncthreads();
  }
#pragma unroll
  for (int pass = 0; pass < T::BM / RP; pass++) {
    if (wm * T::TM >= pass * RP && wm * T::TM < (pass + 1) * RP) {
#pragma unroll
      for (int i = 0; i < T::TM / MF; i++)
#pragma unroll
        for (int j = 0; j < T::TN / MF; j++)
#pragma unroll
          for (int r = 0; r < L::R; r++) {
            const int row = wm * T::TM - pass * RP + MF * i + L::row(r, lane);
            const int col = wn * T::TN + MF * j + L::col(lane);
            *(E *)(lds + off(row, col * ESZ / 16) + (col * ESZ) % 16) = (E)acc[i][j][r];
          }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < RPW / RPI; it++) {
      const int row = wave * RPW + it * RPI + lane / CPR;
      const int chunk = lane % CPR;
      const u32x4 v = *(const u32x4 *)(lds + off(row, chunk));
      const int grow = m0 + pass * RP + row;
      const int gcol = n0 + chunk * (16 / ESZ);
      if (grow < M) {
        E *dst = (E *)C + (int64_t)grow * ldc + gcol;
        if (gcol + 16 / ESZ <= N) {
          __builtin_nontemporal_store(v, (u32x4 *)dst);
        } else {
          const E *e = (const E *)&v;
#pragma unroll
          for (int q = 0; q < 16 / ESZ; q++)
            if (gcol + q < N) __builtin_nontemporal_store(e[q], dst + q);
        }
      }
    }
    if (pass + 1 < T::BM / RP) __syncthreads();
  }
}

// Operand fragment for input type IN (k-step kk of the tile).
template <class OT, int IN>
__device__ __forceinline__ typename InT<IN>::frag read_frag_in(const char *lds, int lane, int base,
                                                               int kk) {
  if constexpr (IN == IN_E4M3)
    return read_frag8<OT>(lds, lane, base, kk);
  else
    return read_frag<OT>(lds, lane, base, kk);
}

// LDS read instructions per fragment.
template <class OT, int IN>
constexpr int frag_reads() {
  return IN == IN_E4M3 ? (OT::kcontig ? 2 : 4) : (OT::kcontig ? 1 : 2);
}

}  // namespace lsm
