// hw_probe.hip -- small one-wave kernels that exercise, in isolation, the
// hardware behaviour the GEMM kernels rely on, so that tests can check it
// against the CPU formulas of lds_layout.h and gemm_common.h:
//
//  * the fragment reads: an LDS tile image laid out by the host with the
//    library's own layout functions is read back with the library's own
//    device read functions (ds_read_b128, ds_read_b64_tr_b16,
//    ds_read_b64_tr_b8 and their address functions), and each lane's
//    fragment is returned;
//  * the MFMA operand and accumulator layouts: one MFMA (16x16x32 or
//    32x32x16 on 16-bit inputs, 16x16x128 or 32x32x64 on E4M3) on operand
//    registers the host fills, with every accumulator register returned;
//  * the buffer range check the direct-to-LDS loads use for their edges:
//    loads whose vector offset is in range and whose vector plus scalar
//    offset is not, into registers and into LDS;
//  * a one-wave strided column read of a padded 64 x (64 + PAD) fp16 LDS
//    tile ("Lds Optimization", "Optimization Method 2: Padding", the
//    measured padding table), for calibrating the bank-conflict counters;
//  * one wave repeating one LDS read (ds_read_b64, ds_read_b64_tr_b8 or
//    ds_read_b128) at 64 lane addresses the host chooses, so the counters can
//    tell how the hardware groups a wave's lanes into bank passes.
//
// Built into libhw_probe.so next to the library; only the tests and the
// benchmark's probe modes load it.  Every kernel runs one wave (64 threads)
// and touches only the buffers it is given, at offsets the host has sized.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "gemm_kernel_dma.h"

using namespace lsm;

namespace {

constexpr int kImageMax = 32768;   // largest tile image a probe copies into LDS

// ------------------------------------------------------------ fragment reads

// Copies `bytes` (a multiple of 16, at most kImageMax) of the tile image into
// LDS, then every lane reads its fragment (base, kk) of operand tile OT with
// the library's read function for MFMA shape MF and input type IN and writes
// it to out[lane].
template <class OT, int IN, int MF>
__global__ __launch_bounds__(64) void frag_probe_kernel(const u32x4 *__restrict__ image, int bytes,
                                                        int base, int kk,
                                                        typename InT<IN>::frag *__restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[kImageMax];
  const int lane = threadIdx.x;
  for (int i = lane; i < bytes / 16; i += 64) ((u32x4 *)lds)[i] = image[i];
  __syncthreads();
  typename InT<IN>::frag f;
  if constexpr (MF == 16)
    f = read_frag16_in<OT, IN>(lds, lane, base, kk);
  else
    f = read_frag_in<OT, IN>(lds, lane, base, kk);
  out[lane] = f;
}

// Tile geometries of the kernels (256 loader threads; K-contiguous rows of
// BK elements, MN-contiguous rows of the tile width).
using KC256 = OperandTile<256, 64, KC, 256, 2>;         // 128-byte rows
using KC64x128 = OperandTile<64, 128, KC, 256, 2>;      // 256-byte rows
using MN256 = OperandTile<256, 64, MNC, 256, 2>;        // 512-byte rows, 32x32 layout
using MN128 = OperandTile<128, 64, MNC, 256, 2>;        // 256-byte rows
using MN64 = OperandTile<64, 64, MNC, 256, 2>;          // 128-byte rows
using MN256_16 = OperandTile<256, 64, MNC, 256, 2, 1>;  // 512-byte rows, 16x16x32 layout
using KC256_16 = OperandTile<256, 64, KC, 256, 2, 1>;
using KC8 = OperandTile<256, 128, KC, 256, 1>;          // E4M3, 128-byte rows
using MN8 = OperandTile<256, 128, MNC, 256, 1>;         // E4M3, 256-byte rows
using MN8_128 = OperandTile<128, 128, MNC, 256, 1>;     // E4M3, 128-byte rows
using KC8_16 = OperandTile<256, 128, KC, 256, 1, 1>;    // E4M3, 16x16x128 fragments
using MN8_16 = OperandTile<256, 128, MNC, 256, 1, 1>;   // E4M3, 256-byte rows, 16x16x128 layout

// ------------------------------------------------------------ MFMA layouts

// One MFMA on operand fragments a[lane], b[lane] with a zero accumulator;
// accumulator register r of lane l goes to out[r * 64 + l].
template <int IN, int MF>
__global__ __launch_bounds__(64) void mfma_probe_kernel(const typename InT<IN>::frag *__restrict__ a,
                                                        const typename InT<IN>::frag *__restrict__ b,
                                                        float *__restrict__ out) {
  const int lane = threadIdx.x;
  using L = AccLayout<MF>;
  typename L::type acc;
#pragma unroll
  for (int r = 0; r < L::R; r++) acc[r] = 0.f;
  if constexpr (MF == 16)
    acc = mfma16_step<IN>(a[lane], b[lane], acc);
  else
    acc = mfma_step<IN>(a[lane], b[lane], acc);
#pragma unroll
  for (int r = 0; r < L::R; r++) out[r * 64 + lane] = acc[r];
}

// ------------------------------------------------------------ buffer range check

// Lane l loads the 16 bytes at buffer offset voff = 16*l plus the scalar
// offset `soff` through a buffer resource of `num_records` bytes, once into
// registers (out_reg[l]) and once with the direct-to-LDS form the GEMM
// kernels use (out_lds[l], read back from LDS).  The host keeps
// 16*63 + soff + 16 within the allocation behind `buf`.
__global__ __launch_bounds__(64) void range_probe_kernel(const void *buf, uint32_t num_records,
                                                         uint32_t soff, u32x4 *__restrict__ out_reg,
                                                         u32x4 *__restrict__ out_lds) {
  __shared__ __attribute__((aligned(1024))) u32x4 lds[64];
  const int lane = threadIdx.x;
  const i32x4 rs = buffer_rsrc(buf, num_records);
  lds[lane] = u32x4{0xDEADBEEFu, 0xDEADBEEFu, 0xDEADBEEFu, 0xDEADBEEFu};
  __syncthreads();
  u32x4 v;
  // the load and its wait in one statement, so the result registers are
  // complete when the statement ends
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen\n\ts_waitcnt vmcnt(0)"
               : "=v"(v)
               : "v"((uint32_t)(16 * lane)), "s"(rs), "s"(soff)
               : "memory");
  out_reg[lane] = v;
  const uint32_t block = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
  dma16(rs, block, (uint32_t)(16 * lane), soff);
  wait_dma();
  __syncthreads();
  out_lds[lane] = lds[lane];
}

// ------------------------------------------------------------ padded column reads

// One wave walks a column of a 64 x (64 + PAD) fp16 LDS tile: lane t reads
// element [t][c] for c = 0, 1, ..., `iters` times in a dependent chain (each
// read's column comes from the previous value), and lane 0 writes the sum.
template <int PAD>
__global__ __launch_bounds__(64) void pad_probe_kernel(int iters, float *__restrict__ out) {
  constexpr int W = 64 + PAD;
  __shared__ _Float16 tile[64 * W];
  const int lane = threadIdx.x;
  for (int i = lane; i < 64 * W; i += 64) tile[i] = (_Float16)0.0f;
  __syncthreads();
  float acc = 0.f;
  int c = 0;
  for (int it = 0; it < iters; it++) {
    const float v = (float)tile[lane * W + c];
    acc += v;
    c = (c + 1 + (int)v) & 63;       // v is 0: the next column, chained on the read
  }
  if (lane == 0) out[0] = acc;
}

// ------------------------------------------------------------ lane-address reads

constexpr int kReadLds = 65536;   // LDS bytes of the read probe
struct LaneAddrs { int a[64]; };

// Fills the LDS with a counting pattern, then every lane repeats one read of
// kind MODE (0 ds_read_b64, 1 ds_read_b64_tr_b8, 2 ds_read_b128) at its byte
// address a[lane], `iters` times, each read's result folded into a sum that
// lane writes to out[lane].  The host checks every address (in range and
// aligned) before the launch.
template <int MODE>
__global__ __launch_bounds__(64) void read_probe_kernel(LaneAddrs addrs, int iters, int *__restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[kReadLds];
  const int lane = threadIdx.x;
  for (int i = lane; i < kReadLds / 4; i += 64) ((int *)lds)[i] = i;
  __syncthreads();
  int acc = 0;
  for (int it = 0; it < iters; it++) {
    int off = addrs.a[lane];
    asm volatile("" : "+v"(off));   // opaque address: one read per iteration
    if constexpr (MODE == 2) {
      const u32x4 w = *(const u32x4 *)(lds + off);
      acc += (int)(w[0] ^ w[1] ^ w[2] ^ w[3]);
    } else {
      v2i32 v;
      if constexpr (MODE == 1)
        v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32 *)(lds + off));
      else
        v = *(const lds_v2i32 *)(lds + off);
      acc += v[0] ^ v[1];
    }
  }
  out[lane] = acc;
}

template <class OT, int IN, int MF>
int launch_frag(const void *image, int bytes, int base, int kk, void *out, hipStream_t s) {
  if (bytes != OT::BYTES || bytes > kImageMax || bytes % 16) return -1;
  hipLaunchKernelGGL((frag_probe_kernel<OT, IN, MF>), dim3(1), dim3(64), 0, s,
                     (const u32x4 *)image, bytes, base, kk, (typename InT<IN>::frag *)out);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" {

// Tile kinds of lsm_probe_frag.
enum {
  PROBE_KC256 = 0, PROBE_KC64x128 = 1, PROBE_MN256 = 2, PROBE_MN128 = 3, PROBE_MN64 = 4,
  PROBE_MN256_16 = 5, PROBE_KC256_16 = 6, PROBE_KC8 = 7, PROBE_MN8 = 8, PROBE_MN8_128 = 9,
  PROBE_KC8_16 = 10, PROBE_MN8_16 = 11
};

// Reads fragment (base, kk) of a tile image of `bytes` bytes; out receives
// 64 lanes x 16 bytes (16-bit kinds) or 64 x 32 bytes (E4M3 kinds).
// Returns 0, or -1 for an unknown kind or a size that is not the tile's.
int lsm_probe_frag(int kind, const void *image, int bytes, int base, int kk, void *out,
                   hipStream_t s) {
  switch (kind) {
    case PROBE_KC256: return launch_frag<KC256, IN_BF16, 32>(image, bytes, base, kk, out, s);
    case PROBE_KC64x128: return launch_frag<KC64x128, IN_BF16, 32>(image, bytes, base, kk, out, s);
    case PROBE_MN256: return launch_frag<MN256, IN_BF16, 32>(image, bytes, base, kk, out, s);
    case PROBE_MN128: return launch_frag<MN128, IN_BF16, 32>(image, bytes, base, kk, out, s);
    case PROBE_MN64: return launch_frag<MN64, IN_BF16, 32>(image, bytes, base, kk, out, s);
    case PROBE_MN256_16: return launch_frag<MN256_16, IN_BF16, 16>(image, bytes, base, kk, out, s);
    case PROBE_KC256_16: return launch_frag<KC256_16, IN_BF16, 16>(image, bytes, base, kk, out, s);
    case PROBE_KC8: return launch_frag<KC8, IN_E4M3, 32>(image, bytes, base, kk, out, s);
    case PROBE_MN8: return launch_frag<MN8, IN_E4M3, 32>(image, bytes, base, kk, out, s);
    case PROBE_MN8_128: return launch_frag<MN8_128, IN_E4M3, 32>(image, bytes, base, kk, out, s);
    case PROBE_KC8_16: return launch_frag<KC8_16, IN_E4M3, 16>(image, bytes, base, kk, out, s);
    case PROBE_MN8_16: return launch_frag<MN8_16, IN_E4M3, 16>(image, bytes, base, kk, out, s);
    default: return -1;
  }
}

// One MFMA: shape 16 (v_mfma_f32_16x16x32, or v_mfma_scale_f32_16x16x128_f8f6f4
// with unit scales for in_type 2) or 32 (v_mfma_f32_32x32x16, or
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales for in_type 2), input
// type 0 bf16, 1 fp16, 2 E4M3.  a, b: 64 lanes x 16 bytes (32 for E4M3);
// out: 4 or 16 registers x 64 lanes of fp32.
int lsm_probe_mfma(int shape, int in_type, const void *a, const void *b, float *out,
                   hipStream_t s) {
  if (shape == 16 && in_type == IN_BF16)
    hipLaunchKernelGGL((mfma_probe_kernel<IN_BF16, 16>), dim3(1), dim3(64), 0, s, (const v8i16 *)a,
                       (const v8i16 *)b, out);
  else if (shape == 16 && in_type == IN_F16)
    hipLaunchKernelGGL((mfma_probe_kernel<IN_F16, 16>), dim3(1), dim3(64), 0, s, (const v8i16 *)a,
                       (const v8i16 *)b, out);
  else if (shape == 32 && in_type == IN_BF16)
    hipLaunchKernelGGL((mfma_probe_kernel<IN_BF16, 32>), dim3(1), dim3(64), 0, s, (const v8i16 *)a,
                       (const v8i16 *)b, out);
  else if (shape == 32 && in_type == IN_F16)
    hipLaunchKernelGGL((mfma_probe_kernel<IN_F16, 32>), dim3(1), dim3(64), 0, s, (const v8i16 *)a,
                       (const v8i16 *)b, out);
  else if (shape == 16 && in_type == IN_E4M3)
    hipLaunchKernelGGL((mfma_probe_kernel<IN_E4M3, 16>), dim3(1), dim3(64), 0, s, (const v8i32 *)a,
                       (const v8i32 *)b, out);
  else if (shape == 32 && in_type == IN_E4M3)
    hipLaunchKernelGGL((mfma_probe_kernel<IN_E4M3, 32>), dim3(1), dim3(64), 0, s, (const v8i32 *)a,
                       (const v8i32 *)b, out);
  else
    return -1;
  return (int)hipGetLastError();
}

// Buffer range check: see range_probe_kernel.  The caller guarantees that
// `buf` spans at least 16*64 + soff bytes; out_reg and out_lds receive 64 x 16
// bytes each.
int lsm_probe_range(const void *buf, uint32_t num_records, uint32_t soff, void *out_reg,
                    void *out_lds, hipStream_t s) {
  hipLaunchKernelGGL(range_probe_kernel, dim3(1), dim3(64), 0, s, buf, num_records, soff,
                     (u32x4 *)out_reg, (u32x4 *)out_lds);
  return (int)hipGetLastError();
}

// Lane-address read probe: mode 0 ds_read_b64, 1 ds_read_b64_tr_b8, 2
// ds_read_b128; addr: 64 host ints (byte addresses, 8-byte aligned, 16 for
// mode 2, each read inside the 64 KiB probe LDS); out: 64 device ints.
// Returns -1, launching nothing, for a bad mode or address.
int lsm_probe_lds_read(int mode, const int *addr, int iters, int *out, hipStream_t s) {
  LaneAddrs a;
  const int width = mode == 2 ? 16 : 8;
  if (mode < 0 || mode > 2 || iters < 0) return -1;
  for (int l = 0; l < 64; l++) {
    if (addr[l] < 0 || addr[l] % width != 0 || addr[l] + width > kReadLds) return -1;
    a.a[l] = addr[l];
  }
  if (mode == 2)
    hipLaunchKernelGGL(read_probe_kernel<2>, dim3(1), dim3(64), 0, s, a, iters, out);
  else if (mode == 1)
    hipLaunchKernelGGL(read_probe_kernel<1>, dim3(1), dim3(64), 0, s, a, iters, out);
  else
    hipLaunchKernelGGL(read_probe_kernel<0>, dim3(1), dim3(64), 0, s, a, iters, out);
  return (int)hipGetLastError();
}

// Padded column walk: pad 0, 1, 2, 4 or 32; out receives one float.
int lsm_probe_pad(int pad, int iters, float *out, hipStream_t s) {
  switch (pad) {
    case 0: hipLaunchKernelGGL(pad_probe_kernel<0>, dim3(1), dim3(64), 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL(pad_probe_kernel<1>, dim3(1), dim3(64), 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL(pad_probe_kernel<2>, dim3(1), dim3(64), 0, s, iters, out); break;
    case 4: hipLaunchKernelGGL(pad_probe_kernel<4>, dim3(1), dim3(64), 0, s, iters, out); break;
    case 32: hipLaunchKernelGGL(pad_probe_kernel<32>, dim3(1), dim3(64), 0, s, iters, out); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
