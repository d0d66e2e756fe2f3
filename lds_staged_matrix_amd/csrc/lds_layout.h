// lds_layout.h -- LDS tile layouts and per-lane LDS addresses of the GEMM.
//
// Pure integer functions, usable on the host (the bank-conflict model in the
// tests evaluates exactly these) and on the device (the kernel computes every
// LDS address with them).
//
// gfx950 LDS: 64 banks of 4 bytes, bank = (byte_address / 4) mod 64, so one
// 256-byte line touches every bank once ("Lds Optimization", section "LDS
// Architecture on CDNA4 (gfx950)", Hardware Facts).  Addresses that differ by
// a multiple of 256 bytes share banks; a 256-byte row stride is a 64-way
// conflict for a column walk (same page, "Impact on Bank Conflict Analysis").
// The fix used here is an XOR swizzle of the 16-byte chunk index with bits of
// the row index (same page, "Optimization Method 1: Swizzle Layout"), applied
// identically on the write and the read side (same page, "Verification
// Checklist", item 1).  The swizzle unit is a whole 16-byte chunk, never less
// than one lane's access, so every ds_write_b128 / ds_read_b128 stays one
// contiguous 16-byte vector ("Fix LDS vectorization logic to allow for bank
// conflict resolution when kPack > kPerThread": a write that is neither
// vectorised nor rotated is the 8-way case).
//
// Two tile kinds:
//  * K-contiguous tile: rows are M (or N) indices, each row holds the tile's
//    K extent contiguously (row_bytes = 2*BK).  Read with ds_read_b128: one
//    lane takes 8 consecutive k of one row.  A 16-lane phase reads 16
//    consecutive rows at one logical chunk; the swizzle puts them in 16
//    distinct 16-byte bank groups.
//  * MN-contiguous tile: rows are k indices, each row holds the tile's M (or
//    N) extent contiguously.  Read with ds_read_b64_tr_b16 ("Lds
//    Optimization", section "MFMA Transpose Load from LDS (gfx950 only)"): a
//    lane reads 4 consecutive M/N values of one k row and the hardware
//    redistributes them so each lane ends up with 4 consecutive k of one
//    column.  Bank conflicts are decided by the source addresses ("A Deep
//    Dive into LDS Optimizations on AMD Instinct MI450 GPUs", Part I, end of
//    "What Does ds_load_tr Do?").
//
// Lane redistribution of ds_read_b64_tr_b16 on gfx950 (measured on MI355X;
// tests/test_gpu_hw_maps.py reads every fragment of every tile kind through
// the probe kernels of hw_probe.hip and checks it against these functions):
// inside each aligned group of 16 lanes, destination lane d receives,
// as its element j (j = 0..3), element (d & 3) of source lane (d >> 2) + 4*j.
// Hence, for destination lane d to hold column c0 + d of rows r0..r0+3,
// source lane s reads row r0 + (s >> 2), columns c0 + 4*(s & 3) .. +3.
#pragma once

#include <hip/hip_runtime.h>

// LSM_LDS_SWIZZLE = 0 builds the same kernels with unswizzled (row-major)
// LDS tiles; it exists only for the A/B build that measures what the
// swizzle buys.  The library is built with the default, 1.
#ifndef LSM_LDS_SWIZZLE
#define LSM_LDS_SWIZZLE 1
#endif

namespace lsm {

// ---------------------------------------------------------------- swizzles

// XOR applied to the chunk index of row `row` of a K-contiguous tile.
__host__ __device__ constexpr int kc_swizzle(int row, int row_bytes) {
  // rows per 256-byte bank line and chunks per row
  return !LSM_LDS_SWIZZLE ? 0
         : row_bytes >= 256 ? (row & 15)
                            : ((row / (256 / row_bytes)) & (row_bytes / 16 - 1));
}

// XOR applied to the chunk index of k-row `k` of an MN-contiguous tile of
// `es`-byte elements.  16-bit elements (ds_read_b64_tr_b16): one 32-lane
// transposed-read phase reads 4 k-rows x 64 bytes, and the XOR puts the four
// rows in four distinct 64-byte quarters of the bank line.  8-bit elements
// (ds_read_b64_tr_b8): a phase reads 8 k-rows x 32 bytes, and the XOR puts
// the eight rows in eight distinct 32-byte eighths of the bank line.
__host__ __device__ constexpr int mn_swizzle(int k, int row_bytes, int es = 2) {
  return !LSM_LDS_SWIZZLE ? 0
         : es == 2 ? (row_bytes >= 256 ? 4 * (k & 3) : (row_bytes == 128 ? 4 * ((k >> 1) & 1) : 0))
                   : (row_bytes >= 256 ? 2 * (k & 7)
                                       : row_bytes == 128 ? 2 * ((k >> 1) & 3)
                                                          : (row_bytes == 64 ? 2 * ((k >> 2) & 1) : 0));
}

// XOR applied to the chunk index of k-row `k` of an MN-contiguous tile of
// 16-bit elements read by the transposed fragments of v_mfma_f32_16x16x32.
// Those fragments hold k = 8g .. 8g+7 in lane group g (16 lanes), so one
// 32-lane phase of ds_read_b64_tr_b16 reads k-rows {k..k+3} and {k+8..k+11},
// 32 bytes each.  For rows of 256 bytes or more every row starts at the same
// bank, and the XOR (k & 3) | ((k >> 1) & 4), on chunk bits 1-3, puts those
// eight rows in the eight distinct 32-byte eighths of the bank line.  Its
// period in k is 16, so a loader whose rounds are 8 rows apart needs one lane
// offset for even and one for odd rounds.
__host__ __device__ constexpr int mn16_swizzle(int k, int row_bytes) {
  return (!LSM_LDS_SWIZZLE || row_bytes < 256) ? 0 : 2 * ((k & 3) | ((k >> 1) & 4));
}

// The same for 8-bit elements read by the transposed fragments of
// v_mfma_scale_f32_16x16x128_f8f6f4.  Those fragments (frag16_tr8_offset)
// hold k-rows 16g .. 16g+15 and 64+16g .. 64+16g+15 in lane group g, eight
// k-rows per ds_read_b64_tr_b8, so one 32-lane phase reads k-rows
// {k..k+7} and {k+16..k+23}, 16 bytes each.  The XOR (k & 7) | ((k >> 1) & 8)
// puts those sixteen rows in the sixteen 16-byte bank groups of the line.  It
// depends on k only through k & 7 and bit 4, so a loader whose rounds are 16
// rows apart needs one lane offset for even and one for odd rounds.
__host__ __device__ constexpr int mn16_swizzle8(int k, int row_bytes) {
  return (!LSM_LDS_SWIZZLE || row_bytes < 256) ? 0 : (k & 7) | ((k >> 1) & 8);
}

// Byte offset of 16-byte chunk `chunk` of row `row` in a K-contiguous tile.
__host__ __device__ constexpr int kc_chunk_offset(int row, int chunk, int row_bytes) {
  return row * row_bytes + 16 * (chunk ^ kc_swizzle(row, row_bytes));
}

// Byte offset of 16-byte chunk `chunk` of k-row `k` in an MN-contiguous tile.
__host__ __device__ constexpr int mn_chunk_offset(int k, int chunk, int row_bytes, int es = 2) {
  return k * row_bytes + 16 * (chunk ^ mn_swizzle(k, row_bytes, es));
}

// Byte offset of 16-byte chunk `chunk` of k-row `k` in an MN-contiguous tile
// laid out for the 16 x 16 x 32 transposed reads.
__host__ __device__ constexpr int mn16_chunk_offset(int k, int chunk, int row_bytes, int es = 2) {
  return k * row_bytes + 16 * (chunk ^ (es == 2 ? mn16_swizzle(k, row_bytes) : mn16_swizzle8(k, row_bytes)));
}

// ---------------------------------------------------------------- loader

// The global->LDS loader splits a tile of `rows` x `row_bytes` into 16-byte
// chunks numbered row-major; chunk id = thread + i * threads for load i.
// Consecutive lanes take consecutive chunks of a row, so a wave's global
// access is contiguous along the operand's unit-stride dimension.
__host__ __device__ constexpr int loader_row(int id, int row_bytes) { return id / (row_bytes / 16); }
__host__ __device__ constexpr int loader_chunk(int id, int row_bytes) { return id % (row_bytes / 16); }

__host__ __device__ constexpr int loader_lds_offset(int id, int row_bytes, bool k_contig, int es = 2) {
  return k_contig ? kc_chunk_offset(loader_row(id, row_bytes), loader_chunk(id, row_bytes), row_bytes)
                  : mn_chunk_offset(loader_row(id, row_bytes), loader_chunk(id, row_bytes), row_bytes, es);
}

// The same for an MN-contiguous 16-bit tile in the 16 x 16 x 32 layout.
__host__ __device__ constexpr int loader_lds_offset16(int id, int row_bytes, int es = 2) {
  return mn16_chunk_offset(loader_row(id, row_bytes), loader_chunk(id, row_bytes), row_bytes, es);
}

// ---------------------------------------------------------------- fragment reads
//
// Fragments of v_mfma_f32_32x32x16_{bf16,f16} (checked on the GPU by the
// hardware-map probes, tests/test_gpu_hw_maps.py):
// lane l holds operand row/column (l & 31) and k = 8*(l >> 5) + i, i = 0..7,
// for both A and B.  `base` is the first M/N index of the 32-wide fragment
// inside the tile, `kk` the 16-deep k step inside the tile.

// K-contiguous operand: one ds_read_b128 per fragment.
__host__ __device__ constexpr int frag_kc_offset(int lane, int base, int kk, int row_bytes) {
  return kc_chunk_offset(base + (lane & 31), 2 * kk + (lane >> 5), row_bytes);
}

// MN-contiguous operand: two ds_read_b64_tr_b16 per fragment, half h = 0, 1
// delivering k = 8*(l >> 5) + 4*h + 0..3.  Source lane l reads k-row
// 16*kk + 8*(l >> 5) + 4*h + ((l >> 2) & 3) at columns
// base + 16*((l >> 4) & 1) + 4*(l & 3) .. +3.
__host__ __device__ constexpr int frag_tr_offset(int lane, int base, int kk, int h, int row_bytes) {
  return mn_chunk_offset(16 * kk + 8 * (lane >> 5) + 4 * h + ((lane >> 2) & 3),
                         (base + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) / 8, row_bytes) +
         8 * (lane & 1);
}

// Fragments of v_mfma_f32_16x16x32_{bf16,f16}, used by the ping-pong kernel
// on 16-bit inputs: lane l holds operand row/column (l & 15) and
// k = 8*(l >> 4) + i, i = 0..7; `kk` is the 32-deep k step inside the tile.
// `base`, the fragment's first row/column in the tile, is a multiple of 16.
// Both offsets are written as a lane-dependent part plus a part that depends
// only on `base` and `kk`, so that in an unrolled loop the compiler keeps a
// few lane constants and folds the rest into the instructions' immediates.

// K-contiguous operand: one ds_read_b128 per fragment, row base + (l & 15),
// chunk 4*kk + (l >> 4).  Every K-contiguous swizzle has a period in the row
// that divides 16, so the row's swizzle is that of row (l & 15).
__host__ __device__ constexpr int frag16_kc_offset(int lane, int base, int kk, int row_bytes) {
  return base * row_bytes + kc_chunk_offset(lane & 15, 4 * kk + (lane >> 4), row_bytes);
}

// MN-contiguous operand in the 16 x 16 x 32 layout (mn16_chunk_offset, rows
// of 256 bytes or more): two ds_read_b64_tr_b16 per fragment, half h = 0, 1
// delivering k = 8*(l >> 4) + 4*h + 0..3.  Source lane l reads k-row
// k = 32*kk + 8*(l >> 4) + 4*h + ((l >> 2) & 3) at columns base + 4*(l & 3) .. +3,
// i.e. chunk c = 2f + ((l & 3) >> 1) with f = base / 16, bytes 8*(l & 1) .. +7.
// mn16_swizzle(k) = 2s, with s = (k & 3) | ((k >> 1) & 4) a function of the
// lane alone, so the swizzled chunk is 2(f ^ s) + ((l & 3) >> 1), and with
// f = 8 fw + fi (fi < 8) the offset is
//   32*8*fw + (frag16_tr_lane(l) XOR 32*fi) + (32*kk + 4*h)*row_bytes,
// where the lane part holds the k-row, the byte within the chunk pair and
// 32*s in bits 5-7.  The kernel adds the lane part to a stage base whose bits
// 5-7 are zero and applies the XOR to the sum, so one register per operand
// serves every fragment.
__host__ __device__ constexpr int frag16_tr_lane(int lane, int row_bytes) {
  const int k0 = 8 * (lane >> 4) + ((lane >> 2) & 3);      // the k-row, less 32*kk + 4*h
  return k0 * row_bytes + 32 * (mn16_swizzle(k0, row_bytes) >> 1) + 16 * ((lane & 3) >> 1) +
         8 * (lane & 1);
}
__host__ __device__ constexpr int frag16_tr_offset(int lane, int base, int kk, int h, int row_bytes) {
  return 256 * (base >> 7) + (frag16_tr_lane(lane, row_bytes) ^ (32 * ((base >> 4) & 7))) +
         (32 * kk + 4 * h) * row_bytes;
}

// Fragments of v_mfma_scale_f32_32x32x64_f8f6f4 on 8-bit elements (checked
// on the GPU by the hardware-map probes): lane l holds operand row/column (l & 31) and 32 bytes; the
// k of byte b only has to be the same for A and B, and here it is
// k = 64*kk + 32*(l >> 5) + b.

// K-contiguous 8-bit operand: two ds_read_b128 per fragment, q = 0, 1
// delivering bytes 16q .. 16q + 15.
__host__ __device__ constexpr int frag_kc8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return kc_chunk_offset(base + (lane & 31), 4 * kk + 2 * (lane >> 5) + q, row_bytes);
}

// MN-contiguous 8-bit operand: four ds_read_b64_tr_b8 per fragment, q = 0..3
// delivering bytes 8q .. 8q + 7.  ds_read_b64_tr_b8 on gfx950 (measured, and
// checked on the GPU by the hardware-map probes): inside each aligned group of 16 lanes, destination lane d
// receives as byte j the byte (d & 7) of source lane (d >> 3) + 2j.  So
// source lane s of group g (s' = s & 15) reads k-row
// 64*kk + 32*(g >> 1) + 8q + (s' >> 1) at columns base + 16*(g & 1) +
// 8*(s' & 1) .. +7, and destination lane l ends with column base + (l & 31),
// k-rows 64*kk + 32*(l >> 5) + 8q + 0..7.
__host__ __device__ constexpr int frag_tr8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return mn_chunk_offset(64 * kk + 32 * (lane >> 5) + 8 * q + ((lane & 15) >> 1),
                         (base + 16 * ((lane >> 4) & 1)) / 16, row_bytes, 1) +
         8 * (lane & 1);
}

// Fragments of v_mfma_scale_f32_16x16x128_f8f6f4 on 8-bit elements: lane l
// holds operand row/column (l & 15) and 32 bytes; as for the 32 x 32 form only
// A and B sharing the numbering of k matters, and here byte b of lane group
// g = l >> 4 stands for k = 128*kk + 16*(g + 4*(b >> 4)) + (b & 15): the
// group's 16-byte chunks g and g + 4 of the 128-deep k step.
//
// K-contiguous: two ds_read_b128 per fragment, q = 0, 1 delivering bytes
// 16q .. 16q + 15 (chunk g + 4q).  A 16-lane group reads 16 consecutive rows
// at one logical chunk.  gfx950 serves a 64-lane ds_read_b128 in two passes
// of 32 lanes, lanes 0-15 with 32-47 and 16-31 with 48-63, over 64 banks of
// 16 bytes (measured with the bank-conflict counters); the groups that share
// a pass read chunks g and g + 2, which the K-contiguous swizzle keeps apart.
// (Chunks 2g + q would pair chunks c and c + 4, which the swizzle of rows
// r and r + 8 maps onto one bank: 2-way.)
__host__ __device__ constexpr int frag16_kc8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return kc_chunk_offset(base + (lane & 15), 8 * kk + (lane >> 4) + 4 * q, row_bytes);
}

// MN-contiguous (rows of 256 bytes or more): four ds_read_b64_tr_b8 per
// fragment, q = 0..3 delivering bytes 8q .. 8q + 7, i.e. k-rows
// 128*kk + 16g + 64*(q >> 1) + 8*(q & 1) + 0..7 of column base + (l & 15).
// With the tr_b8 lane exchange above, source lane s of group g (s' = s & 15)
// reads k-row 128*kk + 16g + 64*(q >> 1) + 8*(q & 1) + (s' >> 1) at columns
// base + 8*(s' & 1) .. +7.  The swizzle of those k-rows does not depend on q
// or kk (k & 7 and bit 4 are fixed by the lane), so the address is a lane
// part, XORed with the fragment's chunk on bits 4-7, plus the q and kk rows;
// frag16_tr8_offset is that sum.
__host__ __device__ constexpr int frag16_tr8_lane(int lane, int row_bytes) {
  const int k0 = 16 * (lane >> 4) + ((lane & 15) >> 1);   // the k-row, less the q and kk rows
  return k0 * row_bytes + 16 * mn16_swizzle8(k0, row_bytes) + 8 * (lane & 1);
}
__host__ __device__ constexpr int frag16_tr8_rows(int kk, int q) { return 128 * kk + 64 * (q >> 1) + 8 * (q & 1); }
__host__ __device__ constexpr int frag16_tr8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return 256 * (base >> 8) + (frag16_tr8_lane(lane, row_bytes) ^ (16 * ((base >> 4) & 15))) +
         frag16_tr8_rows(kk, q) * row_bytes;
}

// ---------------------------------------------------------------- epilogue staging
//
// The LDS-staged epilogue writes each wave's accumulators, converted to the
// output type, into a private region with `row_bytes` per row, then reads
// it back 16 bytes per lane.  The 16-byte chunk index is XORed with a
// function of the row so that the rows one accumulator write covers land in
// different banks:
//   32 x 32 blocks (mf = 32): lanes 0-31 and 32-63 write rows r and r + 4,
//     XOR ((row >> 2) & 1) * (chunks per row / 2), the two halves of a row;
//   16 x 16 blocks (mf = 16): the four 16-lane groups write rows r, r + 4,
//     r + 8, r + 12, XOR ((row >> 2) & 3) * (chunks per row / 4), its quarters.
// The XOR permutes chunks within a row, so reads of whole rows, 16 bytes per
// lane, touch every bank once.
__host__ __device__ constexpr int epi_stage_offset(int row, int chunk, int row_bytes, int mf) {
  return row * row_bytes + 16 * (chunk ^ (mf == 32 ? ((row >> 2) & 1) * (row_bytes / 32)
                                                   : ((row >> 2) & 3) * (row_bytes / 64)));
}

// The ping-pong kernel's workgroup-row staging (epilogue_lds_rows): rows of
// the whole workgroup tile, `row_bytes` each, written by the MFMA
// accumulator layout of block size `mf` with `esz`-byte elements and read
// back 16 bytes per lane.  One 16 x 16 accumulator write covers rows r, r + 4,
// r + 8 and r + 12 at 16 consecutive columns (16 * esz bytes); a 32 x 32 one
// rows r and r + 4 at 32 columns.  The chunk XOR ((row >> 2) & 3) * esz
// (16 x 16) or ((row >> 2) & 1) * 2 * esz (32 x 32) moves each of those row
// groups to its own bank range; it stays below 16, so it permutes the chunks
// inside each 256-byte piece of a row and whole-row reads stay conflict-free.
__host__ __device__ constexpr int epi_row_stage_offset(int row, int chunk, int row_bytes, int mf, int esz) {
  return row * row_bytes + 16 * (chunk ^ (mf == 16 ? ((row >> 2) & 3) * esz : ((row >> 2) & 1) * 2 * esz));
}

// ---------------------------------------------------------------- workgroup -> tile
//
// Workgroups are handed to the 8 XCDs round-robin (workgroup b on XCD b mod 8),
// and each XCD has its own L2.  The logical tile id gives each XCD one
// contiguous range of ids, then walks tiles in groups of `group_m` tile rows
// so the workgroups resident on one XCD at a time share A and B panels.
// LSM_XCD_REMAP=0 (an A/B build only) keeps the hardware order instead.
#ifndef LSM_XCD_REMAP
#define LSM_XCD_REMAP 1
#endif
__host__ __device__ constexpr int xcd_logical_id(int bid, int nwg) {
#if LSM_XCD_REMAP
  return (bid & 7) * (nwg >> 3) + ((bid & 7) < (nwg & 7) ? (bid & 7) : (nwg & 7)) + (bid >> 3);
#else
  (void)nwg;
  return bid;
#endif
}

__host__ __device__ inline void tile_coords(int lid, int tiles_m, int tiles_n, int group_m,
                                            int &tm, int &tn) {
  const int width = group_m * tiles_n;
  const int group = lid / width;
  const int first_m = group * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in = lid - group * width;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Operand bytes one XCD's workgroups touch over the whole K range, largest
// over the 8 XCDs: the distinct tile rows (A panels of `a_panel` bytes) plus
// the distinct tile columns (B panels of `b_panel` bytes) of that XCD's
// contiguous range of logical ids under tile_coords.  When this exceeds one
// XCD's L2, the panels cannot stay resident while the XCD's workgroups
// stream through K, and the loads come from further out.
__host__ __device__ inline long long xcd_max_panel_bytes(int tiles_m, int tiles_n, int group_m,
                                                         long long a_panel, long long b_panel) {
  const int nwg = tiles_m * tiles_n;
  const int width = group_m * tiles_n;              // logical ids per group of tile rows
  long long most = 0;
  for (int x = 0; x < 8; x++) {
    const int cnt = (nwg >> 3) + (x < (nwg & 7) ? 1 : 0);
    if (cnt == 0) continue;
    const int lo = x * (nwg >> 3) + (x < (nwg & 7) ? x : (nwg & 7));
    const int hi = lo + cnt;                         // this XCD's ids: [lo, hi)
    const int g0 = lo / width, g1 = (hi - 1) / width;
    int rows = 0, first_c0 = 0, last_c1 = 0;
    for (int g = g0; g <= g1; g++) {
      const int first_m = g * group_m;
      const int gm = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
      const int a = (lo > g * width ? lo : g * width) - g * width;     // [a, b) inside the group
      const int b = (hi < g * width + gm * tiles_n ? hi : g * width + gm * tiles_n) - g * width;
      const int c0 = a / gm, c1 = (b - 1) / gm;      // columns touched in this group
      if (c1 == c0)
        rows += b - a;
      else if (c1 == c0 + 1)                         // two partial columns
        rows += (gm - a % gm) + ((b - 1) % gm + 1) < gm ? (gm - a % gm) + ((b - 1) % gm + 1) : gm;
      else
        rows += gm;
      if (g == g0) first_c0 = c0;
      if (g == g1) last_c1 = c1;
    }
    // Columns: one group -> [first_c0, last_c1]; two -> the first group's tail
    // [first_c0, tiles_n) and the last group's head [0, last_c1]; more -> all.
    int cols;
    if (g1 == g0)
      cols = last_c1 - first_c0 + 1;
    else if (g1 == g0 + 1)
      cols = last_c1 + 1 >= first_c0 ? tiles_n : (last_c1 + 1) + (tiles_n - first_c0);
    else
      cols = tiles_n;
    const long long bytes = rows * a_panel + cols * b_panel;
    if (bytes > most) most = bytes;
  }
  return most;
}

}  // namespace lsm
