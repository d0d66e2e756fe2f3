// layout_probe.cpp -- host-callable views of the LDS address functions of
// lds_layout.h, built host-only into a small shared library so that the
// bank-conflict model in the tests evaluates exactly the addresses the
// kernels use.  Nothing here runs on the GPU.
#include "lds_layout.h"
#include "gemm_common.h"

extern "C" {
int lsm_layout_swizzled() { return LSM_LDS_SWIZZLE; }
int lsm_kc_chunk_offset(int row, int chunk, int row_bytes) {
  return lsm::kc_chunk_offset(row, chunk, row_bytes);
}
int lsm_mn_chunk_offset(int k, int chunk, int row_bytes) {
  return lsm::mn_chunk_offset(k, chunk, row_bytes);
}
int lsm_loader_lds_offset(int id, int row_bytes, int k_contig) {
  return lsm::loader_lds_offset(id, row_bytes, k_contig != 0);
}
int lsm_frag_kc_offset(int lane, int base, int kk, int row_bytes) {
  return lsm::frag_kc_offset(lane, base, kk, row_bytes);
}
int lsm_frag_tr_offset(int lane, int base, int kk, int h, int row_bytes) {
  return lsm::frag_tr_offset(lane, base, kk, h, row_bytes);
}
int lsm_frag16_kc_offset(int lane, int base, int kk, int row_bytes) {
  return lsm::frag16_kc_offset(lane, base, kk, row_bytes);
}
int lsm_frag16_tr_offset(int lane, int base, int kk, int h, int row_bytes) {
  return lsm::frag16_tr_offset(lane, base, kk, h, row_bytes);
}
int lsm_mn16_swizzle(int k, int row_bytes) { return lsm::mn16_swizzle(k, row_bytes); }
int lsm_mn16_chunk_offset(int k, int chunk, int row_bytes) {
  return lsm::mn16_chunk_offset(k, chunk, row_bytes);
}
int lsm_loader_lds_offset16(int id, int row_bytes) { return lsm::loader_lds_offset16(id, row_bytes); }
int lsm_frag16_tr_lane(int lane, int row_bytes) { return lsm::frag16_tr_lane(lane, row_bytes); }
int lsm_epi_stage_offset(int row, int chunk, int row_bytes, int mf) {
  return lsm::epi_stage_offset(row, chunk, row_bytes, mf);
}
int lsm_mn_chunk_offset8(int k, int chunk, int row_bytes) {
  return lsm::mn_chunk_offset(k, chunk, row_bytes, 1);
}
int lsm_loader_lds_offset8(int id, int row_bytes, int k_contig) {
  return lsm::loader_lds_offset(id, row_bytes, k_contig != 0, 1);
}
int lsm_frag_kc8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return lsm::frag_kc8_offset(lane, base, kk, q, row_bytes);
}
int lsm_frag_tr8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return lsm::frag_tr8_offset(lane, base, kk, q, row_bytes);
}
int lsm_mn16_swizzle8(int k, int row_bytes) { return lsm::mn16_swizzle8(k, row_bytes); }
int lsm_epi_row_stage_offset(int row, int chunk, int row_bytes, int mf, int esz) {
  return lsm::epi_row_stage_offset(row, chunk, row_bytes, mf, esz);
}
int lsm_mn16_chunk_offset8(int k, int chunk, int row_bytes) {
  return lsm::mn16_chunk_offset(k, chunk, row_bytes, 1);
}
int lsm_loader_lds_offset16_8(int id, int row_bytes) { return lsm::loader_lds_offset16(id, row_bytes, 1); }
int lsm_frag16_kc8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return lsm::frag16_kc8_offset(lane, base, kk, q, row_bytes);
}
int lsm_frag16_tr8_offset(int lane, int base, int kk, int q, int row_bytes) {
  return lsm::frag16_tr8_offset(lane, base, kk, q, row_bytes);
}
// The ping-pong kernel's MN-contiguous operand tiles in the 16 x 16 layouts
// (256 wide, BK 64 for 16-bit and 128 for 8-bit elements, 256 loader
// threads): the loader's round step, swizzle and choice of lane offset.
using PP16 = lsm::OperandTile<256, 64, lsm::MNC, 256, 2, 1>;
using PP8 = lsm::OperandTile<256, 128, lsm::MNC, 256, 1, 1>;
int lsm_pp_mn_row_step(int es) { return es == 2 ? PP16::ROW_STEP : PP8::ROW_STEP; }
int lsm_pp_mn_loads(int es) { return es == 2 ? PP16::LOADS : PP8::LOADS; }
int lsm_pp_mn_lane_offsets(int es) { return es == 2 ? PP16::LANE_OFFSETS : PP8::LANE_OFFSETS; }
int lsm_pp_mn_phase_rows(int es) { return es == 2 ? PP16::PHASE_ROWS : PP8::PHASE_ROWS; }
int lsm_pp_mn_round_phase(int es, int d) { return es == 2 ? PP16::round_phase(d) : PP8::round_phase(d); }
int lsm_pp_mn_swizzle(int es, int row) { return es == 2 ? PP16::swizzle(row) : PP8::swizzle(row); }
int lsm_xcd_logical_id(int bid, int nwg) { return lsm::xcd_logical_id(bid, nwg); }
void lsm_tile_coords(int lid, int tiles_m, int tiles_n, int group_m, int *tm, int *tn) {
  lsm::tile_coords(lid, tiles_m, tiles_n, group_m, *tm, *tn);
}
long long lsm_xcd_max_panel_bytes(int tiles_m, int tiles_n, int group_m, long long a_panel,
                                  long long b_panel) {
  return lsm::xcd_max_panel_bytes(tiles_m, tiles_n, group_m, a_panel, b_panel);
}
}
