// Tile scheduling shared by the tile GEMM kernels (plain and grouped).
#pragma once

#include "common.hpp"

namespace w4a16 {

// Linear workgroup id -> (m-tile, n-tile). Workgroup ids are first remapped
// so that each XCD owns a contiguous run of tiles, then tiles are ordered in
// bands of GROUP_M = 8 m-tiles, column by column ("Add Triton BF16xINT4
// rowwise GEMM for ROCm gfx942/gfx950", Implementation: XCD remapping and
// GROUP_SIZE_M grouping): neighbouring workgroups share weight columns and
// activation rows in one L2.
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int MT, int NT, int* mt, int* nt) {
  constexpr int GM = 8;
  const int lid = xcd_remap(bid, nblocks);
  const int per_group = GM * NT;
  const int grp = lid / per_group;
  const int first_m = grp * GM;
  const int gsz = min(MT - first_m, GM);
  *mt = first_m + (lid % per_group) % gsz;
  *nt = (lid % per_group) / gsz;
}

// Rows of linear m-tile `mt` (BM rows each). Plain: one weight group of
// M_total rows. Grouped ("Native fused grouped kernel" on the MI350X Triton
// page): the m-tiles of group g follow those of groups < g; each group's
// size is clamped to [0, M_total - start). rows <= 0 means no work.
struct TileRows {
  int wg, row0, rows;
};
// Batched (m_uniform > 0, no M_sizes): G weight groups of m_uniform rows
// each, ceil(m_uniform / BM) m-tiles per group, all computed from the tile id.
__device__ __forceinline__ TileRows tile_rows(int mt, int BM, int M_total, const int32_t* m_sizes, int G,
                                              int m_uniform) {
  TileRows t{0, mt * BM, min(BM, M_total - mt * BM)};
  if (m_uniform > 0) {
    const int tpg = (m_uniform + BM - 1) / BM;
    const int g = mt / tpg, r = (mt - g * tpg) * BM;
    t.wg = g;
    t.row0 = g * m_uniform + r;
    t.rows = g < G ? min(BM, m_uniform - r) : 0;
    return t;
  }
  if (m_sizes == nullptr) return t;
  int cnt = 0, start = 0;
  bool found = false;
  for (int gg = 0; gg < G; ++gg) {
    int ms = m_sizes[gg];
    ms = ms < 0 ? 0 : ms;
    ms = start >= M_total ? 0 : min(ms, M_total - start);
    const int tiles = (ms + BM - 1) / BM;
    if (!found && mt < cnt + tiles) {
      t.wg = gg;
      t.row0 = start + (mt - cnt) * BM;
      t.rows = min(BM, start + ms - t.row0);
      found = true;
    }
    cnt += tiles;
    start += ms;
  }
  if (!found) t.rows = 0;
  // the walk reads m_sizes with vector loads; the results are the same in
  // every lane, and saying so keeps the buffer descriptors built from them in
  // scalar registers (otherwise every buffer access becomes a waterfall loop)
  t.wg = __builtin_amdgcn_readfirstlane(t.wg);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.rows = __builtin_amdgcn_readfirstlane(t.rows);
  return t;
}

// Grouped: the m-tiles that hold rows, sum over groups of ceil(m_g / BM)
// (same clamping as tile_rows). The grid is sized on the host from the bound
// ceil(M_total / BM) + G per column; mapping only the real tiles, spread
// evenly over the XCDs, keeps the empty ones from taking a share of one XCD
// that its 32 compute units then lack for real tiles.
__device__ __forceinline__ int real_mtiles(int BM, int M_total, const int32_t* m_sizes, int G) {
  int cnt = 0, start = 0;
  for (int gg = 0; gg < G; ++gg) {
    int ms = m_sizes[gg];
    ms = ms < 0 ? 0 : ms;
    ms = start >= M_total ? 0 : min(ms, M_total - start);
    cnt += (ms + BM - 1) / BM;
    start += ms;
  }
  return __builtin_amdgcn_readfirstlane(cnt);
}

}  // namespace w4a16
