// Tile orders of the int8 digit GEMM (digitgemm.hip), as plain functions so
// that the host side (and a host-only test) can check them.
#pragma once

#if defined(__HIPCC__)
#define MPQ_TILE_HD __host__ __device__
#else
#define MPQ_TILE_HD
#endif

namespace mpq {

constexpr int DG_GROUP_M = 8;   // tile rows per group of the tile order

// Lower-triangle tile order (tc <= tr, square M = N): the groups of
// DG_GROUP_M tile rows column by column, but each column of a group starts at
// the diagonal and the columns end at the group's last row, so only tiles
// that touch the lower triangle are enumerated and the contiguous runs of the
// XCDs carry equal work.  Tiles of group q before it: GM^2 q (q - 1) / 2 +
// q GM (GM + 1) / 2.
MPQ_TILE_HD inline int dg_lower_before(int q) {
  return DG_GROUP_M * DG_GROUP_M * q * (q - 1) / 2 + q * DG_GROUP_M * (DG_GROUP_M + 1) / 2;
}
MPQ_TILE_HD inline int dg_lower_tiles(int tm) {
  const int full = tm / DG_GROUP_M, gm = tm - full * DG_GROUP_M;
  return dg_lower_before(full) + full * DG_GROUP_M * gm + gm * (gm + 1) / 2;
}
// Tile t (0 <= t < dg_lower_tiles(tm)) of the order: tile row tr, tile column tc <= tr.
MPQ_TILE_HD inline void dg_lower_tile(int t, int tm, int& tr, int& tc) {
  int q = 0;
  while ((q + 1) * DG_GROUP_M < tm && dg_lower_before(q + 1) <= t) ++q;
  const int first = q * DG_GROUP_M, gm = tm - first < DG_GROUP_M ? tm - first : DG_GROUP_M;
  int l = t - dg_lower_before(q);
  if (l < first * gm) {   // columns left of the group's diagonal block: gm tiles each
    tc = l / gm;
    tr = first + l % gm;
    return;
  }
  l -= first * gm;   // diagonal block: column first + u holds gm - u tiles
  int u = 0;
  while (l >= gm - u) {
    l -= gm - u;
    ++u;
  }
  tc = first + u;
  tr = first + u + l;
}

}  // namespace mpq
