// scheduler.hpp -- persistent static tile scheduler.
//
// The CUTLASS SM90 cooperative kernel runs one persistent CTA per SM; each
// asks its tile scheduler for an initial work tile and then for the next one
// until the tile is no longer valid, and the grid is sized from the SM count
// with a raster order and swizzle (kernel page: get_grid_shape, and the
// scheduler fetch loop of the producer and consumer warp groups).  Here one
// workgroup runs per compute unit and walks the tiles w', w'+G, w'+2G, ...
// of a grouped raster order, where G is the grid size.
#pragma once

#include "params.hpp"

namespace migemm {

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// and each XCD has its own L2.  Renumber so that the G/8 workgroups resident
// on one XCD take G/8 consecutive logical slots: at every step they then
// work on neighbouring tiles of one raster group and share A and B panels in
// that XCD's L2.
__device__ __forceinline__ int persistent_slot(int bid, int grid) {
  if (grid % 8 != 0) return bid;
  return (bid % 8) * (grid / 8) + bid / 8;
}

struct TileCoord {
  int tm, tn;
};

// Logical tile index -> (tile row, tile column).  Tiles are taken in groups
// of `group_m` tile rows; inside a group they run down the columns, so that
// consecutive indices share the B panel and nearby ones share A panels.
__device__ __forceinline__ TileCoord tile_of(int L, const KernelArgs& a) {
  const int per_group = a.group_m * a.tiles_n;
  const int g = L / per_group;
  const int first_m = g * a.group_m;
  const int rows = min(a.tiles_m - first_m, a.group_m);
  const int r = L - g * per_group;
  return {first_m + r % rows, r / rows};
}

}  // namespace migemm
