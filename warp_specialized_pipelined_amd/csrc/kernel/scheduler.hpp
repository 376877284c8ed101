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
// and each XCD has its own L2.  Renumber so that the workgroups resident on
// one XCD take consecutive logical slots: at every step they then work on
// neighbouring tiles of one raster group and share A and B panels in that
// XCD's L2.  With G = 8q + r workgroups, XCD x holds q + (x < r) of them
// (ids x, x + 8, ...), and its slots start after those of XCDs 0 .. x-1.
__device__ __forceinline__ int persistent_slot(int bid, int grid) {
  const int q = grid / 8, r = grid % 8, x = bid % 8;
  return x * q + min(x, r) + bid / 8;
}

struct TileCoord {
  int tm, tn;
  int l;  // batch
};

// Logical tile index -> (tile row, tile column, batch).  Batches come one
// after another.  Inside one, tiles are taken in groups of `group_m` tile
// rows, running down the columns inside a group, so that consecutive indices
// share the B panel and nearby ones share A panels.
__device__ __forceinline__ TileCoord tile_of(int L, const KernelArgs& a) {
  const int l = L / a.tiles_per_batch;
  L -= l * a.tiles_per_batch;
  const int per_group = a.group_m * a.tiles_n;
  const int g = L / per_group;
  const int first_m = g * a.group_m;
  const int rows = min(a.tiles_m - first_m, a.group_m);
  const int r = L - g * per_group;
  return {first_m + r % rows, r / rows, l};
}

// The arguments as batch l sees them: every operand pointer moved to its
// matrix of that batch, so the K loop and the epilogue work on one product.
__device__ __forceinline__ KernelArgs batch_args(const KernelArgs& a, int l) {
  KernelArgs b = a;
  b.A = static_cast<const unsigned char*>(a.A) + l * a.a_bs_bytes;
  b.B = static_cast<const unsigned char*>(a.B) + l * a.b_bs_bytes;
  if (a.C) b.C = static_cast<const unsigned char*>(a.C) + l * a.c_bs_bytes;
  b.D = static_cast<unsigned char*>(a.D) + l * a.d_bs_bytes;
  if (a.D_copy) b.D_copy = static_cast<unsigned char*>(a.D_copy) + l * a.d_bs_bytes;
  return b;
}

// Stream-K.  With fewer tiles left than would fill the grid evenly, whole
// tiles leave compute units idle in the last round (192 tiles on 256 CUs
// keep 64 idle).  The CUTLASS stream-K scheduler the kernel page selects
// cuts such tiles into K-stage units instead; here the units of tiles
// [sk_first, num_tiles), tile after tile, K stage after K stage, are cut
// into G contiguous ranges, workgroup slot w taking [U w / G, U (w+1) / G).
// A range covers at most two partial tiles (where it starts and where it
// ends) and any number of whole ones in between.
__device__ __forceinline__ int64_t sk_units(const KernelArgs& a) {
  return (int64_t)(a.num_tiles - a.sk_first) * a.sk_kt;
}
__device__ __forceinline__ int64_t sk_begin(int64_t U, int w, int G) { return U * w / G; }
// The slot whose range holds unit u (the last w with U w / G <= u).
__device__ __forceinline__ int sk_owner(int64_t U, int64_t u, int G) {
  return (int)(((u + 1) * G + U - 1) / U) - 1;
}

}  // namespace migemm
