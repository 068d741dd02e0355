// Block -> tile maps of the grouped GEMMs, aware of the chip's 8 XCDs (each
// with its own L2): hardware hands out blocks to the XCDs round robin, so
// block b runs on XCD b % 8, and the tiles an XCD gets consecutively are the
// ones that share its L2.
#pragma once

#include "kernels.hpp"

namespace moe {

constexpr int NXCD = 8;
static_assert(NXCD == MT_SEGMENTS, "one tile-list segment per XCD");

// Tiles over the m-tile list (m-tiles x nb_n n-blocks).  Logical tile index
// of this block, or -1 if the block has no work.  XCD x (blocks bid with
// bid % 8 == x) takes the tiles of list segment x (whose first m-tiles the
// scan kernel stores in mtc[1..9]), or, when the segments do not fit the
// grid (mtc[1] < 0), an equal share of the tile list.
__device__ __forceinline__ int xcd_tile(const int32_t* mtc, int nb_n) {
  const int bid = blockIdx.x;
  const int xcd = bid % NXCD, j = bid / NXCD;
  if (mtc[1] < 0) {
    const int n_tiles = mtc[0] * nb_n;
    const int chunk = ceil_div(n_tiles, NXCD);
    if (j >= chunk) return -1;
    const int q = xcd * chunk + j;
    return q < n_tiles ? q : -1;
  }
  const int q = mtc[1 + xcd] * nb_n + j;
  return q < mtc[2 + xcd] * nb_n ? q : -1;
}

// Tile q -> (m-tile, n-block): within a unit of up to MT_UNIT m-tiles of one
// group, the m-tile index runs fastest, so the tiles that read the same weight
// block are dispatched back to back (onto the same XCD) and share its L2.
__device__ __forceinline__ void tile_coords(const int4* mtiles, int q, int nb_n, int& mt, int& nb, int& in_unit) {
  const int t = q / nb_n;
  const int w = mtiles[t].w;
  const int s = t - (w >> 8), k = w & 0xff;
  const int local = q - s * nb_n;
  nb = local / k;
  in_unit = local % k;
  mt = s + in_unit;
}

// Blocks of a grid over the m-tile list: NXCD x (tiles of the largest list
// segment the scan may form).
inline int mtile_grid(int max_mtiles, int nb_n) {
  return static_cast<int>(static_cast<long long>(NXCD) * seg_cap(max_mtiles) * nb_n);
}

}  // namespace moe
