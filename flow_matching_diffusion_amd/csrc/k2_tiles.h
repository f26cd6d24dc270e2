// Tile order of the GEMM kernels (host and device; the CPU tests compile it with a host compiler).
#pragma once

#include <stddef.h>

namespace k2 {

// Workgroup bid (of nb = tiles_m * tiles_n) -> output tile (tm, tn).
//
// The hardware hands workgroups to the 8 XCDs round-robin (XCD = bid % 8, in bid order), and each
// XCD has its own L2. Tiles are walked in super-columns of scn N-tiles, one after another, so the
// weight rows in use at any time (scn * BN rows) stay within the last-level cache that all XCDs
// share. Within a super-column each XCD takes a contiguous range of a raster that runs down GM
// M-tiles before stepping to the next N-tile, so the tiles one XCD runs together share A and B
// rows in its L2. A super-column of T tiles gives each XCD T/8 tiles; its T%8 remaining tiles go
// to the XCDs that follow the previous super-column's, so every XCD's count matches the
// round-robin hand-out and the map is a bijection.
constexpr int kTileGroupM = 8;

__host__ __device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int scn, int& tm, int& tn) {
  const int xcd = bid & 7;
  int loc = bid >> 3;             // position in this XCD's own sequence
  int n_base = 0, off = 0;        // first N-tile of the super-column; XCD of its first remainder
  int w = scn < tiles_n ? scn : tiles_n;
  for (;;) {
    const int T = tiles_m * w, e = T & 7;
    const bool extra = ((xcd - off) & 7) < e;
    const int c = (T >> 3) + (extra ? 1 : 0);
    if (loc < c || n_base + w >= tiles_n) {
      // XCDs before this one in index order that received a remainder tile of this super-column
      int before;
      if (off + e <= 8) {
        before = xcd - off < 0 ? 0 : (xcd - off > e ? e : xcd - off);
      } else {
        const int wrap = off + e - 8;  // remainder tiles at XCDs 0 .. wrap-1 and off .. 7
        before = (xcd < wrap ? xcd : wrap) + (xcd > off ? xcd - off : 0);
      }
      const int lid = xcd * (T >> 3) + before + loc;
      const int GM = kTileGroupM;
      const int group = lid / (GM * w), first_m = group * GM;
      const int gm = tiles_m - first_m < GM ? tiles_m - first_m : GM;
      const int r = lid - group * GM * w;
      tm = first_m + r % gm;
      tn = n_base + r / gm;
      return;
    }
    loc -= c;
    off = (off + e) & 7;
    n_base += w;
    w = scn < tiles_n - n_base ? scn : tiles_n - n_base;
  }
}

// Workgroup bid (of total) -> work item, such that each XCD (bid % 8) takes one contiguous range of
// items, in order: XCD x gets total / 8 items (one more for x < total % 8) starting at
// x * (total / 8) + min(x, total % 8). A bijection on [0, total). Items next to each other in the
// caller's order (e.g. query blocks of one attention head) then run together on one XCD and share
// its L2, instead of being dealt across all eight.
__host__ __device__ inline int xcd_item(int bid, int total) {
  const int x = bid & 7, s = bid >> 3, q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + s;
}

// The same for items in B consecutive groups of per_b (one group per batch row, whose items can
// cost different amounts from one group to the next): when per_b is a multiple of 8, XCD x takes
// items [x per_b / 8, (x + 1) per_b / 8) of every group, one group after the other, so that every
// XCD gets the same share of each group's work while its neighbouring slots still share one group's
// data; otherwise xcd_item over all B per_b items. A bijection on [0, B per_b).
__host__ __device__ inline int xcd_item_rows(int bid, int per_b, int B) {
  if (per_b & 7) return xcd_item(bid, per_b * B);
  const int x = bid & 7, s = bid >> 3, cnt = per_b >> 3;
  return (s / cnt) * per_b + x * cnt + s % cnt;
}

// N-tiles per super-column: about kSuperColumnBytes of weight rows, in equal super-columns.
constexpr size_t kSuperColumnBytes = size_t(96) << 20;
inline int super_cols(int tiles_n, int BN, int K, int elem) {
  const size_t per_tile = (size_t)BN * K * elem;
  int maxw = (int)(kSuperColumnBytes / (per_tile ? per_tile : 1));
  if (maxw < 1) maxw = 1;
  const int nsc = (tiles_n + maxw - 1) / maxw;
  return (tiles_n + nsc - 1) / nsc;
}

}  // namespace k2
