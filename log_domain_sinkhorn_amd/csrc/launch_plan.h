// Launch-size arithmetic of the pair kernels, free of HIP so that the host
// tests can compile and check it with a plain C++ compiler.
//
// One dispatch covers at most 2^32 - 1 work-items per grid dimension (the
// dispatch packet stores the grid size in work-items as a 32-bit number), so
// a 1-D launch of `threads` work-items per workgroup may hold at most
// (2^32 - 1) / threads workgroups.
#pragma once

#include <cstdint>

namespace sk {

constexpr int64_t kMaxDispatchItems = (int64_t(1) << 32) - 1;

constexpr int64_t max_blocks_1d(int64_t threads) { return kMaxDispatchItems / threads; }

constexpr bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= max_blocks_1d(threads);
}

// Column split of the dense VALU pair kernel for nrows x ncols pairs: tiles
// of `rows_per_tile` rows, chunks of `chunk` columns, G workgroups of
// `threads` work-items (`waves` waves) per tile, G a power of two.
struct DenseSplit {
  int32_t G = 1;
  int32_t glog = 0;
  int64_t cps = 0;      // chunks per split
  int64_t nchunks = 0;  // column chunks
  int64_t tiles = 0;    // row tiles
  bool ok = false;      // false: the tiles alone exceed one dispatch
};

// `slots`: workgroups resident on the whole chip at once; `l2_bytes`: column
// bytes one XCD's L2 keeps comfortably; `xcds`: XCD count.
//   * at least 4 chunks per wave (1 when the tiles are too few to fill the
//     chip even so), at most `max_split` splits;
//   * the workgroups run in rounds of `slots` and finish unevenly, so aim at
//     three rounds or more for the load to even out;
//   * workgroups are dealt to the XCDs in turn, so with G a multiple of
//     `xcds` each XCD streams its own column splits: preferred whenever the
//     column data would not fit an XCD's L2 whole, or G reaches it anyway;
//   * tiles * G workgroups must fit one dispatch: G is halved until they do.
inline DenseSplit plan_dense_split(int64_t nrows, int64_t ncols, int64_t slots, int d,
                                   int64_t chunk, int64_t rows_per_tile, int64_t waves,
                                   int64_t threads, int64_t max_split, int64_t xcds,
                                   int64_t l2_bytes) {
  DenseSplit s;
  s.nchunks = (ncols + chunk - 1) / chunk;
  s.tiles = (nrows + rows_per_tile - 1) / rows_per_tile;
  int64_t maxsplit = s.nchunks / (4 * waves);
  if (s.tiles * (maxsplit > 1 ? maxsplit : 1) < slots) maxsplit = s.nchunks / waves;
  if (maxsplit > max_split) maxsplit = max_split;
  if (maxsplit < 1) maxsplit = 1;
  const int64_t want = (3 * slots + s.tiles - 1) / (s.tiles > 0 ? s.tiles : 1);
  const bool big = s.nchunks * chunk * (int64_t)(d + 1) * 4 > l2_bytes;
  int64_t G = 1;
  while (2 * G <= maxsplit && G < want) G *= 2;
  if (big && G < xcds && xcds <= maxsplit) G = xcds;
  while (G > 1 && !grid_fits(s.tiles * G, threads)) G /= 2;
  s.ok = grid_fits(s.tiles * G, threads);
  int32_t lg = 0;
  while ((int64_t(1) << lg) < G) ++lg;
  s.G = (int32_t)G;
  s.glog = lg;
  s.cps = (s.nchunks + G - 1) / G;
  return s;
}

}  // namespace sk
