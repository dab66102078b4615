// Launch order of a grouped GEMM tile launch on an 8-XCD MI355X (host side,
// plain C++, no HIP dependency so that it can be unit-tested on the CPU).
//
// The hardware dispatcher hands workgroup w to XCD (w mod 8), and each XCD has
// its own L2.  Tiles that share operand slices must therefore sit at positions
// of the same residue to share an L2.  The tiles of a launch are cut into
// units -- runs of consecutive tiles of one matrix, ordered so that tiles
// running together share operand row blocks -- the units are assigned longest
// first to the least-loaded XCD stream (the greedy the MatrixFSDP owner planner
// uses for roles, section 4.1 Algorithm 1), and the streams are interleaved:
// position 8k + x holds the k-th tile of stream x.  Streams shorter than the
// longest are padded with idle entries (mat = -1), which the kernels skip.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <vector>

namespace matopt {

// tj < 0: a diagonal pair, the diagonal tiles of block rows ti and -tj-1
struct TileRef {
  int32_t mat, ti, tj, pad_;
};

struct TileUnit {
  std::vector<TileRef> tiles;
  int64_t cost = 0;     // sum over tiles of the K extent (diagonal tiles scaled)
  int32_t mat = 0, seq = 0;
};

constexpr int kXcds = 8;
constexpr int kUnitTiles = 64;

// Symmetric-output stage (Gram or polynomial): tiles ti <= tj of a tm x tm
// block grid, row-major, cut into units of at most kUnitTiles.  A diagonal
// tile costs diag16/16 of an off-diagonal one (9/16 where the kernel computes
// only its upper 36 of 64 blocks).  With pair_diag the diagonal tiles of block
// rows 2p and 2p+1 form one entry {mat, 2p, -(2p+1)-1} (a diagonal pair, in
// place of tile (2p, 2p)); a last diagonal tile stays alone when tm is odd.
inline void units_triangle(int mat, int tm, int64_t k_extent, std::vector<TileUnit>& out,
                           int diag16 = 16, bool pair_diag = false) {
  TileUnit u;
  u.mat = mat;
  int seq = 0;
  const int64_t kd = k_extent * diag16 / 16;
  for (int ti = 0; ti < tm; ++ti)
    for (int tj = ti; tj < tm; ++tj) {
      if (ti == tj && pair_diag && ti % 2 == 1) continue;   // in the pair of ti-1
      if (ti == tj && pair_diag && ti + 1 < tm) {
        u.tiles.push_back({mat, ti, -(ti + 1) - 1, 0});
        u.cost += 2 * kd;
      } else {
        u.tiles.push_back({mat, ti, tj, 0});
        u.cost += ti == tj ? kd : k_extent;
      }
      if ((int)u.tiles.size() == kUnitTiles) {
        u.seq = seq++;
        out.push_back(u);
        u.tiles.clear();
        u.cost = 0;
      }
    }
  if (!u.tiles.empty()) {
    u.seq = seq;
    out.push_back(u);
  }
}

// Full-output stage (apply): tm x tn grid, column-major (all row blocks of a
// column block together: they share that column's operand slices, and
// consecutive columns share the row operand), cut into units of whole columns
// of about kUnitTiles tiles.
inline void units_full(int mat, int tm, int tn, int64_t k_extent, std::vector<TileUnit>& out) {
  const int cols_per_unit = std::max(1, kUnitTiles / std::max(1, tm));
  int seq = 0;
  for (int c0 = 0; c0 < tn; c0 += cols_per_unit) {
    TileUnit u;
    u.mat = mat;
    u.seq = seq++;
    for (int tj = c0; tj < std::min(tn, c0 + cols_per_unit); ++tj)
      for (int ti = 0; ti < tm; ++ti) {
        u.tiles.push_back({mat, ti, tj, 0});
        u.cost += k_extent;
      }
    out.push_back(u);
  }
}

// Interleaved launch table (size = nxcd * longest stream).
inline std::vector<TileRef> xcd_schedule(std::vector<TileUnit> units, int nxcd = kXcds) {
  std::stable_sort(units.begin(), units.end(), [](const TileUnit& a, const TileUnit& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    if (a.mat != b.mat) return a.mat < b.mat;
    return a.seq < b.seq;
  });
  std::vector<std::vector<TileRef>> stream(nxcd);
  std::vector<int64_t> load(nxcd, 0);
  for (const TileUnit& u : units) {
    int best = 0;
    for (int x = 1; x < nxcd; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += u.cost;
    stream[best].insert(stream[best].end(), u.tiles.begin(), u.tiles.end());
  }
  size_t longest = 0;
  for (const auto& s : stream) longest = std::max(longest, s.size());
  std::vector<TileRef> table(longest * nxcd, TileRef{-1, 0, 0, 0});
  for (int x = 0; x < nxcd; ++x)
    for (size_t k = 0; k < stream[x].size(); ++k) table[k * nxcd + x] = stream[x][k];
  return table;
}

}  // namespace matopt
