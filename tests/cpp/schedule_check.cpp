// Host check of the grouped-launch tile schedule (tile_schedule.hpp).
// Reads "tm tn k_gram k_poly" lines (one matrix each; the apply K equals the
// polynomial's) from stdin and checks, for the Gram and polynomial (triangle)
// and apply (full) tables:
//   * every tile (ti <= tj, resp. every ti, tj) appears exactly once,
//   * all tiles of one unit sit at positions of the same residue mod 8,
//   * the largest XCD load exceeds the mean by at most one unit's cost.
// Prints "ok <gram> <poly> <apply table sizes>" or the first violation; exit
// status 0 iff ok.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "tile_schedule.hpp"

using namespace matopt;

static int check(const std::vector<TileUnit>& units, const std::vector<TileRef>& table,
                 const char* what) {
  // a diagonal pair (tj < 0) stands for tiles (ti, ti) and (-tj-1, -tj-1)
  auto keys = [](const TileRef& t) {
    std::vector<std::tuple<int, int, int>> k;
    if (t.tj < 0) {
      k.push_back(std::make_tuple(t.mat, t.ti, t.ti));
      k.push_back(std::make_tuple(t.mat, -t.tj - 1, -t.tj - 1));
    } else {
      k.push_back(std::make_tuple(t.mat, t.ti, t.tj));
    }
    return k;
  };
  std::map<std::tuple<int, int, int>, int> pos;
  for (size_t p = 0; p < table.size(); ++p) {
    const TileRef& t = table[p];
    if (t.mat < 0) continue;
    for (const auto& key : keys(t)) {
      if (pos.count(key)) { std::printf("%s: duplicate tile\n", what); return 1; }
      pos[key] = (int)p;
    }
  }
  size_t n = 0;
  int64_t total = 0, maxunit = 0;
  std::vector<int64_t> load(kXcds, 0);
  for (const TileUnit& u : units) {
    total += u.cost;
    maxunit = std::max(maxunit, u.cost);
    std::set<int> res;
    for (const TileRef& t : u.tiles) {
      for (const auto& key : keys(t)) {
        ++n;
        auto it = pos.find(key);
        if (it == pos.end()) { std::printf("%s: missing tile\n", what); return 1; }
        res.insert(it->second % kXcds);
      }
    }
    if (res.size() != 1) { std::printf("%s: unit split across XCDs\n", what); return 1; }
    load[*res.begin()] += u.cost;
  }
  if (n != pos.size()) { std::printf("%s: tile count mismatch\n", what); return 1; }
  if (table.size() % kXcds) { std::printf("%s: table not a multiple of 8\n", what); return 1; }
  int64_t mx = 0;
  for (int64_t l : load) mx = std::max(mx, l);
  if (mx * kXcds > total + (int64_t)kXcds * maxunit) {
    std::printf("%s: imbalance max %lld mean %lld unit %lld\n", what, (long long)mx,
                (long long)(total / kXcds), (long long)maxunit);
    return 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  // optional arguments: cost of a diagonal tile in 16ths (9 for bf16, 16 for
  // fp32); 1 to pair the diagonal tiles (bf16)
  const int diag16 = argc > 1 ? std::atoi(argv[1]) : 16;
  const bool pairs = argc > 2 && std::atoi(argv[2]) != 0;
  std::vector<TileUnit> gram, poly, full;
  int tm, tn;
  long long kg, kp;
  int mat = 0;
  while (std::scanf("%d %d %lld %lld", &tm, &tn, &kg, &kp) == 4) {
    units_triangle(mat, tm, kg, gram, diag16, pairs);
    units_triangle(mat, tm, kp, poly, diag16, pairs);
    units_full(mat, tm, tn, kp, full);
    ++mat;
  }
  const auto t1 = xcd_schedule(gram), t2 = xcd_schedule(poly), t3 = xcd_schedule(full);
  if (check(gram, t1, "gram") || check(poly, t2, "poly") || check(full, t3, "full")) return 1;
  std::printf("ok %zu %zu %zu\n", t1.size(), t2.size(), t3.size());
  return 0;
}
