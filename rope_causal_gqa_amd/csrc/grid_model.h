// Host-side cost model that picks the prefill grid for query counts too small
// for 512 workgroups of 4 waves (plain C++, no HIP: the CPU tests compile it).
//
// Two grids run one 8-wave workgroup per CU:
//   A: 128-row query tiles, keys split over two groups of 4 waves, 64-key K/V tiles;
//   B: 64-row query tiles, keys split over four groups of 2 waves, 32-key K/V
//      tiles, causal tiles paired heavy + light when that keeps 256 workgroups.
// B cuts the work finer; A moves half the K/V tile traffic per flop, runs
// 64-key steps and sets up one query tile per workgroup.  A workgroup's time
// is modelled as a set-up cost per query tile plus its (query row, key) pairs
// over a rate, both fitted to MI355X timings of the two kernels (A: 3.1 us +
// pairs / 7.3e3 per us; B: 7.5 us per tile + pairs / 6.1e3 per us), and B is
// taken when it is estimated to finish first.  Rows see keys by the causal
// and window rules; a cache is taken as full (max_kv keys per sequence).
#pragma once
#include <algorithm>
#include <functional>
#include <vector>

namespace rcgqa {
namespace grid {

constexpr int kCUs = 256;  // compute units of a gfx950 MI355X (8 XCDs of 32)

// sum over query rows i in [a, b) of min(max(i + c, 0), cap): the keys those
// rows see when row i sees keys up to i + c - 1, at most cap of them
inline double rows_keys(long long a, long long b, long long c, long long cap) {
  const long long z = std::min(std::max(a, 1 - c), b);    // first row that sees a key
  const long long u = std::min(std::max(z, cap - c), b);  // first row that sees cap keys
  return 0.5 * (double)(u - z) * (double)(z + c + u - 1 + c) + (double)(b - u) * (double)cap;
}

// Finish time of the busiest CU for a grid of bh * w.size() workgroups (work
// item i = head i / w.size(), slot i % w.size(), taking time w[slot]) that
// run one per CU: each XCD takes its share of the work list (the prefill
// kernel's work mapping: a contiguous eighth of the list when the grid is a
// multiple of 8, else every 8th item) in order and hands every item to
// whichever of its CUs frees first.
inline double busiest_cu(const std::vector<double>& w, long long bh) {
  const long long n = bh * (long long)w.size();
  double worst = 0;
  std::vector<double> load(kCUs / 8);
  for (int x = 0; x < 8; x++) {
    std::fill(load.begin(), load.end(), 0.0);  // a min-heap of this XCD's CU loads
    auto take = [&](long long item) {
      std::pop_heap(load.begin(), load.end(), std::greater<double>());
      load.back() += w[item % (long long)w.size()];
      std::push_heap(load.begin(), load.end(), std::greater<double>());
    };
    if (n % 8 == 0)
      for (long long i = x * (n / 8); i < (x + 1) * (n / 8); i++) take(i);
    else
      for (long long i = x; i < n; i += 8) take(i);
    worst = std::max(worst, *std::max_element(load.begin(), load.end()));
  }
  return worst;
}

struct KeyGroupGrid {
  bool four;   // B (four key groups over 64-row tiles), else A
  int npairs;  // work slots per (batch, head): query tiles, or heavy + light pairs
};

// bh = B * Hq; nk = keys per sequence (Sq without a cache, max_kv with one);
// window = 0 or the causal sliding window.
inline KeyGroupGrid key_group_grid(long long bh, int Sq, bool causal, long long nk, int window) {
  constexpr double kSetupA = 3.1, kRateA = 7.3e3, kSetupB = 7.5, kRateB = 6.1e3;
  const int nqt4 = (Sq + 127) / 128, nqt2 = (Sq + 63) / 64;
  const int npairs2 = causal && nqt2 > 1 && bh * ((nqt2 + 1) / 2) >= 256 ? (nqt2 + 1) / 2 : nqt2;
  const long long c = causal ? nk - Sq + 1 : nk, cap = window > 0 ? std::min<long long>(window, nk) : nk;
  // heavy (late) tiles first, as the kernel orders them
  std::vector<double> wa(nqt4), wb(npairs2);
  for (int t = 0; t < nqt4; t++) {
    const int qt = causal ? nqt4 - 1 - t : t;
    wa[t] = kSetupA + rows_keys(128LL * qt, std::min(128LL * qt + 128, (long long)Sq), c, cap) / kRateA;
  }
  auto w2 = [&](int qt) {
    return kSetupB + rows_keys(64LL * qt, std::min(64LL * qt + 64, (long long)Sq), c, cap) / kRateB;
  };
  for (int p = 0; p < npairs2; p++) {
    const int qt = causal ? nqt2 - 1 - p : p;
    wb[p] = w2(qt) + (npairs2 < nqt2 && p != qt ? w2(p) : 0.0);
  }
  const bool four = busiest_cu(wb, bh) < busiest_cu(wa, bh);
  return {four, four ? npairs2 : nqt4};
}

// Stream-K plan for small causal grids.  A unit is one (query tile of BM
// rows, 64-key tile) step of the causal work.  Units are listed (batch, head)
// by (batch, head); within one, query tiles in heavy / light pairs (the last
// tile, the first, the second last, the second, ...), and within a tile key
// tile by key tile.  Each workgroup takes a contiguous range of the list.  A
// query tile whose units fall to several workgroups is finished by merging
// their partial softmax states; each workgroup has at most two such pieces
// (the first and the last of its range), kept in slots 2 w and 2 w + 1.
// Key tiles that query tile qt sees when query row i sits at key position
// i + off (off = keys before the first query row: 0 for a plain prefill, the
// cached tokens before the chunk for a prefill against a cache).
constexpr int stream_ntiles(int Sq, int qt, int BM, int off = 0) {
  return ((Sq < BM * (qt + 1) ? Sq : BM * (qt + 1)) + off + 63) / 64;
}
// query tile of list position j within a (batch, head) block
constexpr int stream_pair_qt(int j, int nqt) { return (j & 1) ? (j >> 1) : nqt - 1 - (j >> 1); }

struct StreamPlan {
  int nqt;         // query tiles per (batch, head)
  int per;         // units per (batch, head)
  int units;       // all units
  int G;           // workgroups
  int piece_cost;  // cost of a piece (its prologue), in units
  bool ok;         // the sizes fit the 32-bit arithmetic
};

inline StreamPlan stream_plan(long long bh, int Sq, int BM, int slots, int min_units, int piece_cost, int off = 0) {
  const int nqt = (Sq + BM - 1) / BM;
  long long per = 0;
  for (int qt = 0; qt < nqt; qt++) per += stream_ntiles(Sq, qt, BM, off);
  const long long units = bh * per, cost = units + (long long)piece_cost * bh * nqt;
  // at least min_units units and more than piece_cost + 1 of cost per workgroup
  const long long G =
      std::max<long long>(1, std::min<long long>(slots, units / std::max(min_units, piece_cost + 2)));
  const bool ok = cost + G < (1LL << 31);
  return {nqt, (int)per, (int)units, (int)G, piece_cost, ok};
}

// The workgroups' ranges, computed on the host.  A range costs one per unit,
// plus piece_cost per query tile it touches (each piece loads its query rows
// and first K/V tile), plus merge_cost when it ends inside a tile: it then
// holds that tile's first pieces, runs them last and completes the tile's
// count, so it merges the pieces.  The ranges are the greedy cover (each
// workgroup takes the longest range within a budget) under the least budget
// that needs at most G workgroups; trailing workgroups may be left empty.
// For each workgroup: its first unit (wstart[G] = units), the list index of
// the tile holding its first unit, the workgroup holding that tile's first
// unit (lo_owner) and the one holding the last unit of the tile its range
// ends in (hi_owner): a tile shared by workgroups w0..w1 has one piece in
// each of them.
struct StreamRanges {
  std::vector<int> wstart, first_tile, lo_owner, hi_owner;
  long long budget;
};

// Workgroups the greedy cover under `budget` takes (G + 1: more than G);
// fills ws[0..G] when given.  tst[j]: first unit of list tile j within its
// (batch, head) block, tst[nqt] = per.
inline int stream_cover(const std::vector<int>& tst, int nqt, int per, int units, int G, int piece_cost,
                        int merge_cost, long long budget, int* ws) {
  int w = 0, ti = 0;  // ti: list index of the tile holding unit u
  long long u = 0;
  while (u < units) {
    if (w == G) return G + 1;
    if (ws) ws[w] = (int)u;
    const long long a = u;
    long long cost = 0;
    for (;;) {
      const int b = ti / nqt, j = ti - b * nqt;
      const long long end = (long long)b * per + tst[j + 1];
      const long long whole = cost + piece_cost + (end - u);
      if (whole <= budget) {  // the rest of this tile
        cost = whole;
        u = end;
        ti++;
        if (u == units) break;
        continue;
      }
      const long long k = budget - cost - piece_cost - merge_cost;  // a part of it, ending inside it
      if (k >= 1) u += std::min(k, end - u - 1);
      else if (u == a) return G + 1;  // not even one unit fits this budget
      break;
    }
    w++;
  }
  if (ws)
    for (int x = w; x <= G; x++) ws[x] = units;
  return w;
}

inline StreamRanges stream_ranges(const StreamPlan& p, long long bh, int Sq, int BM, int merge_cost, int off = 0) {
  std::vector<int> tst(p.nqt + 1, 0);
  for (int j = 0; j < p.nqt; j++) tst[j + 1] = tst[j] + stream_ntiles(Sq, stream_pair_qt(j, p.nqt), BM, off);
  long long lo = 0, hi = (long long)p.units + (long long)p.piece_cost * bh * p.nqt + merge_cost;  // hi always fits
  while (lo < hi) {
    const long long mid = (lo + hi) / 2;
    if (stream_cover(tst, p.nqt, p.per, p.units, p.G, p.piece_cost, merge_cost, mid, nullptr) <= p.G) hi = mid;
    else lo = mid + 1;
  }
  StreamRanges r;
  r.budget = hi;
  r.wstart.assign(p.G + 1, 0);
  stream_cover(tst, p.nqt, p.per, p.units, p.G, p.piece_cost, merge_cost, hi, r.wstart.data());
  r.first_tile.assign(p.G, 0);
  r.lo_owner.assign(p.G, 0);
  r.hi_owner.assign(p.G, 0);
  // list index and first unit of the tile holding unit u
  auto tile_of = [&](int u) {
    const int b = u / p.per, rr = u - b * p.per;
    const int j = (int)(std::upper_bound(tst.begin(), tst.begin() + p.nqt, rr) - tst.begin()) - 1;
    return std::make_pair(b * p.nqt + j, b * p.per + tst[j]);
  };
  auto owner = [&](int u) {  // the non-empty range holding u
    return (int)(std::upper_bound(r.wstart.begin(), r.wstart.end(), u) - r.wstart.begin()) - 1;
  };
  for (int w = 0; w < p.G; w++) {
    const int a = r.wstart[w], e = r.wstart[w + 1];
    if (a >= e) continue;
    const auto first = tile_of(a);
    r.first_tile[w] = first.first;
    r.lo_owner[w] = owner(first.second);
    const auto last = tile_of(e - 1);
    const int lb = last.first / p.nqt, lj = last.first - lb * p.nqt;
    r.hi_owner[w] = owner(lb * p.per + tst[lj + 1] - 1);
  }
  return r;
}

}  // namespace grid
}  // namespace rcgqa
