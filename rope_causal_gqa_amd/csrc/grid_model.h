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

// Stream-K plan for small causal grids (no cache, no mask).  A unit is one
// (query tile of BM rows, 64-key tile) step of the causal work.  Units are
// listed (batch, head) by (batch, head); within one, query tiles in heavy /
// light pairs (the last tile, the first, the second last, the second, ...),
// and within a tile key tile by key tile.  Each workgroup takes a contiguous
// range of the list.  The ranges balance a cost of one per unit plus
// `tile_cost` per tile started (the prologue and the hand-over a piece of a
// tile brings), through the cumulative cost C(u) = u + tile_cost * (tiles
// that start before unit u): workgroup w starts at the first unit u with
// C(u) G >= w C(units).  A query tile whose units fall to several
// workgroups is finished by merging their partial softmax states; each
// workgroup has at most two such pieces (the first and the last of its
// range), kept in slots 2 w and 2 w + 1.  All in 32-bit integers (the plan
// is used only where C(units) G fits), constexpr so that the kernel runs
// this code: every (batch, head) block has the same layout, so each step is
// one division and a walk over one block's tiles.
// Key tiles that query tile qt sees when query row i sits at key position
// i + off (off = keys before the first query row: 0 for a plain prefill, the
// cached tokens before the chunk for a prefill against a cache).
constexpr int stream_ntiles(int Sq, int qt, int BM, int off = 0) {
  return ((Sq < BM * (qt + 1) ? Sq : BM * (qt + 1)) + off + 63) / 64;
}
// query tile of list position j within a (batch, head) block
constexpr int stream_pair_qt(int j, int nqt) { return (j & 1) ? (j >> 1) : nqt - 1 - (j >> 1); }

struct StreamPlan {
  int nqt;        // query tiles per (batch, head)
  int per;        // units per (batch, head)
  int units;      // all units
  int G;          // workgroups
  int tile_cost;  // cost of starting a tile, in units
  int cost;       // C(units)
  bool ok;        // the sizes fit the 32-bit arithmetic
};

inline StreamPlan stream_plan(long long bh, int Sq, int BM, int slots, int min_units, int tile_cost, int off = 0) {
  const int nqt = (Sq + BM - 1) / BM;
  long long per = 0;
  for (int qt = 0; qt < nqt; qt++) per += stream_ntiles(Sq, qt, BM, off);
  const long long units = bh * per, cost = units + (long long)tile_cost * bh * nqt;
  // at least min_units units and more than tile_cost + 1 of cost per workgroup, so that no range is empty
  const long long G =
      std::max<long long>(1, std::min<long long>(slots, units / std::max(min_units, tile_cost + 2)));
  const bool ok = cost * (G + 1) < (1LL << 31);
  return {nqt, (int)per, (int)units, (int)G, tile_cost, (int)cost, ok};
}

// The query tile that unit u falls in: its (batch, head), query tile qt, key
// tile k within it, its key-tile count n, its first unit t0, its counter
// slot (bh nqt + qt) and the number of tiles that start before it.
struct StreamTile {
  int bh, qt, k, n, t0, tile, before;
};
constexpr StreamTile stream_tile(int u, int nqt, int per, int Sq, int BM, int off = 0) {
  const int b = u / per, r = u - b * per;
  int s = 0, j = 0;
  for (; j < nqt - 1; j++) {
    const int n = stream_ntiles(Sq, stream_pair_qt(j, nqt), BM, off);
    if (r < s + n) break;
    s += n;
  }
  const int qt = stream_pair_qt(j, nqt);
  return {b, qt, r - s, stream_ntiles(Sq, qt, BM, off), b * per + s, b * nqt + qt, b * nqt + j};
}

// C(u) for 0 <= u <= units
constexpr int stream_cost(int u, int units, int nqt, int per, int Sq, int BM, int tile_cost, int off = 0) {
  if (u >= units) return units + tile_cost * (units / per) * nqt;
  const StreamTile t = stream_tile(u, nqt, per, Sq, BM, off);
  return u + tile_cost * (t.before + (u > t.t0 ? 1 : 0));
}

// First unit of workgroup w (w = G gives `units`): the first u with
// C(u) >= c = ceil(w cost / G), found in the (batch, head) block that c
// falls in (each block adds per + tile_cost nqt to C)
constexpr int stream_start(int w, int G, int units, int cost, int nqt, int per, int Sq, int BM, int tile_cost,
                           int off = 0) {
  const int c = (w * cost + G - 1) / G;
  const int cb = per + tile_cost * nqt;
  const int b = c / cb, rem = c - b * cb;
  if (b * per >= units) return units;
  int s = 0;
  for (int j = 0; j < nqt; j++) {
    if (rem <= s + tile_cost * j) return b * per + s;  // at tile j's first unit
    const int n = stream_ntiles(Sq, stream_pair_qt(j, nqt), BM, off);
    if (rem <= s + n + tile_cost * (j + 1)) {           // inside tile j: C = u + tile_cost (j + 1)
      const int r = rem - tile_cost * (j + 1);
      return b * per + (r > s + 1 ? r : s + 1);
    }
    s += n;
  }
  return b * per + per;
}

// Workgroup that runs unit u (u < units)
constexpr int stream_owner(int u, int G, int units, int cost, int nqt, int per, int Sq, int BM, int tile_cost,
                           int off = 0) {
  return stream_cost(u, units, nqt, per, Sq, BM, tile_cost, off) * G / cost;
}

}  // namespace grid
}  // namespace rcgqa
