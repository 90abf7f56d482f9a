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

}  // namespace grid
}  // namespace rcgqa
