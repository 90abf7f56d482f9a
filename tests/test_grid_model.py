"""The prefill launcher's host-side grid model (csrc/grid_model.h), compiled
with g++ on the CPU: the closed-form key counts against brute force, the
per-XCD schedule estimate on cases with known answers, and the grid chosen
for the shapes whose two grids were timed on MI355X (the faster one each)."""
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "rope_causal_gqa_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <vector>
#include "grid_model.h"
using namespace rcgqa::grid;
int main() {
  long long a, b, c, cap;
  char what[16];
  while (std::scanf("%15s", what) == 1) {
    if (what[0] == 'r') {                       // rows_keys a b c cap
      std::scanf("%lld %lld %lld %lld", &a, &b, &c, &cap);
      std::printf("%.1f\n", rows_keys(a, b, c, cap));
    } else if (what[0] == 'b') {                // busiest_cu bh k w0 .. w(k-1)
      long long bh; int k;
      std::scanf("%lld %d", &bh, &k);
      std::vector<double> w(k);
      for (auto& x : w) std::scanf("%lf", &x);
      std::printf("%.3f\n", busiest_cu(w, bh));
    } else if (what[0] == 's') {                // stream bh Sq BM min_units piece_cost merge_cost off
      long long bh; int Sq, BM, mu, pc, mc, off;
      std::scanf("%lld %d %d %d %d %d %d", &bh, &Sq, &BM, &mu, &pc, &mc, &off);
      const StreamPlan p = stream_plan(bh, Sq, BM, kCUs, mu, pc, off);
      const StreamRanges r = stream_ranges(p, bh, Sq, BM, mc, off);
      std::vector<int> tst(p.nqt + 1, 0);
      for (int j = 0; j < p.nqt; j++) tst[j + 1] = tst[j] + stream_ntiles(Sq, stream_pair_qt(j, p.nqt), BM, off);
      const int less = stream_cover(tst, p.nqt, p.per, p.units, p.G, pc, mc, r.budget - 1, nullptr);
      std::printf("%d %d %d %d %lld %d\n", p.nqt, p.units, p.G, p.ok ? 1 : 0, r.budget, less);
      for (int w = 0; w < p.G; w++) {   // the kernel's walk over its range, from the tables
        const int a = r.wstart[w], e = r.wstart[w + 1];
        std::printf("w %d %d %d\n", w, a, e);
        int ti = r.first_tile[w];
        for (int u = a; u < e; ti++) {
          const int b = ti / p.nqt, j = ti - b * p.nqt, qt = stream_pair_qt(j, p.nqt);
          const int t0 = b * p.per + tst[j], n = tst[j + 1] - tst[j], k0 = u - t0;
          const int k_hi = std::min(n, k0 + (e - u));
          const int w0 = t0 < a ? r.lo_owner[w] : w, w1 = t0 + n > e ? r.hi_owner[w] : w;
          const long long me = 2LL * w + (t0 > a ? 1 : 0);
          const long long s0 = 2LL * w0 + (t0 > r.wstart[w0] ? 1 : 0);
          std::printf("%d %d %d %d %d %d %d %d %lld %d %d %lld %d %d\n", w, b, qt, k0, k_hi, n, t0, b * p.nqt + qt,
                      w1 > w0 ? me : -1LL, w0, w1, s0, a, e);
          u += k_hi - k0;
        }
      }
    } else {                                    // grid bh Sq causal nk window
      long long bh, nk; int Sq, causal, window;
      std::scanf("%lld %d %d %lld %d", &bh, &Sq, &causal, &nk, &window);
      const KeyGroupGrid g = key_group_grid(bh, Sq, causal != 0, nk, window);
      std::printf("%d %d\n", g.four ? 1 : 0, g.npairs);
    }
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("grid_model")
    src, exe = d / "drv.cpp", d / "drv"
    src.write_text(DRIVER)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)

    def run(lines):
        r = subprocess.run([str(exe)], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
        return r.stdout.split("\n")[:-1]
    return run


def test_rows_keys_matches_brute_force(model):
    rng = random.Random(7)
    cases = [(rng.randint(0, 300), rng.randint(0, 120), rng.randint(-400, 400), rng.randint(1, 500))
             for _ in range(2000)]
    cases = [(a, a + n, c, cap) for a, n, c, cap in cases]
    got = model([f"r {a} {b} {c} {cap}" for a, b, c, cap in cases])
    for (a, b, c, cap), g in zip(cases, got):
        assert float(g) == sum(min(max(i + c, 0), cap) for i in range(a, b)), (a, b, c, cap)


def _list_schedule(w, bh):
    """Brute force: 8 XCDs of 32 CUs; each XCD takes its share of the items in
    order (a contiguous eighth when the count is a multiple of 8, else every
    8th item) and gives each to the CU with the least work so far."""
    n = bh * len(w)
    worst = 0.0
    for x in range(8):
        items = range(x * (n // 8), (x + 1) * (n // 8)) if n % 8 == 0 else range(x, n, 8)
        load = [0.0] * 32
        for i in items:
            j = min(range(32), key=lambda c: load[c])
            load[j] += w[i % len(w)]
        worst = max(worst, max(load))
    return worst


def test_busiest_cu_known_cases(model):
    cases = [
        (8, [1.0] * 32),                                   # 256 equal items: one per CU
        (8, [1.0] * 33),                                   # 33 items per XCD: one CU takes two
        (1, [1.0] * 5),                                    # 5 items: not a multiple of 8
        (1, [64.0 - i for i in range(64)]),                # 8 items per XCD, one per CU
        (1, [1.0 + (i % 2) for i in range(512)]),          # 64 items of weights 1, 2, 1, 2, ...
        (3, [7.5 + 0.37 * i for i in range(41)]),          # 123 items, uneven
    ]
    got = [float(x) for x in model([f"b {bh} {len(w)} " + " ".join(repr(v) for v in w) for bh, w in cases])]
    assert got[:4] == [1.0, 2.0, 1.0, 64.0]
    for (bh, w), g in zip(cases, got):
        assert g == pytest.approx(_list_schedule(w, bh), abs=1e-3), (bh, len(w))


# (B*Hq, Sq, causal, keys, window) -> four key groups?  Each row is a shape
# whose two grids were both timed on MI355X; the expected choice is the faster.
TIMED = [
    ((8, 4096, 1, 4096, 0), True),     # the 8q/1kv head share of the 70B shape: 57 vs 65 us
    ((64, 512, 1, 4608, 0), False),    # chunk of 512 after 4096 cached: 80 vs 100 us
    ((8, 2048, 0, 2048, 0), True),     # non-causal, 8 heads: 28 vs 34 us
    ((8, 1024, 1, 1024, 0), True),     # 17 vs 21 us
    ((16, 1030, 0, 1030, 0), False),   # non-causal, ragged: 23 vs 32 us
    ((16, 2100, 1, 2100, 0), False),   # 36 vs 50 us
    ((8, 2100, 1, 2100, 0), True),     # 27 vs 34 us
]


@pytest.mark.parametrize("shape,four", TIMED)
def test_grid_choice_on_timed_shapes(model, shape, four):
    got = model(["g " + " ".join(str(x) for x in shape)])[0].split()
    assert bool(int(got[0])) == four
    bh, Sq, causal, _, _ = shape
    nqt2, nqt4 = (Sq + 63) // 64, (Sq + 127) // 128
    paired = causal and nqt2 > 1 and bh * ((nqt2 + 1) // 2) >= 256
    assert int(got[1]) == (((nqt2 + 1) // 2 if paired else nqt2) if four else nqt4)


@pytest.mark.parametrize("bh,Sq,BM,mu,pc,mc,off", [
    (8, 4096, 256, 4, 2, 3, 0), (8, 2100, 256, 4, 2, 3, 0), (1, 1, 256, 4, 2, 3, 0), (1, 257, 256, 4, 2, 3, 0),
    (4, 8192, 256, 4, 2, 3, 0), (16, 300, 256, 4, 2, 3, 0), (2, 64, 256, 1, 0, 0, 0), (8, 1024, 128, 4, 2, 0, 0),
    (3, 5000, 256, 7, 5, 4, 0), (64, 4096, 256, 4, 2, 3, 0), (64, 512, 256, 4, 2, 3, 4096),
    (8, 700, 256, 4, 2, 6, 3000), (3, 1, 256, 4, 2, 3, 77), (1, 32768, 256, 16, 2, 3, 0),
    (4, 16384, 256, 16, 2, 3, 0), (2, 512, 256, 4, 2, 3, 15872), (1, 2048, 256, 4, 2, 3, 6144)])
def test_stream_plan_covers_every_tile_once(model, bh, Sq, BM, mu, pc, mc, off):
    """The stream-K grid (causal problems on unpaired grids, plain or against a
    cache of `off` earlier tokens): workgroups take contiguous ranges of the
    unit list (batch-head, then query tiles in heavy / light pairs, then key
    tile), non-empty but for trailing ones, each within the budget (one per
    unit, pc per tile touched, mc when the range ends inside a tile), which
    is the least one whose greedy cover fits G workgroups; the pieces cover
    every key tile a query tile sees under the causal rule exactly once; a
    tile shared by several workgroups gives each of them a distinct partial
    slot (at most two per workgroup, the first piece of a range in slot 2w,
    the last in 2w + 1), its owners w0..w1 from the tables are the brute-force
    owners, and the merge order (w0..w1, slot s0 for w0 and 2w after) is the
    key order."""
    out = model([f"s {bh} {Sq} {BM} {mu} {pc} {mc} {off}"])
    nqt, units, G, ok, budget, less = (int(x) for x in out[0].split())
    assert ok
    # query row i at key position i + off: tile qt sees keys below min(Sq, BM (qt + 1)) + off
    ntiles = [(min(Sq, BM * (qt + 1)) + off + 63) // 64 for qt in range(nqt)]
    assert nqt == -(-Sq // BM) and units == bh * sum(ntiles)
    assert G == max(1, min(256, units // max(mu, pc + 2)))
    # list order: (batch, head), then query tiles in heavy / light pairs
    pairs = []
    for p in range((nqt + 1) // 2):
        pairs.append(nqt - 1 - p)
        if p != nqt - 1 - p:
            pairs.append(p)
    assert sorted(pairs) == list(range(nqt))
    order = [(b, qt) for b in range(bh) for qt in pairs]
    t0 = {}
    tile_at = np.zeros(units, dtype=np.int64)   # list index of the tile holding each unit
    acc = 0
    for i, (b, qt) in enumerate(order):
        t0[(b, qt)] = acc
        tile_at[acc:acc + ntiles[qt]] = i
        acc += ntiles[qt]
    ends = np.cumsum([ntiles[qt] for _, qt in order])
    bounds = {}
    rows = []
    for line in out[1:]:
        f = line.split()
        if f[0] == "w":
            bounds[int(f[1])] = (int(f[2]), int(f[3]))
        else:
            rows.append(tuple(int(x) for x in f))
    # ranges: contiguous from 0 to units, non-empty but for trailing empty ones
    assert sorted(bounds) == list(range(G))
    assert bounds[0][0] == 0 and bounds[G - 1][1] == units
    used = [w for w in range(G) if bounds[w][0] < bounds[w][1]]
    assert used == list(range(len(used))) and len(used) >= 1
    for w in range(G - 1):
        assert bounds[w][1] == bounds[w + 1][0]
    owner = np.zeros(units, dtype=np.int64)
    for w in used:
        owner[bounds[w][0]:bounds[w][1]] = w

    def cost(a, e):
        t = tile_at[a:e]
        c = (e - a) + pc * (int(t[-1]) - int(t[0]) + 1)
        return c + (mc if e < ends[t[-1]] else 0)
    # every range within the budget; one less needs more than G workgroups
    for w in used:
        assert cost(*bounds[w]) <= budget
    assert less > G
    total = units + pc * len(order)
    assert budget <= total / G + 2 * (pc + mc) + 2
    cover = {}
    slots = {}
    per_wg = {}
    for w, b, qt, klo, khi, n, t, tile, me, w0, w1, s0, a, e in rows:
        assert (a, e) == bounds[w]
        assert 0 <= b < bh and 0 <= qt < nqt and n == ntiles[qt]
        assert t == t0[(b, qt)] and tile == b * nqt + qt
        assert 0 <= klo < khi <= n and a <= t + klo and t + khi <= e
        assert (w0, w1) == (owner[t], owner[t + n - 1])
        per_wg[w] = per_wg.get(w, 0) + khi - klo
        cover.setdefault((b, qt), []).append((klo, khi, w, me, w0, w1, s0))
        if w1 > w0:
            assert 0 <= me < 2 * G and me // 2 == w and me not in slots
            assert me == 2 * w + (1 if t > a else 0)
            slots[me] = (b, qt)
        else:
            assert me == -1 and (klo, khi) == (0, n)
    for w in used:
        assert per_wg[w] == bounds[w][1] - bounds[w][0]
    assert len(cover) == bh * nqt
    for (b, qt), pieces in cover.items():
        pieces.sort()
        assert pieces[0][0] == 0 and pieces[-1][1] == ntiles[qt]
        assert all(pieces[i][1] == pieces[i + 1][0] for i in range(len(pieces) - 1))
        ws = [p[2] for p in pieces]
        w0, w1 = pieces[0][4], pieces[0][5]
        assert ws == list(range(w0, w1 + 1))          # one piece per workgroup w0..w1, in key order
        if w1 > w0:
            s0 = pieces[0][6]
            merge_slots = [s0] + [2 * w for w in range(w0 + 1, w1 + 1)]
            assert merge_slots == [p[3] for p in pieces]
