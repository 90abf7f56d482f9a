"""The prefill launcher's host-side grid model (csrc/grid_model.h), compiled
with g++ on the CPU: the closed-form key counts against brute force, the
per-XCD schedule estimate on cases with known answers, and the grid chosen
for the shapes whose two grids were timed on MI355X (the faster one each)."""
import os
import random
import shutil
import subprocess

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
