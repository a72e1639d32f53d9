// CPU checks of the work-plan index helpers the planner kernel and the grouped GEMM use
// (moe_expert_layer_top_amd/csrc/plan.h): unit tables built from random, skewed and edge
// case group sizes in the planner's table order, cut into per-XCD chunks, then every work
// item of every unit must be reached by exactly one workgroup slot of the launch grid.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "plan.h"

static int failures = 0;

static void expect(bool ok, const char* what, int trial) {
  if (!ok && failures < 20) std::printf("FAILED (trial %d): %s\n", trial, what);
  if (!ok) ++failures;
}

struct U {
  int group, row0, rows, first, count;
};

// One plan: groups of counts[g] rows (contiguous from row 0), plus extra_rows rows of
// group G spread through the table; cap = the unit bound the grid is sized for.
static void check_plan(const std::vector<int>& counts, int BM, int extra_rows, int cap, int cost_floor,
                       int per_unit, int trial) {
  const int G = static_cast<int>(counts.size());
  const int X = 8;
  const int nx = moe::plan_units_of(extra_rows, BM);
  const int per_x = nx > 0 ? moe::plan_slice_rows(extra_rows, nx) : 0;
  std::vector<U> units(cap, U{-1, 0, 0, 0, 0});
  int base = 0, start = 0;
  for (int g = 0; g < G; ++g) {
    const int n = counts[g];
    const int nu = moe::plan_units_of(n, BM);
    const int x0 = moe::plan_extra_upto(g - 1, nx, G), x1 = moe::plan_extra_upto(g, nx, G);
    for (int i = x0; i < x1; ++i) {
      const int r = per_x < extra_rows - i * per_x ? per_x : extra_rows - i * per_x;
      if (base + i < cap) units[base + i] = U{G, i * per_x, r, base + x0, x1 - x0};
    }
    if (nu > 0) {
      const int per = moe::plan_slice_rows(n, nu);
      expect(per <= BM || BM % 16 != 0, "slice rows within BM", trial);
      int covered = 0;
      for (int i = 0; i < nu; ++i) {
        const int r = per < n - i * per ? per : n - i * per;
        expect(r >= 1, "every slice holds a row", trial);
        covered += r;
        if (base + x1 + i < cap) units[base + x1 + i] = U{g, start + i * per, r, base + x1, nu};
      }
      expect(covered == n, "a group's slices cover its rows exactly", trial);
    }
    base += nu;
    start += n;
  }
  expect(moe::plan_extra_upto(G - 1, nx, G) == nx, "every extra slice is placed", trial);
  const int total = base + nx < cap ? base + nx : cap;
  for (int i = 0; i < total; ++i) {
    expect(units[i].group >= 0, "table entries below the count are written", trial);
    expect(units[i].first <= i && i < units[i].first + units[i].count, "a unit lies in its run", trial);
  }
  // chunk bounds by cost
  long long all = 0;
  for (int i = 0; i < total; ++i) all += moe::plan_unit_cost(units[i].rows, cost_floor);
  int below[8] = {0};
  long long before = 0;
  for (int i = 0; i < total; ++i) {
    const long long c = moe::plan_unit_cost(units[i].rows, cost_floor);
    for (int x = 1; x < X; ++x) below[x] += moe::plan_below(2 * before + c, x, X, all) ? 1 : 0;
    before += c;
  }
  int bounds[9];
  moe::plan_chunk_bounds(below, total, cap, X, bounds);
  const int per_chunk = (cap + X - 1) / X;
  expect(bounds[0] == 0 && bounds[X] == total, "chunks span the table", trial);
  for (int x = 0; x < X; ++x) {
    expect(bounds[x] <= bounds[x + 1], "chunk bounds are ordered", trial);
    expect(bounds[x + 1] - bounds[x] <= per_chunk, "a chunk fits the grid's slots of its XCD", trial);
  }
  // the grid: per_chunk units' worth of slots per XCD, block id mod 8 = XCD
  std::vector<int> seen(static_cast<size_t>(total) * per_unit, 0);
  const long long blocks = static_cast<long long>(per_chunk) * X * per_unit;
  for (long long bid = 0; bid < blocks; ++bid) {
    const int xcd = static_cast<int>(bid % X), slot = static_cast<int>(bid / X);
    const int c0 = bounds[xcd], c1 = bounds[xcd + 1];
    if (slot >= (c1 - c0) * per_unit) continue;
    const int q = c0 + slot / per_unit;
    int u = -1, item = -1;
    const bool ok = moe::plan_map_slot(slot, per_unit, c0, c1, units[q].first, units[q].count, &u, &item);
    expect(ok, "an in-chunk slot maps", trial);
    if (!ok) continue;
    expect(u >= c0 && u < c1, "the unit lies in the XCD's chunk", trial);
    expect(item >= 0 && item < per_unit, "the item is in range", trial);
    if (u < c0 || u >= c1 || item < 0 || item >= per_unit) continue;
    expect(units[u].group == units[q].group, "the unit is of the slot's run", trial);
    // item (N tile) major inside a run: the slot before, unless it starts a new item of
    // the run, is the previous unit of the same run and the same item
    const int rs = units[q].first > c0 ? units[q].first : c0;
    if (u > rs) {
      int pu = -1, pitem = -1;
      const int pq = c0 + (slot - 1) / per_unit;
      moe::plan_map_slot(slot - 1, per_unit, c0, c1, units[pq].first, units[pq].count, &pu, &pitem);
      expect(pu == u - 1 && pitem == item, "consecutive slots of a run share the item", trial);
    }
    ++seen[static_cast<size_t>(u) * per_unit + item];
  }
  for (size_t i = 0; i < seen.size(); ++i) expect(seen[i] == 1, "every item of every unit runs once", trial);
}

int main() {
  std::mt19937 rng(12345);
  int trial = 0;
  auto max_units = [](int BM, int G, int R, int extra) {
    return R / BM + (G < R ? G : R) + (extra > 0 ? extra / BM + 1 : 0);
  };
  // edge cases: one dense group, empty groups, one hot group, more units than the cap
  check_plan({65536}, 320, 0, max_units(320, 1, 65536, 0), 160, 16, ++trial);
  check_plan({0, 0, 5, 0}, 256, 0, max_units(256, 4, 5, 0), 128, 16, ++trial);
  check_plan({4000, 0, 1, 1}, 256, 1000, max_units(256, 4, 4002, 1000), 128, 28, ++trial);
  check_plan({5000, 0, 3000}, 256, 0, 8, 128, 4, ++trial);          // rows beyond the sized bound
  check_plan({17, 33, 1}, 32, 100, max_units(32, 3, 51, 100), 32, 1, ++trial);
  for (int t = 0; t < 400; ++t) {
    static const int Gs[] = {1, 3, 8, 16, 32, 64, 256, 1024};
    static const int BMs[] = {32, 64, 256, 320};
    static const int PUs[] = {1, 2, 4, 16, 28};
    const int G = Gs[rng() % 8], BM = BMs[rng() % 4], per_unit = PUs[rng() % 5];
    const int R = 1 + static_cast<int>(rng() % 40000);
    const int extra = (rng() % 3 == 0) ? 1 + static_cast<int>(rng() % 9000) : 0;
    // counts: uniform, Zipf-like or clustered on a few groups, some groups empty
    std::vector<double> w(G);
    const int kind = static_cast<int>(rng() % 3);
    for (int g = 0; g < G; ++g)
      w[g] = kind == 0 ? 1.0 : kind == 1 ? 1.0 / (1 + g) : ((rng() % 8 == 0) ? 8.0 : 0.05);
    double sw = 0;
    for (double v : w) sw += v;
    std::vector<int> counts(G, 0);
    int left = R;
    for (int g = 0; g < G && left > 0; ++g) {
      int c = static_cast<int>(R * w[g] / sw);
      if (c > left) c = left;
      counts[g] = c;
      left -= c;
    }
    counts[rng() % G] += left;
    if (rng() % 5 == 0) counts[rng() % G] = 0;
    int sum = 0;
    for (int c : counts) sum += c;
    const int cap = max_units(BM, G, sum, extra) > 0 ? max_units(BM, G, sum, extra) : 1;
    const int floor = (rng() % 2) ? BM / 2 : BM;
    check_plan(counts, BM, extra, cap, floor, per_unit, ++trial);
  }
  if (failures) {
    std::printf("%d plan check(s) failed\n", failures);
    return 1;
  }
  std::printf("all plan checks passed (%d plans)\n", trial);
  return 0;
}
