// Index arithmetic of the grouped-GEMM work plan, shared by the planner kernel, the
// grouped GEMM kernels and a plain C++ build that checks it on the CPU (no HIP
// dependency).  [MND §Roofline / GroupGEMM]: group i multiplies its own m_i rows by its
// own weights; here a group's rows are cut into slices (units) of at most BM rows.
#pragma once

#include "addr.h"   // MOE_HD

namespace moe {

// Units of a group of n rows: ceil(n / BM) near-equal slices.
MOE_HD inline int plan_units_of(int n, int BM) { return n > 0 ? (n + BM - 1) / BM : 0; }

// Rows per slice of a group of n rows cut into nu units, rounded up to whole 16-row tiles
// (the last slice takes the rest: n - (nu - 1) * per >= 1 rows, since per <= BM).
MOE_HD inline int plan_slice_rows(int n, int nu) { return ((n + nu - 1) / nu + 15) & ~15; }

// The extra group's (the shared expert's) nx slices spread through the table: slices
// placed before the units of groups 0 .. g, min(nx, ceil((g + 1) * nx / G)).
MOE_HD inline int plan_extra_upto(int g, int nx, int G) {
  if (nx == 0 || g < 0) return 0;
  const long long c = (static_cast<long long>(g + 1) * nx + G - 1) / G;
  return static_cast<int>(c < nx ? c : nx);
}

// Cost of a unit of `rows` rows when the table is cut into per-XCD chunks: its 16-row
// tiles, counted as at least cost_floor rows, plus one for its prologue and epilogue.
MOE_HD inline long long plan_unit_cost(int rows, int cost_floor) {
  const int r = rows > cost_floor ? rows : cost_floor;
  return (r + 15) / 16 + 1;
}

// Whether a unit whose cost midpoint is mid2 / 2 (mid2 = 2 * cost before it + its cost)
// lies before x / nx of the total cost `all`.
MOE_HD inline bool plan_below(long long mid2, int x, int nx, long long all) {
  return mid2 * nx < 2LL * x * all;
}

// Chunk bounds from below[x] (x = 1 .. nx-1: units whose midpoints lie before x / nx of
// the cost): bounds[0] = 0, bounds[nx] = total, and in between each bound clamped in
// order so that every chunk holds at most per_chunk = ceil(cap / nx) units (the most a
// grid sized for cap units gives one XCD) and what is left still fits the later chunks.
// Needs total <= cap.
MOE_HD inline void plan_chunk_bounds(const int* below, int total, int cap, int nx, int* bounds) {
  const int per_chunk = (cap + nx - 1) / nx;
  int b = 0;
  bounds[0] = 0;
  for (int x = 1; x < nx; ++x) {
    const int rest = total - (nx - x) * per_chunk;
    const int lo = b > rest ? b : rest;
    const int hi = b + per_chunk;
    const int v = below[x] > lo ? below[x] : lo;
    b = v < hi ? v : hi;
    bounds[x] = b;
  }
  bounds[nx] = total;
}

// Work item of slot `slot` of an XCD whose chunk is units [c0, c1), per_unit items per
// unit: the chunk is walked run by run (a run: the consecutive units of one group,
// [first, first + count)), item major inside a run.  `first` and `count` are those of unit
// c0 + slot / per_unit.  Returns false past the chunk's last item; otherwise *u is the
// unit and *item its item (N tile and split).
MOE_HD inline bool plan_map_slot(int slot, int per_unit, int c0, int c1, int first, int count,
                                 int* u, int* item) {
  if (slot >= (c1 - c0) * per_unit) return false;
  const int rs = first > c0 ? first : c0;
  const int re = first + count < c1 ? first + count : c1;
  const int l = slot - (rs - c0) * per_unit;
  *item = l / (re - rs);
  *u = rs + l % (re - rs);
  return true;
}

}  // namespace moe
