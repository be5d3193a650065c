// dsa_topk_tile.h -- per-tile candidate reports for the exact Top-K.
//
// A score row is cut into tiles of `tile` consecutive positions.  Each tile
// reports a PREFIX of its elements in the selection order (score descending,
// position ascending): every element it leaves out is worse than the worst
// element it reports.  The resolve kernel then takes the K-th best element
// theta of the union of all reports and certifies the result: if, for every
// tile that left elements out, the worst reported element is not better than
// theta, no left-out element can belong to the top K, so the top K of the
// union is the exact top K of the row.  If any tile fails the check, the
// resolve kernel falls back to an exact radix select over the whole row.
//
// A tile is handled by one wave, its order keys in registers (each lane a
// run of consecutive elements).  It reports exactly min(kRep, n) elements:
// the kRep-th best key T is found by bisection over the tile's key interval
// [min, max] with per-lane counts joined across the wave (or across the
// lane group of a sub-tile), and the report is {key > T} plus the lowest
// positions with key == T, which is an exact prefix.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int kRep = 16;  // candidates reported per tile

// Rows of at most kDirectMax positions are selected straight from their
// scores (the whole row fits the resolve block's registers); longer rows
// are reported in sub-tiles of topk_subtile(n, K) positions.
constexpr int kDirectMax = 16384;
constexpr int kSubMin = 32;
constexpr int kSubMax = 2048;
constexpr int kSubTiles = 1024;  // most sub-tiles a row may have on the fast path

// Sub-tile size for a row of n positions: the largest power of two S in
// [kSubMin, kSubMax] with S <= 4 n / K (about four of the row's top K per
// sub-tile, so one rarely holds more than kRep of them), raised until the row
// has at most kSubTiles sub-tiles.  Non-decreasing in n.
__host__ __device__ inline int topk_subtile(int64_t n, int K) {
  const int64_t k = K > 0 ? K : 1;
  const int64_t by_tiles = (n + kSubTiles - 1) / kSubTiles;
  int s = kSubMin;
  // 2 s <= floor(4 n / k)  <=>  2 s k <= 4 n  (no division on the device)
  while (s < kSubMax && 2 * (int64_t)s * k <= 4 * n) s <<= 1;
  while (s < kSubMax && s < by_tiles) s <<= 1;
  return s;
}

struct RepHeader {
  uint32_t count;     // reported elements
  uint32_t complete;  // 1: every element of the tile is reported
  uint32_t worst_u;   // order key of the worst reported element
  int32_t worst_j;    // its position
};

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

__device__ __forceinline__ uint64_t lanes_below() {
  const int l = lane_id();
  return (l == 0) ? 0ull : (~0ull >> (64 - l));
}

// Wave-level tile report.  Lane l holds the V order keys u[i] of the tile's
// elements V l + i (lane-major, so position order is lane order, then i);
// the first nv of them are valid and the lane's element 0 sits at position
// jbase.  Writes the report (positions ascending) and its header.  Every
// count, rank and placement is a per-lane sum joined by one wave scan or
// reduction (DPP); the bisection of short lanes counts with ballots.
template <int V>
__device__ void wave_tile_report(const uint32_t (&u)[V], int nv, int64_t jbase, RepHeader* hdr,
                                 uint32_t* rep_u, int32_t* rep_j) {
  uint32_t uz[V];  // invalid slots as key 0: every probe below is >= 1
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool v = i < nv;
    uz[i] = v ? u[i] : 0u;
    mn = min(mn, v ? u[i] : 0xffffffffu);
    mx = max(mx, uz[i]);
  }
  const uint32_t n = wave_sum_u32((uint32_t)nv);
  mn = wave_min_u32(mn);
  bool sel[V];
  uint32_t wu;  // key of the worst reported element
  const bool complete = n <= (uint32_t)kRep;
  if (complete) {
#pragma unroll
    for (int i = 0; i < V; ++i) sel[i] = i < nv;
    wu = mn;
  } else {
    // largest T with count(key >= T) >= kRep: the kRep-th best key.  A
    // probe with exactly kRep keys at or above it ends the search early:
    // those kRep elements are the report.
    uint32_t lo = mn, hi = wave_max_u32(mx);
    bool exact = false;
    while (lo < hi) {
      const uint32_t mid = lo + ((hi - lo) >> 1) + 1;  // in (lo, hi]
      uint32_t c = 0;
      if constexpr (V >= 8) {
#pragma unroll
        for (int i = 0; i < V; ++i) c += uz[i] >= mid ? 1u : 0u;
        c = wave_sum_u32(c);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) c += popc64(__ballot(uz[i] >= mid));
      }
      if (c == (uint32_t)kRep) {
        lo = mid;
        exact = true;
        break;
      }
      if (c > (uint32_t)kRep) lo = mid; else hi = mid - 1;
    }
    const uint32_t T = lo;
    if (exact) {
      uint32_t m = 0xffffffffu;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        sel[i] = uz[i] >= T;
        m = min(m, sel[i] ? u[i] : 0xffffffffu);
      }
      wu = wave_min_u32(m);
    } else {
      // T is a key: {key > T} plus the need lowest positions with key == T
      uint32_t g = 0, ce = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        g += uz[i] > T ? 1u : 0u;
        ce += (i < nv && u[i] == T) ? 1u : 0u;
      }
      const uint32_t need = (uint32_t)kRep - wave_sum_u32(g);
      uint32_t r = wave_incl_scan(ce) - ce;  // copies of T in lower lanes
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const bool eq = i < nv && u[i] == T;
        sel[i] = uz[i] > T || (eq && r < need);
        r += eq ? 1u : 0u;
      }
      wu = T;
    }
  }
  // placement in position order: lanes in order, each lane's elements in order
  uint32_t cs = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) cs += sel[i] ? 1u : 0u;
  const uint32_t incl = wave_incl_scan(cs);
  const uint32_t count = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  uint32_t pos = incl - cs;
  int32_t wj = -1;  // highest selected position with key wu
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (sel[i]) {
      rep_u[pos] = u[i];
      rep_j[pos] = (int32_t)(jbase + i);
      ++pos;
      if (u[i] == wu) wj = (int32_t)(jbase + i);
    }
  }
  wj = wave_max_i32(wj);
  if (lane_id() == 0) {
    RepHeader h;
    h.count = count;
    h.complete = complete ? 1u : 0u;
    h.worst_u = wu;
    h.worst_j = wj;
    *hdr = h;
  }
}

// Segmented wave primitives over aligned groups of g lanes (g a power of
// two, 1 <= g <= 64, uniform over the wave), built from DPP row shifts and
// row broadcasts like the whole-wave scans.  Every step runs for every g
// (steps that cross a group boundary are masked per lane), so there are no
// branches.
//   seg_scan:      inclusive scan with `op` (identity id) within each group;
//   seg_last:      every lane of a group gets the value of the group's last
//                  lane.
template <typename Op>
__device__ __forceinline__ uint32_t seg_scan(uint32_t v, uint32_t id, int g, Op op) {
  // a row shift by k reads lane l - k; it stays in the group iff r >= k,
  // which never holds for k >= g
  const int r = lane_id() & (g - 1);
  uint32_t t = dpp_u32<kDppRowShr1, 0xf, 0xf>(id, v);
  v = op(v, r >= 1 ? t : id);
  t = dpp_u32<kDppRowShr2, 0xf, 0xf>(id, v);
  v = op(v, r >= 2 ? t : id);
  t = dpp_u32<kDppRowShr4, 0xf, 0xf>(id, v);
  v = op(v, r >= 4 ? t : id);
  t = dpp_u32<kDppRowShr8, 0xf, 0xf>(id, v);
  v = op(v, r >= 8 ? t : id);
  // rows 1 and 3 add the previous row's last lane (groups of 32 and 64),
  // rows 2 and 3 lane 31 (groups of 64)
  t = dpp_u32<kDppRowBcast15, 0xa, 0xf>(id, v);
  v = op(v, g >= 32 ? t : id);
  t = dpp_u32<kDppRowBcast31, 0xc, 0xf>(id, v);
  v = op(v, g >= 64 ? t : id);
  return v;
}

constexpr int kDppRowShl1 = 0x101, kDppRowShl2 = 0x102, kDppRowShl4 = 0x104, kDppRowShl8 = 0x108;

__device__ __forceinline__ uint32_t seg_last(uint32_t v, int g) {
  const int l = lane_id(), r = l & (g - 1);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  const uint32_t wide = (g == 64 || l >= 32) ? b : a;  // groups of 32 or 64 lanes
  // lane r takes lane r + k's value while that lane is in the group: after
  // the steps k = 1, 2, 4, 8 it holds the value of lane g - 1 (g <= 16)
  uint32_t t = dpp_u32<kDppRowShl1, 0xf, 0xf>(v, v);
  v = r + 1 < g ? t : v;
  t = dpp_u32<kDppRowShl2, 0xf, 0xf>(v, v);
  v = r + 2 < g ? t : v;
  t = dpp_u32<kDppRowShl4, 0xf, 0xf>(v, v);
  v = r + 4 < g ? t : v;
  t = dpp_u32<kDppRowShl8, 0xf, 0xf>(v, v);
  v = r + 8 < g ? t : v;
  return g >= 32 ? wide : v;
}

__device__ __forceinline__ uint32_t seg_sum(uint32_t v, int g) {
  return seg_last(seg_scan(v, 0u, g, [](uint32_t a, uint32_t b) { return a + b; }), g);
}
__device__ __forceinline__ uint32_t seg_min(uint32_t v, int g) {
  return seg_last(seg_scan(v, 0xffffffffu, g, [](uint32_t a, uint32_t b) { return a < b ? a : b; }), g);
}
__device__ __forceinline__ uint32_t seg_max(uint32_t v, int g) {
  return seg_last(seg_scan(v, 0u, g, [](uint32_t a, uint32_t b) { return a > b ? a : b; }), g);
}

// Sub-tile reports of one tile of 64 V positions whose row uses sub-tiles of
// S < 64 V positions (S a power of two, S >= V).  The tile holds NS = 64 V / S
// sub-tiles; each is served by a group of g = S / V consecutive lanes, lane r
// of group s holding the sub-tile's elements V r + i (i < V), so that
// position order is lane order, then i.  Every count, rank and placement is
// a per-lane sum joined by a segmented DPP scan over the group, so all
// groups bisect at once.  `get(e)` returns the score of tile element e
// (e < n_valid); sub-tile s of the tile writes report s (header hdr[s],
// slots rep[kRep s ..]) when it holds at least one valid element.
template <int V, typename Get>
__device__ void wave_subtile_reports(Get get, int n_valid, int64_t j0, int S, RepHeader* hdr,
                                     uint32_t* rep_u, int32_t* rep_j) {
  const int l = lane_id();
  const int g = S / V;
  const int lg = 31 - __clz(g);
  const int grp = l >> lg, r = l & (g - 1);
  const int e0 = grp * S + V * r;  // tile index of this lane's element 0
  const int nv = min(max(n_valid - e0, 0), V);
  uint32_t u[V];  // invalid slots as key 0: every probe below is >= 1
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    u[i] = i < nv ? order_key(get(e0 + i)) : 0u;
    mn = min(mn, i < nv ? u[i] : 0xffffffffu);
    mx = max(mx, u[i]);
  }
  const uint32_t n = seg_sum((uint32_t)nv, g);
  mn = seg_min(mn, g);
  mx = seg_max(mx, g);
  const bool complete = n <= (uint32_t)kRep;
  // per group: largest T with count(key >= T) >= kRep; a probe with exactly
  // kRep keys at or above it ends the group's search early
  uint32_t lo = mn, hi = mx;
  bool exact = false;
  bool done = complete || lo >= hi;
  while (__ballot(!done) != 0ull) {
    const uint32_t mid = lo + ((hi - lo) >> 1) + 1;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) c += u[i] >= mid ? 1u : 0u;
    c = seg_sum(c, g);
    if (!done) {
      if (c == (uint32_t)kRep) {
        lo = mid;
        exact = true;
        done = true;
      } else {
        if (c > (uint32_t)kRep) lo = mid; else hi = mid - 1;
        done = lo >= hi;
      }
    }
  }
  const uint32_t T = lo;
  bool sel[V];
  uint32_t wu;  // key of the worst reported element of the group
  if (complete) {
#pragma unroll
    for (int i = 0; i < V; ++i) sel[i] = i < nv;
    wu = mn;
  } else if (exact) {
    uint32_t m = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      sel[i] = u[i] >= T;
      m = min(m, sel[i] ? u[i] : 0xffffffffu);
    }
    wu = seg_min(m, g);
  } else {
    // T is a key: {key > T} plus the need lowest positions with key == T
    uint32_t gt = 0, ce = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      gt += u[i] > T ? 1u : 0u;
      ce += (i < nv && u[i] == T) ? 1u : 0u;
    }
    const uint32_t need = (uint32_t)kRep - seg_sum(gt, g);
    uint32_t rk = seg_scan(ce, 0u, g, [](uint32_t a, uint32_t b) { return a + b; }) - ce;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool eq = i < nv && u[i] == T;
      sel[i] = u[i] > T || (eq && rk < need);
      rk += eq ? 1u : 0u;
    }
    wu = T;
  }
  // placement in position order; worst position: the highest selected
  // position with key wu (biased by 1 so that none is 0)
  uint32_t cs = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) cs += sel[i] ? 1u : 0u;
  const uint32_t incl = seg_scan(cs, 0u, g, [](uint32_t a, uint32_t b) { return a + b; });
  const uint32_t count = seg_last(incl, g);
  const bool live = n > 0u;
  uint32_t pos = incl - cs;
  uint32_t wj1 = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (sel[i]) {
      if (live) {
        rep_u[grp * kRep + pos] = u[i];
        rep_j[grp * kRep + pos] = (int32_t)(j0 + e0 + i);
      }
      ++pos;
      if (u[i] == wu) wj1 = (uint32_t)(j0 + e0 + i) + 1u;
    }
  }
  wj1 = seg_max(wj1, g);
  if (r == 0 && live) {
    RepHeader h;
    h.count = count;
    h.complete = complete ? 1u : 0u;
    h.worst_u = wu;
    h.worst_j = (int32_t)wj1 - 1;
    hdr[grp] = h;
  }
}

}  // namespace dsa
