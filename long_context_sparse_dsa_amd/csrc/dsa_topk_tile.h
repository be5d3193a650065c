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
// A tile is handled by one wave, its order keys in registers.  It reports
// exactly min(kRep, n) elements: the kRep-th best key T is found by
// bisection over the tile's key interval [min, max] with wave-ballot
// counts, and the report is {key > T} plus the lowest positions with key
// == T, which is an exact prefix.
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

// Sub-tile reports of one tile of 64 V positions whose row uses sub-tiles of
// S < 64 V positions (S a power of two, S >= V).  The tile holds NS = 64 V / S
// sub-tiles; each is served by a group of g = S / V consecutive lanes, lane r
// of group s holding the sub-tile's elements r + g i (i < V), so that the
// order (i, r) is position order.  Every count is a wave ballot masked to the
// group, so all groups bisect at once.  `get(e)` returns the score of tile
// element e (e < n_valid); sub-tile s of the tile writes report s (header
// hdr[s], slots rep[kRep s ..]) when it holds at least one valid element.
template <int V, typename Get>
__device__ void wave_subtile_reports(Get get, int n_valid, int64_t j0, int S, RepHeader* hdr,
                                     uint32_t* rep_u, int32_t* rep_j) {
  const int l = lane_id();
  const int g = S / V;
  const int lg = 31 - __clz(g);
  const int grp = l >> lg, r = l & (g - 1);
  const int sh = grp << lg;
  const uint64_t gm = g >= 64 ? ~0ull : ((1ull << g) - 1ull);
  const uint64_t below_r = (1ull << r) - 1ull;
  const int e0 = grp * S + r;
  uint32_t u[V];
  uint32_t vmask = 0;
  uint32_t nv = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = e0 + g * i;
    const bool v = e < n_valid;
    u[i] = v ? order_key(get(e)) : 0u;
    vmask |= (uint32_t)v << i;
    nv += popc64((__ballot(v) >> sh) & gm);
    if (v) {
      mn = min(mn, u[i]);
      mx = max(mx, u[i]);
    }
  }
  for (int o = 1; o < g; o <<= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  }
  const bool complete = nv <= (uint32_t)kRep;
  // per group: largest T with count(key >= T) >= kRep (invalid keys are 0
  // and every probe is >= 1); stops early on a probe with exactly kRep
  uint32_t lo = mn, hi = mx;
  bool done = complete || lo >= hi;
  while (__ballot(!done) != 0ull) {
    const uint32_t mid = lo + ((hi - lo) >> 1) + 1;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) c += popc64((__ballot(u[i] >= mid) >> sh) & gm);
    if (!done) {
      if (c == (uint32_t)kRep) {
        lo = mid;
        done = true;
      } else {
        if (c > (uint32_t)kRep) lo = mid; else hi = mid - 1;
        done = lo >= hi;
      }
    }
  }
  const uint32_t T = lo;
  uint32_t gt = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) gt += popc64((__ballot(((vmask >> i) & 1u) && u[i] > T) >> sh) & gm);
  const uint32_t need = (uint32_t)kRep - gt;  // copies of T kept, lowest positions first
  uint32_t sel = 0, seen = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool v = (vmask >> i) & 1u;
    const bool eq = v && u[i] == T;
    const uint64_t m = (__ballot(eq) >> sh) & gm;
    const bool si = complete ? v : ((v && u[i] > T) || (eq && seen + popc64(m & below_r) < need));
    sel |= (uint32_t)si << i;
    seen += popc64(m);
  }
  // compaction in position order; worst reported element per group
  const bool live = grp * S < n_valid;
  uint32_t base = 0, wu = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool si = (sel >> i) & 1u;
    const uint64_t m = (__ballot(si) >> sh) & gm;
    if (si && live) {
      const uint32_t pos = base + popc64(m & below_r);
      rep_u[grp * kRep + pos] = u[i];
      rep_j[grp * kRep + pos] = (int32_t)(j0 + e0 + g * i);
    }
    if (si) wu = min(wu, u[i]);
    base += popc64(m);
  }
  for (int o = 1; o < g; o <<= 1) wu = min(wu, (uint32_t)__shfl_xor((int)wu, o));
  int32_t wj = -1;
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (((sel >> i) & 1u) && u[i] == wu) wj = max(wj, (int32_t)(j0 + e0 + g * i));
  for (int o = 1; o < g; o <<= 1) wj = max(wj, __shfl_xor(wj, o));
  if (r == 0 && live) {
    RepHeader h;
    h.count = base;
    h.complete = complete ? 1u : 0u;
    h.worst_u = wu;
    h.worst_j = wj;
    hdr[grp] = h;
  }
}

}  // namespace dsa
