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
// The prefix a tile reports holds at least kRepMin elements and at most
// kRepMax; it is found with 8-bit radix passes over the order keys of the
// tile held in LDS, stopping as soon as the boundary digit fits.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int kRepMin = 16;
constexpr int kRepMax = 32;

struct RepHeader {
  uint32_t count;     // reported elements
  uint32_t complete;  // 1: every element of the tile is reported
  uint32_t worst_u;   // order key of the worst reported element
  int32_t worst_j;    // its position
};

// Scratch the report needs in LDS.
struct TileReportSmem {
  uint32_t hist[256];
  uint32_t scan[20];
  uint32_t st[8];
  uint64_t red[16];
};

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o);
    uint64_t t = ((uint64_t)hi << 32) | lo;
    v = t < v ? t : v;
  }
  return v;
}

// su[0..n) are the order keys of positions j0 .. j0+n-1.  Called by every
// thread of the block (blockDim.x a multiple of 64, at most 1024).
__device__ void tile_report(const uint32_t* su, int n, int64_t j0, TileReportSmem& sm,
                            RepHeader* hdr, uint32_t* rep_u, int32_t* rep_j) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (n <= kRepMax) {
    for (int i = tid; i < n; i += nt) {
      rep_u[i] = su[i];
      rep_j[i] = (int32_t)(j0 + i);
    }
    if (tid == 0) {
      RepHeader h;
      h.count = (uint32_t)n;
      h.complete = 1u;
      h.worst_u = 0u;
      h.worst_j = -1;
      *hdr = h;
    }
    return;
  }
  // --- radix passes: find the boundary of a prefix of kRepMin..kRepMax ---
  // st[0] = prefix digits so far, st[1] = count strictly above the bucket,
  // st[2] = done flag, st[3] = threshold key, st[4] = tie mode,
  // st[5] = tie count needed at the threshold key.
  if (tid == 0) {
    sm.st[0] = 0; sm.st[1] = 0; sm.st[2] = 0; sm.st[3] = 0; sm.st[4] = 0; sm.st[5] = 0;
  }
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += nt) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sm.st[0];
    for (int i = tid; i < n; i += nt) {
      uint32_t u = su[i];
      bool in = (shift == 24) || ((u >> (shift + 8)) == prefix);
      if (in) atomicAdd(&sm.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const int l = tid;
      uint32_t h0 = sm.hist[4 * l], h1 = sm.hist[4 * l + 1], h2 = sm.hist[4 * l + 2],
               h3 = sm.hist[4 * l + 3];
      uint32_t mine = h0 + h1 + h2 + h3;
      uint32_t inc = wave_incl_scan(mine);
      uint32_t tot = __shfl(inc, 63);
      uint32_t above = tot - inc;  // elements in digits above this lane's four
      const uint32_t base = sm.st[1];
      uint32_t hs[4] = {h0, h1, h2, h3};
      uint32_t gt = above;
      for (int k = 3; k >= 0; --k) {
        uint32_t d = 4 * l + k;
        uint32_t c_gt = base + gt;
        uint32_t c_ge = c_gt + hs[k];
        if (c_gt < (uint32_t)kRepMin && c_ge >= (uint32_t)kRepMin) {
          uint32_t key_prefix = (prefix << 8) | d;
          if (c_ge <= (uint32_t)kRepMax) {
            sm.st[2] = 1;
            sm.st[3] = key_prefix << shift;
          } else if (shift == 0) {
            sm.st[2] = 1;
            sm.st[3] = key_prefix;
            sm.st[4] = 1;
            sm.st[5] = (uint32_t)kRepMin - c_gt;
            sm.st[1] = c_gt;
          } else {
            sm.st[0] = key_prefix;
            sm.st[1] = c_gt;
          }
        }
        gt += hs[k];
      }
    }
    __syncthreads();
    if (sm.st[2]) break;
  }
  const uint32_t thr = sm.st[3];
  const bool tie = sm.st[4] != 0;
  const uint32_t need = sm.st[5];
  // --- compaction in position order (contiguous chunk per thread) ---
  const int per = (n + nt - 1) / nt;
  const int lo = tid * per, hi = min(n, lo + per);
  uint32_t tie_base = 0;
  if (tie) {
    uint32_t c = 0;
    for (int i = lo; i < hi; ++i) c += (su[i] == thr);
    uint32_t tot;
    tie_base = block_excl_scan(c, sm.scan, &tot);
  }
  uint32_t cnt = 0;
  {
    uint32_t tr = tie_base;
    for (int i = lo; i < hi; ++i) {
      uint32_t u = su[i];
      bool f = tie ? (u > thr || (u == thr && tr < need)) : (u >= thr);
      if (tie && u == thr) ++tr;
      cnt += f;
    }
  }
  uint32_t total;
  uint32_t pos = block_excl_scan(cnt, sm.scan, &total);
  uint64_t worst = ~0ull;
  {
    uint32_t tr = tie_base;
    for (int i = lo; i < hi; ++i) {
      uint32_t u = su[i];
      bool f = tie ? (u > thr || (u == thr && tr < need)) : (u >= thr);
      if (tie && u == thr) ++tr;
      if (f) {
        rep_u[pos] = u;
        rep_j[pos] = (int32_t)(j0 + i);
        ++pos;
        // selection order: larger key first, then lower position first
        uint64_t ord = ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)i);
        worst = ord < worst ? ord : worst;
      }
    }
  }
  worst = wave_min_u64(worst);
  if (lane_id() == 0) sm.red[wave_id()] = worst;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = ~0ull;
    for (int i = 0; i < (nt >> 6); ++i) m = sm.red[i] < m ? sm.red[i] : m;
    RepHeader h;
    h.count = total;
    h.complete = 0u;
    h.worst_u = (uint32_t)(m >> 32);
    h.worst_j = (int32_t)(j0 + (int64_t)(0xffffffffu - (uint32_t)m));
    *hdr = h;
  }
}

}  // namespace dsa
