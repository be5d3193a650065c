// dsa_topk.hip -- exact per-query Top-K of fp32 score rows.
//
// Selection ("Open-Source LLM Architecture Evolution ...", Architecture
// Breakdown, Top-K selection: each query goes on with only its K = 2048
// best-scoring past positions; ties, order and padding are the readings
// stated in dsa.h): K_eff = min(K, p+1) best positions by (score desc,
// position asc), -0.0 == +0.0, output ascending, padded with -1.
//
// Three kernels:
//   tile_report_kernel  one workgroup per (row, tile): loads the tile's
//                       scores, writes its candidate prefix (dsa_topk_tile.h).
//                       The decode indexer writes the same reports from its
//                       epilogue, so the layer path skips this kernel.
//   topk_resolve_kernel one workgroup per row: loads the reports (they come
//                       in ascending position order) into registers, finds
//                       the K_eff-th best candidate with radix passes over
//                       the candidates' key range and a directly ranked
//                       boundary bucket, certifies the union, and writes the
//                       selected positions in ascending order with a block
//                       prefix sum.  If certification fails, or the union
//                       does not fit the block, it runs an exact radix
//                       select over the whole score row from global memory.
//   topk_rows_kernel    calls with many rows (no reports): one workgroup per
//                       row collects the keys at or above a threshold (from
//                       a sample of the row, else from histogram sweeps) in
//                       position order and selects among them the same way.
#include <algorithm>

#include "dsa_attn_tile.h"
#include "dsa_kernels.h"
#include "dsa_topk_tile.h"

namespace dsa {

constexpr int kResolveTiles = 1024;                         // tiles in the fast path
constexpr int kResolveSlots = kResolveTiles * kRep;         // union capacity (16384)

template <int TILE>
__global__ __launch_bounds__(64) void tile_report_kernel(const float* __restrict__ scores,
                                                         int64_t ld, const int32_t* cu_q,
                                                         const int32_t* ctx_len, int B, int K,
                                                         int stride, RepHeader* hdr,
                                                         uint32_t* rep_u, int32_t* rep_j) {
  constexpr int V = TILE / 64;
  const int t = blockIdx.y, ti = blockIdx.x;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t j0 = (int64_t)ti * TILE;
  const int64_t nrow = ri.p + 1;
  if (j0 > ri.p || nrow <= kDirectMax) return;  // short rows are selected directly
  const int n = (int)min<int64_t>(TILE, nrow - j0);
  const float* row = scores + (int64_t)t * ld + j0;
  const int S = topk_subtile(nrow, K);  // <= TILE
  const int64_t slot = (int64_t)t * stride + (int64_t)ti * (TILE >> (31 - __clz(S)));
  if (S < TILE) {
    wave_subtile_reports<V>([&](int e) { return row[e]; }, n, j0, S, hdr + slot,
                            rep_u + slot * kRep, rep_j + slot * kRep);
    return;
  }
  const int l = lane_id();
  const int nv = min(max(n - V * l, 0), V);  // valid elements V l .. V l + nv - 1
  uint32_t uv[V];
#pragma unroll
  for (int i = 0; i < V; ++i) uv[i] = order_key(row[i < nv ? V * l + i : 0]);
  wave_tile_report<V>(uv, nv, j0 + V * l, hdr + slot, rep_u + slot * kRep, rep_j + slot * kRep);
}

// ---------------------------------------------------------------------------
// Radix select helpers for the resolve kernel (1024 threads, 2048 bins).
// ---------------------------------------------------------------------------
constexpr int kBucketMax = 64;  // boundary-bucket size ranked directly by wave 0

// An empty hook: nothing to issue or stage at the hook's point.
struct NoPost {
  __device__ void operator()() const {}
};

template <int NTILE>
struct ResolveSmemT {
  // two 2048-bin histograms (the union select alternates between them);
  // once the threshold is known, the staging area of up to 4096 outputs
  alignas(16) uint32_t hbuf[4096];
  __device__ uint32_t* hist() { return hbuf; }
  __device__ uint32_t* hist2() { return hbuf + 2048; }
  alignas(16) uint32_t bu[kBucketMax];
  alignas(16) int32_t bj[kBucketMax];
  // per sub-tile: worst reported (key, position | complete << 31), kept for
  // the certification so the headers need not stay in registers
  uint32_t wu[NTILE];
  uint32_t wj[NTILE];
  uint32_t red[64];
  uint32_t red0[48];  // count / min / max per wave, read only by the register path's first step
  uint32_t flag[16];
  uint32_t scan[32];  // excl_scan_active uses [0, 16); the ping-pong scan both halves
  uint32_t st[8];
};
using ResolveSmem = ResolveSmemT<kResolveTiles>;
using RowsSmem = ResolveSmemT<1>;  // no certification: no per-sub-tile words

// Wave 0 of the block: given the 2048-bin histogram h of the current
// bucket and `above` elements strictly above the bucket, find digit d with
// above + gt(d) < k <= above + gt(d) + h[d] (gt(d): elements in digits > d).
// Writes st[0] = d, st[1] = above + gt(d), st[5] = h[d].  Two levels of one
// wave scan each: the 64 chunks of 32 bins, then the 32 bins of the chunk
// that holds d.
template <class SM>
__device__ void wave_find_digit(SM& sm, const uint32_t* h, uint32_t above, uint32_t k) {
  const int l = lane_id();
  // level 1: lane l sums bins 32 l .. 32 l + 31 (chunk reads in a
  // lane-rotated order, so fewer lanes share a bank)
  uint32_t mine = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(h + 32 * l + 4 * ((c + l) & 7));
    mine += v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t incl = wave_incl_scan(mine);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint32_t gt = total - incl;  // elements in the bins of higher lanes
  const uint64_t m1 = __ballot(above + gt < k && above + gt + mine >= k);
  const int L = m1 ? __ffsll((long long)m1) - 1 : 0;  // the chunk holding the k-th
  const uint32_t base = above + (uint32_t)__builtin_amdgcn_readlane((int)gt, L);
  // level 2: lane i < 32 takes bin 32 L + i; elements in the chunk's higher
  // bins come from one more scan
  const uint32_t x = l < 32 ? h[32 * L + l] : 0u;
  const uint32_t incl2 = wave_incl_scan(x);
  const uint32_t gt2 = base + (uint32_t)__builtin_amdgcn_readlane((int)incl2, 31) - incl2;
  const bool hit = l < 32 && gt2 < k && gt2 + x >= k;
  if (hit) {
    sm.st[0] = 32 * L + l;
    sm.st[1] = gt2;
    sm.st[5] = x;
  }
}

// Register path of the resolve.  A candidate set in position order (the
// union of a row's sub-tile reports: slot s is slot s % kRep of sub-tile
// s / kRep; or, for a direct row, slot s is position s) is held q-major:
// group q of thread tid holds slots 4 nt q + 4 tid + e (e < 4, nt threads).
// The first qn groups of all threads therefore hold the first 4 nt qn slots,
// and every loop skips the groups at or beyond qn (block-uniform), so a short
// set costs no more than its size.  Loads are coalesced 16-byte loads;
// per-slot validity is a bitmask (bit 4q+e).
template <int NSL>
struct UnionRegs {
  uint32_t u[NSL];
  int32_t j[NSL];
  uint32_t vmask;  // bit i: slot i holds a candidate
  int qn;          // live groups
};

__device__ __forceinline__ int slot_of(int q, int tid, int nt) { return 4 * nt * q + 4 * tid; }

// Exclusive position-ordered prefix of per-slot flags (bitmask, bit 4q+e)
// over the live groups; returns each slot's rank among flagged slots and the
// total.  Also ORs the per-thread flag `bad` over the block into *any_bad
// (same exchange).  One cross-wave exchange of the per-(group, wave) counts
// (at most 64 of them: NSL/4 groups x nt/64 waves).  nt: active threads.
// Ends with a barrier (sm.red / sm.flag free again) unless tail_barrier is
// false.
template <int NSL, class SM>
__device__ __forceinline__ void ordered_ranks(SM& sm, uint32_t fmask, int qn, int nt,
                                              uint32_t (&rank)[NSL], uint32_t* total,
                                              bool bad = false, bool* any_bad = nullptr,
                                              bool tail_barrier = true) {
  static_assert((NSL / 4) * (kResolveSlots / NSL / 64) <= 64, "exchange size");
  const int l = lane_id(), wv = wave_id(), nw = nt >> 6;
  uint32_t lane_ex[NSL / 4];
#pragma unroll
  for (int q = 0; q < NSL / 4; ++q) {
    lane_ex[q] = 0;
    if (q < qn) {
      const uint32_t c = (uint32_t)__popc((fmask >> (4 * q)) & 15u);
      const uint32_t inc = wave_incl_scan(c);
      lane_ex[q] = inc - c;
      if (l == 63) sm.red[q * nw + wv] = inc;
    }
  }
  const bool wbad = __ballot(bad) != 0;
  if (l == 0) sm.flag[wv] = wbad ? 1u : 0u;
  lds_barrier();
  // (a wave with no slots needs neither the exchange's prefix nor its total)
  const uint32_t x = l < qn * nw ? sm.red[l] : 0u;
  const uint32_t xi = qn > 0 ? wave_incl_scan(x) : 0u;
  const uint32_t xe = xi - x;
  *total = (uint32_t)__builtin_amdgcn_readlane((int)xi, 63);
  if (any_bad) *any_bad = __ballot(l < nw && sm.flag[l] != 0u) != 0;
#pragma unroll
  for (int q = 0; q < NSL / 4; ++q) {
    uint32_t r = 0;
    if (q < qn) r = (uint32_t)__builtin_amdgcn_readlane((int)xe, q * nw + wv) + lane_ex[q];
    const uint32_t m = (fmask >> (4 * q)) & 15u;
    rank[4 * q + 0] = r;
    rank[4 * q + 1] = r + (m & 1u);
    rank[4 * q + 2] = r + __popc(m & 3u);
    rank[4 * q + 3] = r + __popc(m & 7u);
  }
  if (tail_barrier) lds_barrier();
}

// Appends the candidates with keys in [lo, lo + wm1] to sm.bu / sm.bj
// (in no particular order): a wave scan of the per-lane counts places each
// lane's candidates after those of the lanes below it, at a wave base taken
// with one LDS atomic (sm.st[4] counts the bucket; the caller guarantees at
// most kBucketMax).
template <int NSL, class SM>
__device__ __forceinline__ void gather_bucket(SM& sm, const UnionRegs<NSL>& R,
                                              uint32_t lo, uint32_t wm1) {
  if (R.qn == 0) return;  // a wave outside the selecting threads
  const int l = lane_id();
  uint32_t inb = 0;
#pragma unroll
  for (int i = 0; i < NSL; ++i)
    if (i / 4 < R.qn) inb |= (uint32_t)(R.u[i] - lo <= wm1) << i;  // wraps below lo
  inb &= R.vmask;
  const uint32_t c = (uint32_t)__popc(inb);
  const uint32_t inc = wave_incl_scan(c);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  if (wtot == 0) return;
  uint32_t base = 0;
  if (l == 0) base = atomicAdd(&sm.st[4], wtot);
  uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)base, 0) + inc - c;
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    if (i / 4 < R.qn && ((inb >> i) & 1u)) {
      sm.bu[pos] = R.u[i];
      sm.bj[pos] = R.j[i];
      ++pos;
    }
  }
}

// Finds the need-th best of the h <= kBucketMax gathered candidates under
// (key desc, position asc) and writes it to st[2] (key), st[3] (position).
// The nw waves share the work: lane i holds candidate i, and a wave takes
// candidates e = wave, wave + nw, ...; the rank of e is the ballot count of
// the lanes whose candidate beats it (ranks are distinct, so exactly one
// candidate has rank need - 1).  Called by the block; ends with a barrier.
template <class SM>
__device__ __forceinline__ void rank_bucket(SM& sm, uint32_t h, uint32_t need, int nw) {
  const int l = lane_id(), wv = wave_id();
  const bool mine_ok = (uint32_t)l < h;
  const uint32_t um = mine_ok ? sm.bu[l] : 0u;
  const int32_t jm = mine_ok ? sm.bj[l] : 0;
#pragma unroll 1
  for (int e = wv < nw ? wv : (int)h; e < (int)h; e += nw) {
    const uint32_t ue = sm.bu[e];
    const int32_t je = sm.bj[e];
    const uint64_t beats = __ballot(mine_ok && (um > ue || (um == ue && jm < je)));
    if (l == 0 && popc64(beats) == need - 1) {
      sm.st[2] = ue;
      sm.st[3] = (uint32_t)je;
    }
  }
  lds_barrier();
}

// Exact K-th best candidate of the set: selected <=> key > tau_u, or
// key == tau_u and position <= tau_j.  Radix digits (11, 11, 10 bits) are
// taken relative to the set's key range [mn, mx], so the first pass
// spreads the candidates over the 2048 bins instead of piling them onto the
// few bins the leading exponent bits would give.  Each pass is one LDS
// histogram and one wave-0 digit search (the other waves clear the other
// histogram meanwhile).  As soon as the boundary bucket holds at most
// kBucketMax candidates they are gathered and wave 0 ranks them directly
// under (key desc, position asc), which gives (tau_u, tau_j) at once.  Both
// histograms are zero and st[4] is 0 on entry.  nt: active threads.
template <int NSL, class SM>
__device__ __forceinline__ void union_threshold(SM& sm, const UnionRegs<NSL>& R,
                                                uint32_t k, uint32_t mn, uint32_t mx, int nt,
                                                uint32_t* tau_u, int32_t* tau_j) {
  const int tid = threadIdx.x, wv = wave_id();
  const uint32_t range = mx - mn;
  // bucket = keys in [lo, lo + wm1]; digits (key - lo) >> shift are < 2048.
  // A key below lo wraps to key - lo > wm1 (lo + wm1 never passes 2^32 - 1),
  // so one unsigned compare tests membership.
  int shift = range == 0 ? 0 : max(0, 32 - __clz(range) - 11);
  uint32_t lo = mn;
  uint32_t wm1 = range;
  uint32_t above = 0;  // candidates strictly above the bucket
  uint32_t h = 0;      // candidates in the bucket
  int pass = 0;
  while (true) {
    uint32_t* hc = (pass & 1) ? sm.hist2() : sm.hist();
    uint32_t* hn = (pass & 1) ? sm.hist() : sm.hist2();
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      if (i / 4 < R.qn) {
        const uint32_t x = R.u[i] - lo;
        if (((R.vmask >> i) & 1u) & (uint32_t)(x <= wm1)) atomicAdd(&hc[x >> shift], 1u);
      }
    }
    lds_barrier();
    if (wv == 0) {
      wave_find_digit(sm, hc, above, k);
      if (nt == 64)  // a single wave clears the next pass's histogram itself
        for (int i = tid; i < 2048; i += 64) hn[i] = 0;
    } else if (tid < nt) {
      for (int i = tid - 64; i < 2048; i += nt - 64) hn[i] = 0;  // next pass's histogram
    }
    lds_barrier();
    const uint32_t d = sm.st[0];
    above = sm.st[1];
    h = sm.st[5];
    const uint32_t off = d << shift;
    lo += off;
    wm1 = min(wm1 - off, (1u << shift) - 1u);
    if (shift == 0 || h <= (uint32_t)kBucketMax) break;
    shift = max(0, shift - 11);
    ++pass;
  }
  const uint32_t need = k - above;  // 1..h: the need-th best of the bucket is theta
  if (h <= (uint32_t)kBucketMax) {
    gather_bucket(sm, R, lo, wm1);
    lds_barrier();
    rank_bucket(sm, h, need, nt >> 6);
    *tau_u = sm.st[2];
    *tau_j = (int32_t)sm.st[3];
    return;
  }
  // more than kBucketMax candidates share the single key lo: the need
  // lowest positions among them are selected
  *tau_u = lo;
  uint32_t inb = 0;
#pragma unroll
  for (int i = 0; i < NSL; ++i)
    inb |= (uint32_t)(((R.vmask >> i) & 1u) && R.u[i] == lo) << i;
  uint32_t rk[NSL], tot;
  ordered_ranks<NSL>(sm, inb, R.qn, nt, rk, &tot);
  if (tid == 0) sm.st[3] = 0x7fffffffu;
  lds_barrier();
  if (need < tot) {
#pragma unroll
    for (int i = 0; i < NSL; ++i)
      if (((inb >> i) & 1u) && rk[i] == need - 1) sm.st[3] = (uint32_t)R.j[i];
  }
  lds_barrier();
  *tau_j = (int32_t)sm.st[3];
}

// Threshold, selection and coalesced store for a candidate set held in
// registers.  With ntiles > 0 the set is a report union and is certified
// against the sub-tile headers kept in sm.wu / sm.wj.  Returns false,
// leaving `out` untouched, when the set has fewer than k candidates or the
// certification fails.  On success the selection is also left in sm.hbuf
// (K words, rank order) and `out` may be null.  nt: active threads.  When
// the set holds at least k
// candidates, *theta (if given) receives the key of its k-th best and
// *has_theta is set, whether or not the certification holds; when the
// certification fails, *nbad (if given) receives the number of sub-tiles
// that failed it.  On success, every thread runs stage() right before the
// barrier that publishes the staged selection, so a caller's own LDS writes
// placed there are published by the same barrier.
template <int NSL, class SM, class Stage = NoPost>
__device__ __forceinline__ bool select_from_regs(SM& sm, const UnionRegs<NSL>& R,
                                                 uint32_t k, int K, int ntiles, int nt,
                                                 int32_t* out, uint32_t* theta = nullptr,
                                                 bool* has_theta = nullptr,
                                                 uint32_t* nbad = nullptr,
                                                 Stage stage_hook = Stage()) {
  const int tid = threadIdx.x, l = lane_id(), wv = wave_id();
  // candidate count and key range, in one block reduction; both histograms
  // are cleared meanwhile
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    if (i / 4 < R.qn) {
      const bool vi = (R.vmask >> i) & 1u;
      mn = min(mn, vi ? R.u[i] : 0xffffffffu);
      mx = max(mx, vi ? R.u[i] : 0u);
    }
  }
  if (wv < (nt >> 6)) {  // waves outside the selecting threads hold nothing
    const uint32_t cw = wave_sum_u32((uint32_t)__popc(R.vmask));
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (l == 0) {
      sm.red0[wv] = cw;
      sm.red0[16 + wv] = mn;
      sm.red0[32 + wv] = mx;
    }
  }
  for (int i = tid; i < 2048 && tid < nt; i += nt) {
    sm.hist()[i] = 0;
    sm.hist2()[i] = 0;
  }
  if (tid == 0) sm.st[4] = 0;
  lds_barrier();
  // red0 is written nowhere else, so no second barrier is needed before
  // the next step reuses the LDS
  uint32_t C;
  {
    const int nw = nt >> 6;
    C = wave_sum_u32(l < nw ? sm.red0[l] : 0u);
    mn = wave_min_u32(l < nw ? sm.red0[16 + l] : 0xffffffffu);
    mx = wave_max_u32(l < nw ? sm.red0[32 + l] : 0u);
  }
  if (C < k) return false;
  uint32_t tau_u;
  int32_t tau_j;
  union_threshold(sm, R, k, mn, mx, nt, &tau_u, &tau_j);
  if (theta) {
    *theta = tau_u;
    *has_theta = true;
  }
  // certification: every partly reported sub-tile ends at or below theta
  // (checked in the same block exchange as the ranks)
  bool bad = false;
  for (int ti = tid; ti < ntiles && tid < nt; ti += nt) {
    const uint32_t wu = sm.wu[ti], wj = sm.wj[ti];
    const bool complete = wj >> 31;
    const int32_t wpos = (int32_t)(wj & 0x7fffffffu);
    bad |= !complete && !((wu < tau_u) || (wu == tau_u && wpos >= tau_j));
  }
  // selection mask in bitwise form (no short-circuit branches per slot)
  uint32_t smask = 0;
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    if (i / 4 < R.qn) {
      const uint32_t si = (uint32_t)(R.u[i] > tau_u) |
                          ((uint32_t)(R.u[i] == tau_u) & (uint32_t)(R.j[i] <= tau_j));
      smask |= si << i;
    }
  }
  smask &= R.vmask;
  uint32_t rk[NSL], total;
  bool any_bad = false;
  // no tail barrier: the staging below touches neither sm.red nor sm.flag
  ordered_ranks<NSL>(sm, smask, R.qn, nt, rk, &total, bad, &any_bad, false);
  if (any_bad) {
    lds_barrier();  // the caller's exact select reuses sm.red
    if (nbad) {  // the failing sub-tiles, counted (this path only)
      uint32_t c = 0;
      for (int ti = tid; ti < ntiles && tid < nt; ti += nt) {
        const uint32_t wu = sm.wu[ti], wj = sm.wj[ti];
        const int32_t wpos = (int32_t)(wj & 0x7fffffffu);
        c += (!(wj >> 31) && !((wu < tau_u) || (wu == tau_u && wpos >= tau_j))) ? 1u : 0u;
      }
      c = wave_sum_u32(c);
      if (l == 0) sm.red[wv] = c;
      lds_barrier();
      *nbad = wave_sum_u32(l < (nt >> 6) ? sm.red[l] : 0u);
      lds_barrier();
    }
    return false;
  }
  // each selected slot's position goes to its rank in LDS (the histograms
  // are free once theta is known; K <= 4096 words), then the block writes
  // the K positions with coalesced 16-byte stores
  uint32_t* stage = sm.hbuf;
#pragma unroll
  for (int i = 0; i < NSL; ++i)
    if (i / 4 < R.qn && (((smask >> i) & 1u) & (uint32_t)(rk[i] < k)))
      stage[rk[i]] = (uint32_t)R.j[i];
  stage_hook();
  lds_barrier();
  if (out == nullptr) return true;  // the caller reads the selection from sm.hbuf
  if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    for (int i = tid; i < K / 4 && tid < nt; i += nt)
      *reinterpret_cast<u32x4*>(out + 4 * i) = *reinterpret_cast<const u32x4*>(stage + 4 * i);
  } else {
    for (int i = tid; i < K && tid < nt; i += nt) out[i] = (int32_t)stage[i];
  }
  return true;
}

// PER consecutive keys of a row from position p0 (a multiple of 4);
// returns the validity mask.  Same conditions as load_keys16.
template <int PER>
__device__ __forceinline__ uint32_t load_keys(const float* row, int64_t n, int64_t p0, bool vec,
                                              uint32_t (&u)[PER]) {
  static_assert(PER % 4 == 0 && PER <= 32, "keys per thread");
  uint32_t vm = 0;
#pragma unroll
  for (int c = 0; c < PER / 4; ++c) {
    const int64_t p = p0 + 4 * c;
    float f[4];
    if (vec) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + (p < n ? p : 0));
      f[0] = v[0];
      f[1] = v[1];
      f[2] = v[2];
      f[3] = v[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = row[p + e < n ? p + e : 0];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool v = p + e < n;
      u[4 * c + e] = v ? order_key(f[e]) : 0u;
      vm |= (uint32_t)v << (4 * c + e);
    }
  }
  return vm;
}

// Exclusive prefix sum of one value per thread over the nw active waves;
// *total receives the sum.  Contains barriers.
template <class SM>
__device__ __forceinline__ uint32_t excl_scan_active(SM& sm, uint32_t v, int nw,
                                                     uint32_t* total) {
  const int l = lane_id(), wv = wave_id();
  const uint32_t inc = wave_incl_scan(v);
  if (l == 63) sm.scan[wv] = inc;
  dma_barrier();  // LDS only: global loads in flight stay in flight
  const uint32_t x = l < nw ? sm.scan[l] : 0u;
  const uint32_t xi = wave_incl_scan(x);
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(xi - x), wv);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)xi, 63);
  dma_barrier();
  return base + inc - v;
}

// The same with one barrier: calls alternate between two halves of
// sm.scan (parity), so a call's writes cannot meet the previous call's
// reads (every wave passed that call's barrier only after its reads).
// Every wave sums the wave totals below it itself.  nw <= 16.
template <class SM>
__device__ __forceinline__ uint32_t excl_scan_pingpong(SM& sm, uint32_t v, int nw, uint32_t parity,
                                                       uint32_t* total) {
  const int l = lane_id(), wv = wave_id();
  uint32_t* buf = sm.scan + 16 * (parity & 1u);
  const uint32_t inc = wave_incl_scan(v);
  if (l == 63) buf[wv] = inc;
  dma_barrier();  // LDS only: global loads in flight stay in flight
  const uint32_t x = l < nw ? buf[l] : 0u;
  const uint32_t xi = wave_incl_scan(x);
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(xi - x), wv);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)xi, 63);
  return base + inc - v;
}

// Sixteen consecutive keys of a row from position p0 (a multiple of 16);
// returns the validity mask.  `vec`: the row is 16-byte aligned and its
// stride a multiple of four, so 16-byte loads below n stay inside it.
__device__ __forceinline__ uint32_t load_keys16(const float* row, int64_t n, int64_t p0, bool vec,
                                                uint32_t (&u)[16]) {
  uint32_t vm = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t p = p0 + 4 * c;
    float f[4];
    if (vec) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + (p < n ? p : 0));
      f[0] = v[0];
      f[1] = v[1];
      f[2] = v[2];
      f[3] = v[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = row[p + e < n ? p + e : 0];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool v = p + e < n;
      u[4 * c + e] = v ? order_key(f[e]) : 0u;
      vm |= (uint32_t)v << (4 * c + e);
    }
  }
  return vm;
}

// Exact Top-k of a whole score row from global memory, for rows the
// register paths cannot take (a failed certification, too many sub-tiles).
// Compact code: each sweep is a rolled loop over chunks of 16 consecutive
// positions per thread.  One sweep for the key range, range-relative radix
// histograms (11 bits per sweep) until the boundary bucket holds at most
// kBucketMax keys or a single key; the bucket is gathered and ranked
// directly (or, for one key shared by many positions, its need lowest
// positions are found with ordered block scans); a last ordered sweep
// writes the selected positions in ascending order.
template <class SM>
__device__ __forceinline__ void exact_select_row(SM& sm, const float* row, int64_t n,
                                                 uint32_t k, bool vec, int nt, int32_t* out,
                                                 bool stage = false) {
  const int tid = threadIdx.x, l = lane_id(), wv = wave_id(), nw = nt >> 6;
  const int64_t step = 16 * (int64_t)nt;
  uint32_t u[16];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll 1
  for (int64_t b0 = 0; b0 < n; b0 += step) {
    const uint32_t vm = load_keys16(row, n, b0 + 16 * tid, vec, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool v = (vm >> i) & 1u;
      mn = min(mn, v ? u[i] : 0xffffffffu);
      mx = max(mx, v ? u[i] : 0u);
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (l == 0) {
    sm.red[16 + wv] = mn;
    sm.red[32 + wv] = mx;
  }
  for (int i = tid; i < 2048; i += nt) sm.hist()[i] = 0;
  if (tid == 0) sm.st[4] = 0;
  lds_barrier();
  mn = wave_min_u32(l < nw ? sm.red[16 + l] : 0xffffffffu);
  mx = wave_max_u32(l < nw ? sm.red[32 + l] : 0u);
  const uint32_t range = mx - mn;
  int shift = range == 0 ? 0 : max(0, 32 - __clz(range) - 11);
  uint32_t lo = mn;
  uint32_t wm1 = range;  // bucket [lo, lo + wm1]; keys below lo wrap past wm1
  uint32_t above = 0, h = 0;
#pragma unroll 1
  while (true) {
#pragma unroll 1
    for (int64_t b0 = 0; b0 < n; b0 += step) {
      const uint32_t vm = load_keys16(row, n, b0 + 16 * tid, vec, u);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t x = u[i] - lo;
        if (((vm >> i) & 1u) & (uint32_t)(x <= wm1)) atomicAdd(&sm.hist()[x >> shift], 1u);
      }
    }
    lds_barrier();
    if (wv == 0) wave_find_digit(sm, sm.hist(), above, k);
    lds_barrier();
    const uint32_t d = sm.st[0];
    above = sm.st[1];
    h = sm.st[5];
    const uint32_t off = d << shift;
    lo += off;
    wm1 = min(wm1 - off, (1u << shift) - 1u);
    if (shift == 0 || h <= (uint32_t)kBucketMax) break;
    shift = max(0, shift - 11);
    for (int i = tid; i < 2048; i += nt) sm.hist()[i] = 0;
    lds_barrier();
  }
  const uint32_t need = k - above;  // 1..h
  uint32_t tau_u;
  int32_t tau_j;
  if (h <= (uint32_t)kBucketMax) {
#pragma unroll 1
    for (int64_t b0 = 0; b0 < n; b0 += step) {
      const int64_t p0 = b0 + 16 * tid;
      const uint32_t vm = load_keys16(row, n, p0, vec, u);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (((vm >> i) & 1u) & (uint32_t)(u[i] - lo <= wm1)) {
          const uint32_t pos = atomicAdd(&sm.st[4], 1u);
          sm.bu[pos] = u[i];
          sm.bj[pos] = (int32_t)(p0 + i);
        }
    }
    lds_barrier();
    rank_bucket(sm, h, need, nw);
    tau_u = sm.st[2];
    tau_j = (int32_t)sm.st[3];
  } else {
    // one key shared by more than kBucketMax positions: its need lowest
    tau_u = lo;
    if (tid == 0) sm.st[3] = 0x7fffffffu;
    uint32_t cum = 0;
#pragma unroll 1
    for (int64_t b0 = 0; b0 < n && cum < need; b0 += step) {
      const int64_t p0 = b0 + 16 * tid;
      const uint32_t vm = load_keys16(row, n, p0, vec, u);
      uint32_t f = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) f |= (uint32_t)(((vm >> i) & 1u) && u[i] == lo) << i;
      uint32_t tot;
      uint32_t r = cum + excl_scan_active(sm, (uint32_t)__popc(f), nw, &tot);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((f >> i) & 1u) {
          if (r == need - 1) sm.st[3] = (uint32_t)(p0 + i);
          ++r;
        }
      cum += tot;
    }
    lds_barrier();
    tau_j = (int32_t)sm.st[3];
  }
  uint32_t cum = 0;
#pragma unroll 1
  for (int64_t b0 = 0; b0 < n && cum < k; b0 += step) {
    const int64_t p0 = b0 + 16 * tid;
    const uint32_t vm = load_keys16(row, n, p0, vec, u);
    uint32_t f = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      f |= (uint32_t)(((vm >> i) & 1u) &&
                      ((u[i] > tau_u) || (u[i] == tau_u && (int32_t)(p0 + i) <= tau_j)))
           << i;
    uint32_t tot;
    uint32_t r = cum + excl_scan_active(sm, (uint32_t)__popc(f), nw, &tot);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((f >> i) & 1u) {
        if (r < k) {
          if (out) out[r] = (int32_t)(p0 + i);
          if (stage) sm.hbuf[r] = (uint32_t)(p0 + i);  // the histograms are done with
        }
        ++r;
      }
    cum += tot;
  }
}

// Ordered collection of every key of a row at or above `lo` into cu / cj
// (position order, the first `cap` of them; the rest are only counted):
// rounds of 8 consecutive keys per thread, the next round's loads in
// flight while the current one is ranked with a block prefix sum.  Stops
// once more than `cap` keys were seen; returns the count (block-uniform).
template <class SM>
__device__ uint32_t collect_keys_at_least(SM& sm, const float* row, int64_t n, bool vec,
                                          uint32_t lo, uint32_t* cu, int32_t* cj, uint32_t cap,
                                          int nt) {
  constexpr int PER = 8;
  const int tid = threadIdx.x, nw = nt >> 6;
  const int64_t step = PER * (int64_t)nt;
  uint32_t ua[PER], ub[PER];
  uint32_t cum = 0, par = 0;
  auto rank = [&](const uint32_t(&u)[PER], uint32_t vm, int64_t p0) {
    uint32_t f = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) f |= (uint32_t)(u[i] >= lo) << i;
    f &= vm;
    uint32_t tot;
    uint32_t r = cum + excl_scan_pingpong(sm, (uint32_t)__popc(f), nw, par++, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((f >> i) & 1u) {
        if (r < cap) {
          cu[r] = u[i];
          cj[r] = (int32_t)(p0 + i);
        }
        ++r;
      }
    cum += tot;
  };
  uint32_t va = load_keys<PER>(row, n, PER * tid, vec, ua);
#pragma unroll 1
  for (int64_t b0 = 0; b0 < n && cum <= cap; b0 += 2 * step) {
    const uint32_t vb = load_keys<PER>(row, n, b0 + step + PER * tid, vec, ub);
    rank(ua, va, b0 + PER * tid);
    if (b0 + step >= n || cum > cap) break;
    va = load_keys<PER>(row, n, b0 + 2 * step + PER * tid, vec, ua);
    rank(ub, vb, b0 + step + PER * tid);
  }
  lds_barrier();  // the collected keys are in LDS; sm.scan is free again
  return cum;
}

constexpr int kRefineCap = 4096;  // keys a failed union's second chance collects

// The second chance of a report union that failed its certification: every
// key of the row at or above theta (the union's K-th best, at most the
// row's) collected in one ordered sweep and, if they fit, the K best of
// them selected by the register path.  Returns false if they do not fit.
// Its register path holds 4 slots per thread (4096 keys in a block of
// 1024 threads), so that it needs fewer registers than the union's path
// and leaves the resolve's register allocation as it is.
__device__ __forceinline__ bool resolve_by_collection(ResolveSmem& sm, const float* row,
                                                      int64_t n, bool vec, uint32_t theta,
                                                      uint32_t k, int K, int nt, int32_t* out) {
  constexpr int NSL = 4, QN = 1;
  __shared__ uint32_t fb_u[kRefineCap];
  __shared__ int32_t fb_j[kRefineCap];
  const int tid = threadIdx.x;
  const uint32_t cap = min((uint32_t)kRefineCap, (uint32_t)(nt * NSL));
  const uint32_t C = collect_keys_at_least(sm, row, n, vec, theta, fb_u, fb_j, cap, nt);
  if (C > cap) return false;  // k <= C: the union's top K are among them
  UnionRegs<NSL> R;
  R.vmask = 0;
  R.qn = (int)((C + 4 * nt - 1) / (4 * nt));
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int s0 = slot_of(q, tid, nt);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool v = (uint32_t)(s0 + e) < C;
      R.u[4 * q + e] = v ? fb_u[s0 + e] : 0u;
      R.j[4 * q + e] = v ? fb_j[s0 + e] : 0;
      R.vmask |= (uint32_t)v << (4 * q + e);
    }
  }
  return select_from_regs(sm, R, k, K, 0, nt, out);  // C >= k: always succeeds
}

// One workgroup per row.  Rows of at most kDirectMax positions are selected
// from their scores directly; longer rows from the union of their sub-tile
// reports, certified; anything else (a failed certification, more
// sub-tiles than the block holds) by the exact select over the row.
//
// A failed certification still leaves a bound: the union is part of the
// row, so its K-th best key theta is at most the row's K-th best, and every
// key of the row's top K is at or above theta.  Such a row first collects
// the keys at or above theta in one ordered sweep; when they fit (a few
// sub-tiles that held more than 16 winners add at most S - 16 keys each)
// the K best of them are the row's, found by the same register path.  Only
// rows whose collection overflows take the exact select.
//
// The block is sized for the most slots any row may need; a row that needs
// fewer threads lets the surplus waves exit before the first barrier (a
// barrier waits only for the waves still running), so it pays for the
// threads it uses.  The first eager_q groups of report loads, laid out for
// eager_nt threads (the layout a row of max_ctx positions uses), are issued
// before the row's length is known: one round trip for the common case at
// small batch.  A row that needs another layout or more groups loads them
// after.
//
// ALL (phase one of the fused selection + attention kernel): every thread
// of the block stays to the end (nt is the whole block on every path), the
// selection is always left in sm.hbuf (K words in rank order, -1 past
// K_eff) and idx may be null (then only sm.hbuf receives it).
// QE > 0: the report groups loaded before the row length is known are
// exactly the first QE (a compile-time count, so no load is issued for the
// others); QE = 0: the first eager_q, with the others reading slot 0.
// post() runs once per thread when the row's candidates (or its scores) are
// in registers, before the selection's first exchange: a caller's own loads
// issued there queue behind the candidates' instead of ahead of them, and
// are in flight during the selection.  stage() runs before the barrier that
// publishes the selection when the register path succeeds at once (the
// usual case); returns whether it ran (block-uniform).
template <int NSL, bool ALL, int QE = 0, class Post = NoPost, class Stage = NoPost>
__device__ __forceinline__ bool resolve_row(
    ResolveSmem& sm, int t, const float* __restrict__ scores, int64_t ld, const int32_t* cu_q,
    const int32_t* ctx_len, int B, int K, int stride, int eager_nt, int eager_q,
    const RepHeader* __restrict__ hdr, const uint32_t* __restrict__ rep_u,
    const int32_t* __restrict__ rep_j, int32_t* idx, uint32_t* stats, Post post = Post(),
    Stage stage_hook = Stage()) {
  constexpr int QN = NSL / 4;
  const int tid = threadIdx.x, nb = blockDim.x;
  const int64_t slot0 = (int64_t)t * stride;
  const int nslots = min(stride, kResolveTiles) * kRep;  // a row's slots in the workspace
  UnionRegs<NSL> R;
  // one dword of the sub-tile header per thread: the four threads of a
  // sub-tile's slots are four consecutive lanes (4 slots each), lane l
  // loads dword l % 4 (count, complete, worst key, worst position) and the
  // quad shares them with DPP (a quarter of the bytes of whole headers)
  uint32_t hw[QN];
  const uint32_t* hdr32 = reinterpret_cast<const uint32_t*>(hdr);
  // eager report loads in the layout of nt threads: every group is loaded,
  // groups at or beyond qe from slot 0 (a cached line), so the loads are
  // straight-line code and all go out before the first wait (loads under
  // per-group branches would each wait at the join)
  auto load_eager = [&](int qe, int nt) {
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      if (QE > 0 && q >= QE) continue;
      const int sidx = slot_of(q, tid, nt);
      const int sc = ((QE > 0 || q < qe) && sidx < nslots) ? sidx : 0;
      const u32x4 a = *reinterpret_cast<const u32x4*>(rep_u + slot0 * kRep + sc);
      const u32x4 c = *reinterpret_cast<const u32x4*>(rep_j + slot0 * kRep + sc);
      hw[q] = hdr32[(slot0 + sc / kRep) * 4 + (tid & 3)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        R.u[4 * q + e] = a[e];
        R.j[4 * q + e] = (int32_t)c[e];
      }
    }
  };
  // report loads of groups [q0, q1) in the layout of nt threads, keeping
  // the other groups: slots, positions and sub-tile headers
  auto load_reports = [&](int q0, int q1, int nt) {
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      if (q >= q0 && q < q1) {
        const int sidx = slot_of(q, tid, nt);
        const int sc = sidx < nslots ? sidx : 0;
        const u32x4 a = *reinterpret_cast<const u32x4*>(rep_u + slot0 * kRep + sc);
        const u32x4 c = *reinterpret_cast<const u32x4*>(rep_j + slot0 * kRep + sc);
        hw[q] = hdr32[(slot0 + sc / kRep) * 4 + (tid & 3)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          R.u[4 * q + e] = a[e];
          R.j[4 * q + e] = (int32_t)c[e];
        }
      }
    }
  };
  if (eager_q > 0 && tid < eager_nt) load_eager(eager_q, eager_nt);
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t n = ri.p + 1;
  int32_t* out = idx ? idx + (int64_t)t * K : nullptr;
  if (n <= K) {
    post();
    for (int i = tid; i < K; i += nb) {
      const int32_t v = i < n ? i : -1;
      if (out) out[i] = v;
      if (ALL) sm.hbuf[i] = (uint32_t)v;
    }
    return false;
  }
  const uint32_t k = (uint32_t)K;
  const float* row = scores + (int64_t)t * ld;
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  // threads (whole waves) for a set of `slots` candidates
  auto threads_for = [&](int64_t slots) {
    const int64_t w = (slots + 64 * NSL - 1) / (64 * NSL);
    return (int)min<int64_t>(nb, 64 * max<int64_t>(w, 1));
  };
  int path = -1;   // counter index of the register path taken: 0 union, 2 direct
  int ntiles = 0;  // sub-tiles to certify (union path)
  int sub_s = 0;   // their size
  int nt = nb;     // active threads
  R.vmask = 0;
  if (n <= kDirectMax && n <= (int64_t)nb * NSL) {
    // ---- direct: slot s holds position s ----
    nt = ALL ? nb : threads_for(n);
    if (tid >= nt) return false;
    R.qn = (int)((n + 4 * nt - 1) / (4 * nt));
    // every group is loaded (straight-line loads, one round trip); groups
    // past the row read position 0 and are invalid
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int p = slot_of(q, tid, nt);
      float f[4];
      if (vec) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + (p < n ? p : 0));
        f[0] = v[0];
        f[1] = v[1];
        f[2] = v[2];
        f[3] = v[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = row[p + e < n ? p + e : 0];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v = p + e < n;
        R.u[4 * q + e] = v ? order_key(f[e]) : 0u;
        R.j[4 * q + e] = p + e;
        R.vmask |= (uint32_t)v << (4 * q + e);
      }
    }
    path = 2;
  } else {
    const int S = topk_subtile(n, K);
    sub_s = S;
    const int nt_row = (int)((n + S - 1) >> (31 - __clz(S)));  // S: a power of two
    if (nt_row <= kResolveTiles && nt_row <= stride && nt_row * kRep <= nb * NSL) {
      // ALL: the first eager_nt threads select when the union fits them
      // (the others stay for the caller, with no slots: they take part in
      // the selection's barriers only); otherwise the whole block
      nt = ALL ? (nt_row * kRep <= eager_nt * NSL ? eager_nt : nb)
               : max(threads_for((int64_t)nt_row * kRep), eager_nt);
      if (!ALL && tid >= nt) return false;
      R.qn = tid < nt ? (nt_row * kRep + 4 * nt - 1) / (4 * nt) : 0;
      if (nt != eager_nt || eager_q == 0)
        load_reports(0, R.qn, nt);  // another layout: load every group
      else if (R.qn > eager_q)
        load_reports(eager_q, R.qn, nt);
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        if (q < R.qn) {
          const int sidx = slot_of(q, tid, nt);
          const bool tile_ok = sidx / kRep < nt_row;
          const uint32_t sub = (uint32_t)(sidx % kRep);
          // the sub-tile's header from its quad (every lane of the quad
          // runs this: the group test is block-uniform)
          const uint32_t cnt = quad_bcast<0>(hw[q]);
          const uint32_t hcomplete = quad_bcast<1>(hw[q]);
          const uint32_t hworst_u = quad_bcast<2>(hw[q]);
          const uint32_t hworst_j = quad_bcast<3>(hw[q]);
          // slots sub .. sub+3 of the sub-tile are valid while below its count
          const uint32_t nv = tile_ok ? (cnt > sub ? min(cnt - sub, 4u) : 0u) : 0u;
          R.vmask |= ((1u << nv) - 1u) << (4 * q);
          if (sub == 0 && tile_ok) {
            sm.wu[sidx / kRep] = hworst_u;
            sm.wj[sidx / kRep] = hworst_j | (hcomplete ? 0x80000000u : 0u);
          }
        }
      }
      path = 0;
      ntiles = nt_row;
    }
  }
  post();
  bool ok = false;
  uint32_t theta = 0, nbad = 0;
  bool has_theta = false;
  if (path >= 0) {
    ok = select_from_regs(sm, R, k, K, ntiles, nt, out, &theta, &has_theta, &nbad, stage_hook);
    if (ok && stats && tid == 0) atomicAdd(&stats[path], 1u);
  }
  const bool staged = ok;
  // A report union that failed its certification bounds the row: its keys
  // at or above theta are at most K plus the failing sub-tiles' left-out
  // elements (S - 16 each, ties at theta aside); the second chance is tried
  // when that bound fits its slots.
  const int nt_fb = ALL ? nb : nt;  // the fallbacks take every thread left
  const bool bounded =
      !ok && path == 0 && has_theta &&
      (uint64_t)K + (uint64_t)nbad * (uint64_t)(sub_s - kRep) <=
          (uint64_t)min(kRefineCap, nt_fb * 4);
  if (bounded) {
    ok = resolve_by_collection(sm, row, n, vec, theta, k, K, nt_fb, out);
    if (ok && stats && tid == 0) atomicAdd(&stats[5], 1u);
  }
  if (!ok) {
    exact_select_row(sm, row, n, k, vec, nt_fb, out, ALL);
    if (stats && tid == 0) atomicAdd(&stats[1], 1u);
  }
  return staged;
}

template <int NSL>
__global__ __launch_bounds__(kResolveSlots / NSL) void topk_resolve_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
    int B, int K, int stride, int eager_nt, int eager_q, const RepHeader* __restrict__ hdr,
    const uint32_t* __restrict__ rep_u, const int32_t* __restrict__ rep_j, int32_t* idx,
    uint32_t* stats) {
  __shared__ ResolveSmem sm;
  resolve_row<NSL, false>(sm, blockIdx.x, scores, ld, cu_q, ctx_len, B, K, stride, eager_nt,
                          eager_q, hdr, rep_u, rep_j, idx, stats);
}

// ---------------------------------------------------------------------------
// Decode: selection and split attention in one launch
// ---------------------------------------------------------------------------
// At decode the Top-K resolve (one workgroup per row) and the split
// attention (nsplit workgroups per row, 64 selected rows each) would be two
// dependent launches, and the attention's first step a round trip for its
// part of the index row.  Here each of a row's nsplit workgroups (1024
// threads) first runs the whole selection of the row (resolve_row, ALL
// mode: the same exact result in every workgroup; split 0 also writes the
// row to idx) and then attends over ranks 64 s .. 64 s + 63 of it, read
// from its own LDS.  All 16 waves gather; the attention math runs on 8:
//   wave w < 8: row block rb = w & 1 (selected rows 32 rb .. + 31 of the
//   split), head block hb = (w >> 1) & 1 (heads 32 hb .. + 31), output dim
//   half dh = w >> 2 (dims 64 dh .. + 63).  Waves w and w + 4 share a SIMD
//   (waves go to the SIMDs in turn) and the same (rb, hb);
//   - the split's K and V rows are gathered once, two 1 KiB loads per wave
//     of all 16, into the swizzled row tiles (RowTile); waves 8..15 then
//     exit;
//   - S^T = K_rb . q_hb^T (v_mfma_f32_32x32x16_bf16, 8 k-steps) is computed
//     alike by the two dim-half waves of (rb, hb), so no exchange comes
//     before the softmax (with four dim-quarter waves per (rb, hb) each
//     SIMD's matrix pipe computed the same S four times);
//   - softmax over the row block (each lane holds one head: max and sum
//     take one cross-half exchange); P^T is the B operand of O^T = V^T . P^T
//     for the wave's 64 dims (four MFMAs, V^T through the transpose read);
//   - the rb = 1 waves hand (m, l, O) to their rb = 0 partners through LDS,
//     which merge them and write the split's partial (m, l, O) in the
//     layout of the split attention kernel, merged by the combine kernel.
// Ranks at or past K_eff (-1) are masked; an entry outside [0, p] cannot
// come out of the selection but would be masked the same way, so no gather
// leaves the sequence.
constexpr int kSaThreads = 1024;
constexpr int kSaRows = 64;  // selected rows per split
constexpr int kSaDimBlocks = 2;  // 32-dim output blocks per attention wave (2 or 4)
constexpr int kSaMathWaves = 16 / kSaDimBlocks;  // waves that run the attention math

template <int QE>
__global__ __launch_bounds__(kSaThreads) void select_attend_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ ctx_len, int B,
    int K, int stride, int eager_q, const RepHeader* __restrict__ hdr,
    const uint32_t* __restrict__ rep_u, const int32_t* __restrict__ rep_j, int32_t* idx,
    uint32_t* stats, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int64_t* __restrict__ cu_ctx, float scale_log2,
    float* __restrict__ part, int nsplit, int sel_nt) {
  constexpr int NSL = 16, D = 128, HQ = 64, KS = D / 16;
  using VT = RowTile<D>;
  __shared__ ResolveSmem sm;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4 * VT::kBytes];  // K rb 0, 1; V rb 0, 1
  constexpr int DB = kSaDimBlocks, NMW = kSaMathWaves;
  // (m, l, O) of the rb = 1 waves, per (hb, dh)
  __shared__ float mrg[NMW / 2 * (2 + 16 * DB) * 64];
  // the query's 64 heads, chunk c of head h at 16 (c ^ (h % 16)): the B
  // operand reads (16 heads, one chunk) hit 16 distinct 16-byte slots
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[HQ * D * 2];
  const int t = blockIdx.y, split = blockIdx.x;
  const int l = lane_id(), g = l >> 5, wv = wave_id();
  // wave w loads heads 4 w .. 4 w + 3 (one 1 KiB load, lane: head 4 w + l / 16,
  // chunk l % 16) once its report candidates are in registers, so that the
  // load is in flight during the selection without delaying the reports
  // (0.3 us less per 128K decode step than issuing it first); it goes to
  // LDS at the end of the selection, published by the barrier that
  // publishes the selection
  const int qh = 4 * wv + (l >> 4), qc = l & 15;
  u32x4 qv;
  auto put_q = [&]() {
    *reinterpret_cast<u32x4*>(q_lds + qh * (2 * D) + ((qc ^ (qh & 15)) << 4)) = qv;
  };
  const bool q_put = resolve_row<NSL, true, QE>(
      sm, t, scores, ld, nullptr, ctx_len, B, K, stride, sel_nt, eager_q, hdr, rep_u, rep_j,
      split == 0 ? idx : nullptr, split == 0 ? stats : nullptr,
      [&]() { qv = ld16(q + ((int64_t)t * HQ + qh) * D + 8 * qc); }, put_q);
  if (!q_put) {
    // the selection took another path: the query heads, and the selection
    // itself, are published here
    put_q();
    dma_barrier();
  }
  // the selection is in sm.hbuf (rank order, -1 past K_eff); split 0's
  // stores of it to idx stay in flight

  const int rb = wv & 1, hb = (wv >> 1) & 1, dh = (wv >> 2) & (NMW / 4 - 1);
  const int64_t p = (int64_t)ctx_len[t] - 1;
  const int64_t row0 = cu_ctx[t];
  const uint32_t jmax = (uint32_t)min<int64_t>(p, (int64_t)INT32_MAX);
  const int e0 = kSaRows * split;  // first rank of this split
  auto sel = [&](int r) -> uint32_t {  // selected position of split row r, or ~0
    const int e = e0 + r;
    return e < K ? sm.hbuf[e] : 0xffffffffu;
  };
  bf16x8 qb[KS];
  // gathers: wave w fills tile w >> 2 (0, 1: K rows of row blocks 0, 1;
  // 2, 3: V rows), its load instructions c = 2 (w & 3) and 2 (w & 3) + 1:
  // tile rows kRPI c + l / kNC, chunk l % kNC; invalid rows read row 0
  {
    const int tl = wv >> 2, trb = tl & 1;
    const int gch = l % VT::kNC, grow = l / VT::kNC;
    const uint16_t* base = (tl < 2 ? kc : vc) + row0 * D + 8 * gch;
    u32x4 v[2];
    int rr[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int r = VT::kRPI * (2 * (wv & 3) + c2) + grow;
      const uint32_t j = sel(32 * trb + r);
      v[c2] = ld16(base + (int64_t)(j <= jmax ? j : 0u) * D);
      rr[c2] = r;
    }
    // q heads of the wave's head block from LDS while the gathers are in
    // flight (B operand of S^T: column = head 32 hb + l % 32, k = dims
    // 16 s + 8 g .. + 7); the gather-only waves skip them
    const int h = 32 * hb + (l & 31);
    if (wv < NMW) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(q_lds + h * (2 * D) +
                                                          (((2 * s + g) ^ (h & 15)) << 4)));
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      *reinterpret_cast<u32x4*>(tiles + tl * VT::kBytes + VT::offset(rr[c2], 8 * gch)) = v[c2];
  }
  // bit r: selected row 32 rb + r is valid (lanes 32..63 repeat 0..31)
  const uint32_t vmask = (uint32_t)__ballot(sel(32 * rb + (l & 31)) <= jmax);
  dma_barrier();  // the tiles are complete
  if (wv >= NMW) return;  // the later barrier waits for the math waves left

  // S^T = K . q^T: the A operand of k-step s is tile row l % 32, dims 16 s + 8 g .. + 7
  f32x16 sacc = {};
  {
    const uint8_t* kt = tiles + rb * VT::kBytes;
    u32x4 kf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[s] = *reinterpret_cast<const u32x4*>(kt + VT::offset(l & 31, 16 * s + 8 * g));
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = mfma32(as_bf16x8(kf[s]), qb[s], sacc);
  }
  // softmax of the row block per head (exp2 domain, c > 0)
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int ir = 8 * (r >> 2) + 4 * g + (r & 3);
    if (!((vmask >> ir) & 1u)) sacc[r] = -INFINITY;
    mx = fmaxf(mx, sacc[r]);
  }
  const float m = xor32_max(mx) * scale_log2;
  const float mu = (m == -INFINITY) ? 0.f : m;
  float sv[16];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sv[r] = fexp2(fmaf(sacc[r], scale_log2, -mu));
    psum += sv[r];
  }
  const float lsum = xor32_add(psum);
  bf16x8 pb[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[s2][e] = static_cast<__bf16>(sv[8 * s2 + e]);
  // O^T = V^T . P^T for dims 64 dh .. + 63, as two 32-dim blocks dqq: k slot
  // e of step s2 is accumulator row 16 s2 + 8 (e / 4) + 4 g + e % 4, whose
  // two 4-row groups each come from one transpose read (lane jj of a
  // 16-lane group addresses row k0 + jj / 4, dims n0 + 4 (jj % 4) .. + 3)
  f32x16 o[DB] = {};
  {
    const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(tiles + (2 + rb) * VT::kBytes);
    const int G = l >> 4, jj = l & 15;
#pragma unroll
    for (int d2 = 0; d2 < DB; ++d2) {
      const int n0 = 32 * (DB * dh + d2) + 16 * (G & 1) + 4 * (jj & 3);
      u32x2 av[2][2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int k0 = 16 * s2 + 4 * g + (jj >> 2);
        av[s2][0] = lds_read_tr16(vt16 + VT::offset(k0, n0) / 2);
        av[s2][1] = lds_read_tr16(vt16 + VT::offset(k0 + 8, n0) / 2);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        o[d2] = mfma32(
            as_bf16x8(u32x4{av[s2][0][0], av[s2][0][1], av[s2][1][0], av[s2][1][1]}), pb[s2],
            o[d2]);
    }
  }
  // merge the two row blocks: rb = 1 hands over, rb = 0 writes the partial
  float* ms = mrg + (hb * (NMW / 4) + dh) * (2 + 16 * DB) * 64;
  if (rb == 1) {
    ms[l] = m;
    ms[64 + l] = lsum;
#pragma unroll
    for (int d2 = 0; d2 < DB; ++d2)
#pragma unroll
      for (int r = 0; r < 16; ++r) ms[(2 + 16 * d2 + r) * 64 + l] = o[d2][r];
  }
  lds_barrier();
  if (rb == 1) return;
  const float mo = ms[l], lo2 = ms[64 + l];
  const float M = fmaxf(m, mo);
  const float a = (M == -INFINITY) ? 0.f : fexp2(m - M);
  const float bb = (M == -INFINITY) ? 0.f : fexp2(mo - M);
  const float L = lsum * a + lo2 * bb;
  float* pp = part + (((int64_t)t * nsplit + split) * HQ + 32 * hb + (l & 31)) * (D + 2);
#pragma unroll
  for (int d2 = 0; d2 < DB; ++d2) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d2][r] = o[d2][r] * a + ms[(2 + 16 * d2 + r) * 64 + l] * bb;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f32x4*>(pp + 32 * (DB * dh + d2) + 8 * r4 + 4 * g) =
          f32x4{o[d2][4 * r4], o[d2][4 * r4 + 1], o[d2][4 * r4 + 2], o[d2][4 * r4 + 3]};
  }
  if (dh == 0 && g == 0) {
    pp[D] = M;
    pp[D + 1] = L;
  }
}

bool select_attend_fits(int B, int K, int nsplit, int rows_per_split, int Hq, int D) {
  return Hq == 64 && D == 128 && rows_per_split == kSaRows && nsplit >= 2 && K <= 4096 &&
         (int64_t)B * nsplit <= 256;
}

hipError_t launch_select_attend(const float* scores, int64_t ld, const int32_t* ctx_len, int B,
                                int K, const TopkWs& w, int32_t* idx, uint32_t* stats,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int64_t* cu_ctx, float sm_scale, float* part,
                                int nsplit, hipStream_t stream) {
  // A union of up to 8192 candidates is selected by the first 512 threads
  // (16 slots each): per-wave work (scans, exchanges, address arithmetic)
  // is then paid by 8 waves instead of 16, and the CU's vector issue is the
  // selection's bound.  The eager report loads are laid out for them.
  int eager_q = 0, sel_nt = kSaThreads;
  if (w.max_ctx > kDirectMax) {
    const int s = topk_subtile(w.max_ctx, K);
    const int64_t slots =
        std::min<int64_t>(kResolveSlots, (int64_t)((w.max_ctx + s - 1) / s) * kRep);
    if (slots <= (int64_t)(kSaThreads / 2) * 16) sel_nt = kSaThreads / 2;
    eager_q = (int)((slots + 4 * sel_nt - 1) / (4 * sel_nt));
  }
  const float scale = (sm_scale != 0.f ? sm_scale : 1.f / sqrtf(128.f)) * kLog2e;
  // the groups loaded ahead are a compile-time count (no loads for the rest)
#define DSA_SA_LAUNCH(QE_)                                                                     \
  hipLaunchKernelGGL(select_attend_kernel<QE_>, dim3(nsplit, B), dim3(kSaThreads), 0, stream,  \
                     scores, ld, ctx_len, B, K, w.stride, eager_q, w.hdr, w.rep_u, w.rep_j, idx, \
                     stats, static_cast<const uint16_t*>(q),                                   \
                     static_cast<const uint16_t*>(k_cache),                                    \
                     static_cast<const uint16_t*>(v_cache), cu_ctx, scale, part, nsplit, sel_nt)
  switch (eager_q) {
    case 1: DSA_SA_LAUNCH(1); break;
    case 2: DSA_SA_LAUNCH(2); break;
    case 3: DSA_SA_LAUNCH(3); break;
    case 4: DSA_SA_LAUNCH(4); break;
    default: DSA_SA_LAUNCH(0); break;
  }
#undef DSA_SA_LAUNCH
  return hipGetLastError();
}

// Exact Top-K of many rows straight from their scores (prefill: thousands
// of long rows, where a report per sub-tile costs more than two sweeps over
// the row).  One workgroup of kRowsThreads per row:
//   0. rows of at least kPilotMinRow positions first take a threshold from
//      a sample of about 1/16 of the row, chosen so that about
//      (K + kRowsCap) / 2 keys of the row are expected at or above it, and
//      collect those keys in one ordered sweep (as in 2); if their count is
//      not in [K, kRowsCap] the row continues with 1;
//   1. a sweep builds the 2048-bin histogram of the keys' top 11 bits; one
//      wave finds the bucket of the K-th key; while the keys at or above
//      that bucket would not fit kRowsCap, further sweeps refine it by the
//      next 11 bits;
//   2. an ordered sweep (block prefix sums over 16 consecutive positions
//      per thread) collects every key at or above the bucket into LDS in
//      position order;
//   3. the register path selects the K best of those candidates and writes
//      them in ascending order.
// Rows whose candidates cannot be narrowed to kRowsCap (a key shared by
// very many positions) take the exact sweep select.
constexpr int kRowsThreads = 512;
constexpr int kRowsCap = 4096;  // candidates collected per row
constexpr int kRowsMinT = 1024;  // rows per call from which the row sweeps pay off
constexpr int kPilotMinRow = 16384;  // rows from this length first try a sampled threshold

// Six waves per SIMD (at most 80 VGPRs): three 8-wave workgroups per CU,
// as many as its LDS (about 50 KB each) allows, for more loads in flight.
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(6))) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
    int B, int K, int32_t* idx, uint32_t* stats) {
  constexpr int NSL = 16;
  __shared__ RowsSmem sm;
  __shared__ uint32_t cand_u[kRowsCap];
  __shared__ int32_t cand_j[kRowsCap];
  const int t = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t n = ri.p + 1;
  int32_t* out = idx + (int64_t)t * K;
  if (n <= K) {
    for (int i = tid; i < K; i += nt) out[i] = i < n ? i : -1;
    return;
  }
  const uint32_t k = (uint32_t)K;
  const float* row = scores + (int64_t)t * ld;
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  // Each sweep runs over rounds of PER consecutive keys per thread, the next
  // round's loads in flight while the current one is processed (two key
  // buffers); the barriers inside wait for LDS work only, not those loads.
  constexpr int PER = 8;
  const int64_t step = PER * (int64_t)nt;
  uint32_t ua[PER], ub[PER];
  // ordered collection of the keys >= lo into cand_u / cand_j (position
  // order; positions past kRowsCap are counted, not stored)
  uint32_t lo = 0, cum = 0, par = 0;
  auto collect = [&](const uint32_t(&u)[PER], uint32_t vm, int64_t b0) {
    const int64_t p0 = b0 + PER * tid;
    uint32_t f = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) f |= (uint32_t)(u[i] >= lo) << i;
    f &= vm;
    uint32_t tot;
    uint32_t r = cum + excl_scan_pingpong(sm, (uint32_t)__popc(f), nt >> 6, par++, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((f >> i) & 1u) {
        if (r < (uint32_t)kRowsCap) {
          cand_u[r] = u[i];
          cand_j[r] = (int32_t)(p0 + i);
        }
        ++r;
      }
    cum += tot;
  };
  uint32_t C = 0;  // candidates collected: every key >= lo, k <= C <= kRowsCap
  bool have = false;
  // 0. Long rows: a threshold from a sample (NC chunks of 512 consecutive
  //    keys spread over the row, about 1/16 of it) whose rank in the row is
  //    expected midway between k and kRowsCap; one ordered sweep then
  //    collects every key at or above it.  If the count misses [k,
  //    kRowsCap] (an unrepresentative sample), the row takes steps 1-2.
  if (n >= kPilotMinRow && 4 * (kRowsCap - K) >= K) {
    const int NC = (int)min<int64_t>(32, (n + 8191) / 8192);
    const int64_t P = (n / NC) & ~(int64_t)3;  // chunk period, >= 512
    const int wv = wave_id(), ln = lane_id();
    uint32_t sk[4][PER], svm[4];
#pragma unroll
    for (int rd = 0; rd < 4; ++rd) {
      const int c = 8 * rd + wv;  // one chunk per wave and round
      svm[rd] = 0;
      if (c < NC) svm[rd] = load_keys<PER>(row, n, c * P + PER * ln, vec, sk[rd]);
    }
    for (int i = tid; i < 2048; i += nt) {
      sm.hist()[i] = 0;
      sm.hist2()[i] = 0;
    }
    lds_barrier();
    const uint32_t m = (uint32_t)NC * 512u;
    const uint32_t target = k + ((uint32_t)kRowsCap - k) / 2;
    const uint32_t rk = (uint32_t)(((uint64_t)target * m + (uint64_t)n - 1) / (uint64_t)n);
    // rank rk of the sample: top 11 bits, then the next 11 within that bucket
#pragma unroll
    for (int rd = 0; rd < 4; ++rd)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if ((svm[rd] >> i) & 1u) atomicAdd(&sm.hist()[sk[rd][i] >> 21], 1u);
    lds_barrier();
    if (wv == 0) wave_find_digit(sm, sm.hist(), 0u, rk);
    lds_barrier();
    const uint32_t lo_a = sm.st[0] << 21, above_a = sm.st[1];
#pragma unroll
    for (int rd = 0; rd < 4; ++rd)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (((svm[rd] >> i) & 1u) && (sk[rd][i] >> 21) == (lo_a >> 21))
          atomicAdd(&sm.hist2()[(sk[rd][i] - lo_a) >> 10], 1u);
    lds_barrier();
    if (wv == 0) wave_find_digit(sm, sm.hist2(), above_a, rk);
    lds_barrier();
    lo = lo_a + (sm.st[0] << 10);
    // one ordered sweep over the row
    uint32_t va = load_keys<PER>(row, n, PER * tid, vec, ua);
#pragma unroll 1
    for (int64_t b0 = 0; b0 < n && cum <= (uint32_t)kRowsCap; b0 += 2 * step) {
      const uint32_t vb = load_keys<PER>(row, n, b0 + step + PER * tid, vec, ub);
      collect(ua, va, b0);
      if (b0 + step >= n || cum > (uint32_t)kRowsCap) break;
      va = load_keys<PER>(row, n, b0 + 2 * step + PER * tid, vec, ua);
      collect(ub, vb, b0 + step);
    }
    have = cum >= k && cum <= (uint32_t)kRowsCap;
    C = cum;
    dma_barrier();  // the collection's LDS writes, and st[] reads, before reuse
  }
  if (!have) {
    // 1. bucket of the K-th key: [lo, lo + wm1], `above` keys beyond it (a
    //    key below lo wraps to key - lo > wm1: one unsigned compare)
    for (int i = tid; i < 2048; i += nt) sm.hist()[i] = 0;
    lds_barrier();
    lo = 0;
    uint32_t above = 0, h = 0;
    uint32_t wm1 = 0xffffffffu;
    int shift = 21;
    auto hist_add = [&](const uint32_t(&u)[PER], uint32_t vm) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t x = u[i] - lo;
        if (((vm >> i) & 1u) & (uint32_t)(x <= wm1)) atomicAdd(&sm.hist()[x >> shift], 1u);
      }
    };
#pragma unroll 1
    while (true) {
      uint32_t va = load_keys<PER>(row, n, PER * tid, vec, ua);
#pragma unroll 1
      for (int64_t b0 = 0; b0 < n; b0 += 2 * step) {
        const uint32_t vb = load_keys<PER>(row, n, b0 + step + PER * tid, vec, ub);
        hist_add(ua, va);
        va = load_keys<PER>(row, n, b0 + 2 * step + PER * tid, vec, ua);
        hist_add(ub, vb);
      }
      dma_barrier();
      if (wave_id() == 0) wave_find_digit(sm, sm.hist(), above, k);
      lds_barrier();
      const uint32_t d = sm.st[0];
      above = sm.st[1];
      h = sm.st[5];
      lo += d << shift;
      wm1 = (1u << shift) - 1u;
      if (above + h <= (uint32_t)kRowsCap || shift == 0) break;
      shift = max(0, shift - 11);
      for (int i = tid; i < 2048; i += nt) sm.hist()[i] = 0;
      lds_barrier();
    }
    C = above + h;  // keys >= lo
    if (C > (uint32_t)kRowsCap) {
      exact_select_row(sm, row, n, k, vec, nt, out);
      if (stats && tid == 0) atomicAdd(&stats[1], 1u);
      return;
    }
    // 2. ordered collection of the keys >= lo
    cum = 0;
    uint32_t va = load_keys<PER>(row, n, PER * tid, vec, ua);
#pragma unroll 1
    for (int64_t b0 = 0; b0 < n && cum < C; b0 += 2 * step) {
      const uint32_t vb = load_keys<PER>(row, n, b0 + step + PER * tid, vec, ub);
      collect(ua, va, b0);
      if (b0 + step >= n || cum >= C) break;
      va = load_keys<PER>(row, n, b0 + 2 * step + PER * tid, vec, ua);
      collect(ub, vb, b0 + step);
    }
  }
  dma_barrier();
  // 3. the register path over the candidates (slot s = candidate s)
  UnionRegs<NSL> R;
  R.vmask = 0;
  R.qn = (int)((C + 4 * nt - 1) / (4 * nt));
#pragma unroll
  for (int q = 0; q < NSL / 4; ++q) {
    if (q < R.qn) {
      const int s0 = slot_of(q, tid, nt);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool v = (uint32_t)(s0 + e) < C;
        R.u[4 * q + e] = v ? cand_u[s0 + e] : 0u;
        R.j[4 * q + e] = v ? cand_j[s0 + e] : 0;
        R.vmask |= (uint32_t)v << (4 * q + e);
      }
    }
  }
  select_from_regs(sm, R, k, K, 0, nt, out);  // C >= k: always succeeds
  if (stats && tid == 0) {
    atomicAdd(&stats[3], 1u);
    if (have) atomicAdd(&stats[4], 1u);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
bool topk_use_rows(int T) { return T >= kRowsMinT; }

// Tile of the report-writing kernels (the indexer epilogue and
// tile_report_kernel): the sub-tile size of the longest row, at least one
// wave of positions.  Sub-tile sizes never decrease with the row length, so
// every row's sub-tiles divide this tile.
static_assert(kSubMax == kMaxTile, "report tile range");
int topk_tile_for(int max_ctx, int K) {
  const int s = topk_subtile(max_ctx, K);
  return s < 64 ? 64 : s;
}

// Report entries per row: the most sub-tiles any row of kDirectMax < n <=
// max_ctx positions has.  Over each range of n with one sub-tile size the
// longest row has the most, so only the top of each range is checked.
int topk_report_stride(int max_ctx, int K) {
  int64_t best = 1;
  int64_t n = max_ctx;
  while (n > kDirectMax) {
    const int s = topk_subtile(n, K);
    best = std::max<int64_t>(best, (n + s - 1) / s);
    int64_t lo = kDirectMax + 1, hi = n;  // smallest m with topk_subtile(m) == s
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (topk_subtile(mid, K) >= s) hi = mid; else lo = mid + 1;
    }
    n = lo - 1;
  }
  return (int)best;
}

size_t topk_report_bytes(int T, int max_ctx, int K) {
  if (topk_use_rows(T)) return 0;  // rows selected by sweeps write no reports
  return (size_t)T * topk_report_stride(max_ctx, K) * (sizeof(RepHeader) + kRep * 8);
}

TopkWs topk_ws_carve(void* ws, int T, int max_ctx, int K) {
  TopkWs w;
  w.tile = topk_tile_for(max_ctx, K);
  w.ntiles = (max_ctx + w.tile - 1) / w.tile;
  w.stride = topk_report_stride(max_ctx, K);
  w.max_ctx = max_ctx;
  w.K = K;
  const size_t nslot = (size_t)T * w.stride;
  char* p = static_cast<char*>(ws);
  w.hdr = reinterpret_cast<RepHeader*>(p);
  p += nslot * sizeof(RepHeader);
  w.rep_u = reinterpret_cast<uint32_t*>(p);
  p += nslot * kRep * sizeof(uint32_t);
  w.rep_j = reinterpret_cast<int32_t*>(p);
  return w;
}

hipError_t launch_tile_reports(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int K, const TopkWs& w,
                               hipStream_t stream) {
  if (w.max_ctx <= kDirectMax) return hipSuccess;  // every row is selected directly
  dim3 grid(w.ntiles, T);
  switch (w.tile) {
#define DSA_TILE_CASE(T_)                                                                       \
  case T_:                                                                                      \
    hipLaunchKernelGGL(tile_report_kernel<T_>, grid, dim3(64), 0, stream, scores, ld, cu_q,    \
                       ctx_len, B, K, w.stride, w.hdr, w.rep_u, w.rep_j);                      \
    break;
    DSA_TILE_CASE(64)
    DSA_TILE_CASE(128)
    DSA_TILE_CASE(256)
    DSA_TILE_CASE(512)
    DSA_TILE_CASE(1024)
    DSA_TILE_CASE(2048)
#undef DSA_TILE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topk_rows(const float* scores, int64_t ld, const int32_t* cu_q,
                            const int32_t* ctx_len, int B, int T, int K, int32_t* idx,
                            uint32_t* stats, hipStream_t stream) {
  hipLaunchKernelGGL(topk_rows_kernel, dim3(T), dim3(kRowsThreads), 0, stream, scores, ld, cu_q,
                     ctx_len, B, K, idx, stats);
  return hipGetLastError();
}

hipError_t launch_topk_resolve(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int K, const TopkWs& w,
                               int32_t* idx, uint32_t* stats, hipStream_t stream) {
  // Register slots the longest need: kRep per sub-tile, or one per position
  // of a direct row; 16 per thread (at most 1024 threads).  Rows needing
  // fewer run with fewer waves.
  constexpr int NSL = 16;
  const int direct = std::min(w.max_ctx, kDirectMax);
  const int64_t cap = std::min<int64_t>(kResolveSlots,
                                        std::max<int64_t>((int64_t)w.stride * kRep, direct));
  auto threads = [](int64_t slots) {
    const int64_t wv = (slots + 64 * NSL - 1) / (64 * NSL);
    return (int)(64 * std::max<int64_t>(wv, 1));
  };
  const int nt = threads(cap);
  // Few rows: the report groups a row of max_ctx positions uses are loaded
  // before the row length is known (latency), spread over the whole block
  // (fewer slots per thread is faster than fewer waves); many rows: after
  // (traffic).
  int eager_nt = 0, eager_q = 0;
  if (T <= 256 && w.max_ctx > kDirectMax) {
    const int s = topk_subtile(w.max_ctx, K);
    const int64_t slots = std::min<int64_t>(cap, (int64_t)((w.max_ctx + s - 1) / s) * kRep);
    eager_nt = nt;
    eager_q = (int)((slots + 4 * eager_nt - 1) / (4 * eager_nt));
  }
  hipLaunchKernelGGL(topk_resolve_kernel<NSL>, dim3(T), dim3(nt), 0, stream, scores, ld, cu_q,
                     ctx_len, B, K, w.stride, eager_nt, eager_q, w.hdr, w.rep_u, w.rep_j, idx,
                     stats);
  return hipGetLastError();
}

}  // namespace dsa
