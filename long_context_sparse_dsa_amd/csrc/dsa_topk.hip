// dsa_topk.hip -- exact per-query Top-K of fp32 score rows.
//
// Selection rule (the pages keep "the K highest-scoring historical
// positions", K = 2048; ties, order and padding are the readings stated in
// dsa.h): K_eff = min(K, p+1) best positions by (score desc, position asc),
// -0.0 == +0.0, output ascending, padded with -1.
//
// Two kernels:
//   tile_report_kernel  one workgroup per (row, tile): loads the tile's
//                       scores, writes its candidate prefix (dsa_topk_tile.h).
//                       The decode indexer writes the same reports from its
//                       epilogue, so the layer path skips this kernel.
//   topk_resolve_kernel one workgroup per row: gathers the reports into LDS
//                       (they arrive in ascending position order), finds the
//                       K_eff-th best candidate with three radix passes
//                       (11/11/10 bits) and a position-ordered tie rank,
//                       certifies the union, and writes the selected
//                       positions with a block prefix sum (already ascending).
//                       If certification fails, or the union does not fit
//                       LDS, it runs the same exact radix select over the
//                       whole score row from global memory instead.
#include "dsa_kernels.h"
#include "dsa_topk_tile.h"

namespace dsa {

constexpr int kResolveThreads = 1024;
constexpr int kResolveTiles = 1024;                         // tiles in the fast path
constexpr int kSlots = kResolveTiles * kRep / kResolveThreads;  // report slots per thread (16)

template <int TILE>
__global__ __launch_bounds__(64) void tile_report_kernel(const float* __restrict__ scores,
                                                         int64_t ld, const int32_t* cu_q,
                                                         const int32_t* ctx_len, int B,
                                                         int ntiles_max, RepHeader* hdr,
                                                         uint32_t* rep_u, int32_t* rep_j) {
  constexpr int V = TILE / 64;
  const int t = blockIdx.y, ti = blockIdx.x;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t j0 = (int64_t)ti * TILE;
  if (j0 > ri.p) return;
  const int n = (int)min<int64_t>(TILE, ri.p + 1 - j0);
  const float* row = scores + (int64_t)t * ld + j0;
  const int l = lane_id();
  uint32_t uv[V];
  int32_t jv[V];
  bool vv[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int jl = 64 * i + l;
    vv[i] = jl < n;
    uv[i] = order_key(row[vv[i] ? jl : 0]);
    jv[i] = (int32_t)(j0 + jl);
  }
  const int64_t slot = (int64_t)t * ntiles_max + ti;
  wave_tile_report<V>(uv, jv, vv, hdr + slot, rep_u + slot * kRep, rep_j + slot * kRep);
}

// ---------------------------------------------------------------------------
// Radix select helpers for the resolve kernel (1024 threads, 2048 bins).
// ---------------------------------------------------------------------------
constexpr int kBucketMax = 64;  // boundary-bucket size ranked directly by wave 0

struct ResolveSmem {
  int32_t stage[4096];  // selected positions before the coalesced store (K <= 4096)
  uint32_t hist[2048];
  uint32_t hist2[2048];  // the union select alternates between hist and hist2
  alignas(16) uint32_t bu[kBucketMax];
  alignas(16) int32_t bj[kBucketMax];
  // per tile: worst reported (key, position | complete << 31), kept for the
  // certification so the headers need not stay in registers
  uint32_t wu[kResolveTiles];
  uint32_t wj[kResolveTiles];
  uint32_t red[64];
  uint32_t scan[20];
  uint32_t st[8];
};

// Wave 0 of the block: given the 2048-bin histogram h of the current
// bucket and `above` elements strictly above the bucket, find digit d with
// above + gt(d) < k <= above + gt(d) + h[d] (gt(d): elements in digits > d).
// Writes st[0] = d, st[1] = above + gt(d), st[5] = h[d].  Lane l owns bins
// 32 l .. 32 l + 31: it sums them (chunk reads in a lane-rotated order, so
// fewer lanes share a bank), one wave scan finds the lane holding d, and
// that lane alone walks its bins.
__device__ void wave_find_digit(ResolveSmem& sm, const uint32_t* h, uint32_t above, uint32_t k) {
  const int l = lane_id();
  uint32_t mine = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(h + 32 * l + 4 * ((c + l) & 7));
    mine += v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t incl = wave_incl_scan(mine);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  uint32_t gt = total - incl;  // elements in the bins of higher lanes
  if (above + gt < k && above + gt + mine >= k) {
#pragma unroll 1
    for (int c2 = 3; c2 >= 0; --c2) {  // two chunks per step
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(h + 32 * l + 8 * c2 + 4);
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(h + 32 * l + 8 * c2);
      const uint32_t vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        if (above + gt < k && above + gt + vv[i] >= k) {
          sm.st[0] = 32 * l + 8 * c2 + i;
          sm.st[1] = above + gt;
          sm.st[5] = vv[i];
        }
        gt += vv[i];
      }
    }
  }
}

// Exact threshold (tau_u, tau_j) over an array source; `get(i, &u, &j)`
// returns element i (in ascending position order).  Result in st[2], st[3].
template <typename Get>
__device__ void exact_threshold(ResolveSmem& sm, int64_t n, uint32_t k, Get get) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t prefix = 0, above = 0;
  const int shifts[3] = {21, 10, 0};
  const uint32_t masks[3] = {0x7ffu, 0x7ffu, 0x3ffu};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    for (int i = tid; i < 2048; i += nt) sm.hist[i] = 0;
    lds_barrier();
    for (int64_t i = tid; i < n; i += nt) {
      uint32_t u;
      int32_t j;
      get(i, &u, &j);
      bool in = pass == 0 ? true : (pass == 1 ? (u >> 21) == prefix : (u >> 10) == prefix);
      if (in) atomicAdd(&sm.hist[(u >> sh) & masks[pass]], 1u);
    }
    lds_barrier();
    if (wave_id() == 0) wave_find_digit(sm, sm.hist, above, k);
    lds_barrier();
    const uint32_t d = sm.st[0];
    above = sm.st[1];
    prefix = pass == 0 ? d : (pass == 1 ? ((prefix << 11) | d) : ((prefix << 10) | d));
    lds_barrier();
  }
  const uint32_t tau_u = prefix;
  const uint32_t need = k - above;  // >= 1 elements equal to tau_u, lowest positions
  // tie rank in position order, processed in rounds of nt elements
  if (tid == 0) sm.st[3] = 0xffffffffu;
  uint32_t base = 0;
  for (int64_t r0 = 0; r0 < n; r0 += nt) {
    int64_t i = r0 + tid;
    uint32_t u = 0;
    int32_t j = -1;
    if (i < n) get(i, &u, &j);
    uint32_t f = (i < n && u == tau_u) ? 1u : 0u;
    uint32_t tot;
    uint32_t ex = block_excl_scan(f, sm.scan, &tot);
    if (f && base + ex == need - 1) sm.st[3] = (uint32_t)j;
    base += tot;
    if (base >= need) break;  // uniform: tot is block-wide
  }
  if (tid == 0) sm.st[2] = tau_u;
  lds_barrier();
}

// Fast path of the resolve.  The union of the row's tile reports (up to
// 1024 tiles x kRep slots) is loaded with fully coalesced 16-byte loads:
// wave w, load q, lane l holds slots s = 1024w + 256q + 4l + e (e < 4),
// i.e. slot (4l+e) % kRep of tile s / kRep.  Slot order is position order, so a
// position-ordered scan over the union is a per-q wave scan plus one
// cross-wave prefix.  Per-slot validity is a bitmask (bit 4q+e) and the
// per-element work is branch-free.
constexpr int kQN = kSlots / 4;  // 16-byte loads per thread

struct UnionRegs {
  uint32_t u[kSlots];
  int32_t j[kSlots];
  uint32_t vmask;  // bit i: slot i holds a candidate
};

__device__ __forceinline__ int slot_index(int wv, int q, int l) { return 1024 * wv + 256 * q + 4 * l; }

// Exclusive position-ordered prefix of per-slot flags (bitmask, bit 4q+e);
// returns each slot's rank among flagged slots and the total.  Also ORs the
// per-thread flag `bad` over the block into *any_bad (same exchange).
__device__ void ordered_ranks(ResolveSmem& sm, uint32_t fmask, uint32_t (&rank)[kSlots],
                              uint32_t* total, bool bad = false, bool* any_bad = nullptr) {
  const int l = lane_id(), wv = wave_id(), nw = blockDim.x >> 6;
  uint32_t lane_ex[kQN], qoff[kQN];
  uint32_t woff = 0;
#pragma unroll
  for (int q = 0; q < kQN; ++q) {
    const uint32_t c = (uint32_t)__popc((fmask >> (4 * q)) & 15u);
    const uint32_t inc = wave_incl_scan(c);
    lane_ex[q] = inc - c;
    qoff[q] = woff;
    woff += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  }
  const bool wbad = __ballot(bad) != 0;
  if (l == 0) {
    sm.red[wv] = woff;
    sm.red[32 + wv] = wbad ? 1u : 0u;
  }
  lds_barrier();
  const uint32_t wt = l < nw ? sm.red[l] : 0u;
  const uint32_t wi = wave_incl_scan(wt);
  const uint32_t wbase = (uint32_t)__builtin_amdgcn_readlane((int)(wi - wt), wv);
  *total = (uint32_t)__builtin_amdgcn_readlane((int)wi, 63);
  if (any_bad) *any_bad = __ballot(l < nw && sm.red[32 + l] != 0u) != 0;
#pragma unroll
  for (int q = 0; q < kQN; ++q) {
    const uint32_t r = wbase + qoff[q] + lane_ex[q];
    const uint32_t m = (fmask >> (4 * q)) & 15u;
    rank[4 * q + 0] = r;
    rank[4 * q + 1] = r + (m & 1u);
    rank[4 * q + 2] = r + __popc(m & 3u);
    rank[4 * q + 3] = r + __popc(m & 7u);
  }
  lds_barrier();
}

// Exact K-th best candidate of the union: selected <=> key > tau_u, or
// key == tau_u and position <= tau_j.  Radix digits (11, 11, 10 bits) are
// taken relative to the union's key range [mn, mx], so the first pass
// spreads the candidates over the 2048 bins instead of piling them onto the
// few bins the leading exponent bits would give.  Each pass is one LDS
// histogram and one wave-0 digit search (the other waves clear the other
// histogram meanwhile).  As soon as the boundary bucket holds at most
// kBucketMax candidates they are gathered and wave 0 ranks them directly
// under (key desc, position asc), which gives (tau_u, tau_j) at once.  Both
// histograms are zero and st[4] is 0 on entry.
__device__ void union_threshold(ResolveSmem& sm, const UnionRegs& R, uint32_t k, uint32_t mn,
                                uint32_t mx, uint32_t* tau_u, int32_t* tau_j) {
  const int tid = threadIdx.x, nt = blockDim.x, wv = wave_id(), l = lane_id();
  const uint32_t range = mx - mn;
  // bucket = keys in [lo, lo + width); digits (key - lo) >> shift are < 2048
  int shift = range == 0 ? 0 : max(0, 32 - __clz(range) - 11);
  uint32_t lo = mn;
  uint64_t width = (uint64_t)range + 1;
  uint32_t above = 0;  // candidates strictly above the bucket
  uint32_t h = 0;      // candidates in the bucket
  int pass = 0;
  while (true) {
    uint32_t* hc = (pass & 1) ? sm.hist2 : sm.hist;
    uint32_t* hn = (pass & 1) ? sm.hist : sm.hist2;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const uint32_t x = R.u[i];
      const bool in = ((R.vmask >> i) & 1u) && x >= lo && (uint64_t)(x - lo) < width;
      if (in) atomicAdd(&hc[(x - lo) >> shift], 1u);
    }
    lds_barrier();
    if (wv == 0) {
      wave_find_digit(sm, hc, above, k);
    } else {
      for (int i = tid - 64; i < 2048; i += nt - 64) hn[i] = 0;  // next pass's histogram
    }
    lds_barrier();
    const uint32_t d = sm.st[0];
    above = sm.st[1];
    h = sm.st[5];
    const uint64_t off = (uint64_t)d << shift;
    lo += (uint32_t)off;
    width = min<uint64_t>(width - off, 1ull << shift);
    if (shift == 0 || h <= (uint32_t)kBucketMax) break;
    shift = max(0, shift - 11);
    ++pass;
  }
  const uint32_t need = k - above;  // 1..h: the need-th best of the bucket is theta
  if (h <= (uint32_t)kBucketMax) {
    // gather the bucket: per-wave ballot compaction at a base taken with
    // one LDS atomic per wave
    uint32_t inb = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const uint32_t x = R.u[i];
      const bool in = ((R.vmask >> i) & 1u) && x >= lo && (uint64_t)(x - lo) < width;
      inb |= (uint32_t)in << i;
      cnt += popc64(__ballot(in));
    }
    if (cnt) {
      uint32_t base = 0;
      if (l == 0) base = atomicAdd(&sm.st[4], cnt);
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, 0);
      const uint64_t below = lanes_below();
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        const bool in = (inb >> i) & 1u;
        const uint64_t m = __ballot(in);
        if (in) {
          const uint32_t pos = base + popc64(m & below);
          sm.bu[pos] = R.u[i];
          sm.bj[pos] = R.j[i];
        }
        base += popc64(m);
      }
    }
    lds_barrier();
    if (wv == 0) {
      const bool mine_ok = (uint32_t)l < h;
      const uint32_t um = mine_ok ? sm.bu[l] : 0u;
      const int32_t jm = mine_ok ? sm.bj[l] : 0;
      // every lane reads the whole bucket (broadcast reads, all issued at once)
      uint32_t rank = 0;
#pragma unroll 1
      for (int q0 = 0; q0 < (int)h; q0 += 16) {
        u32x4 uq[4], jq[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uq[c] = *reinterpret_cast<const u32x4*>(sm.bu + q0 + 4 * c);
          jq[c] = *reinterpret_cast<const u32x4*>(sm.bj + q0 + 4 * c);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rank += (uint32_t)(q0 + 4 * c + e) < h &&
                    ((uq[c][e] > um) || (uq[c][e] == um && (int32_t)jq[c][e] < jm));
      }
      if (mine_ok && rank == need - 1) {
        sm.st[2] = um;
        sm.st[3] = (uint32_t)jm;
      }
    }
    lds_barrier();
    *tau_u = sm.st[2];
    *tau_j = (int32_t)sm.st[3];
    return;
  }
  // more than kBucketMax candidates share the single key lo: the need
  // lowest positions among them are selected
  *tau_u = lo;
  uint32_t inb = 0;
#pragma unroll
  for (int i = 0; i < kSlots; ++i)
    inb |= (uint32_t)(((R.vmask >> i) & 1u) && R.u[i] == lo) << i;
  uint32_t rk[kSlots], tot;
  ordered_ranks(sm, inb, rk, &tot);
  if (tid == 0) sm.st[3] = 0x7fffffffu;
  lds_barrier();
  if (need < tot) {
#pragma unroll
    for (int i = 0; i < kSlots; ++i)
      if (((inb >> i) & 1u) && rk[i] == need - 1) sm.st[3] = (uint32_t)R.j[i];
  }
  lds_barrier();
  *tau_j = (int32_t)sm.st[3];
}

__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
    int B, int K, int tile, int ntiles_max, const RepHeader* __restrict__ hdr,
    const uint32_t* __restrict__ rep_u, const int32_t* __restrict__ rep_j, int32_t* idx,
    uint32_t* stats) {
  __shared__ ResolveSmem sm;
  const int t = blockIdx.x, tid = threadIdx.x, nt = blockDim.x, l = lane_id(), wv = wave_id();
  const int64_t slot0 = (int64_t)t * ntiles_max;
  const int nslots = ntiles_max * kRep;
  // Issue the report loads together with the descriptor loads: one round trip.
  UnionRegs R;
  RepHeader hq[kQN];
  {
    u32x4 a[kQN], c[kQN];
#pragma unroll
    for (int q = 0; q < kQN; ++q) {
      const int sidx = slot_index(wv, q, l);
      const int sc = sidx < nslots ? sidx : 0;
      a[q] = *reinterpret_cast<const u32x4*>(rep_u + slot0 * kRep + sc);
      c[q] = *reinterpret_cast<const u32x4*>(rep_j + slot0 * kRep + sc);
      hq[q] = hdr[slot0 + sc / kRep];
    }
#pragma unroll
    for (int q = 0; q < kQN; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        R.u[4 * q + e] = a[q][e];
        R.j[4 * q + e] = (int32_t)c[q][e];
      }
  }
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t n = ri.p + 1;
  int32_t* out = idx + (int64_t)t * K;
  if (n <= K) {
    for (int i = tid; i < K; i += nt) out[i] = i < n ? i : -1;
    return;
  }
  const uint32_t k = (uint32_t)K;
  const int ntiles = (int)((n + tile - 1) / tile);
  R.vmask = 0;
#pragma unroll
  for (int q = 0; q < kQN; ++q) {
    const int sidx = slot_index(wv, q, l);
    const bool tile_ok = sidx < nslots && sidx / kRep < ntiles;
    const uint32_t sub = (uint32_t)(sidx % kRep);
    const uint32_t cnt = hq[q].count;
    // slots sub .. sub+3 of the tile are valid while below its count
    const uint32_t nv = tile_ok ? (cnt > sub ? min(cnt - sub, 4u) : 0u) : 0u;
    R.vmask |= ((1u << nv) - 1u) << (4 * q);
    if (sub == 0 && sidx < nslots) {
      sm.wu[sidx / kRep] = hq[q].worst_u;
      sm.wj[sidx / kRep] = (uint32_t)hq[q].worst_j | (hq[q].complete ? 0x80000000u : 0u);
    }
  }
  bool ok = false;
  if (ntiles <= kResolveTiles && ntiles <= ntiles_max) {
    // candidate count and key range of the union, in one block reduction;
    // both histograms are cleared meanwhile
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const bool vi = (R.vmask >> i) & 1u;
      mn = min(mn, vi ? R.u[i] : 0xffffffffu);
      mx = max(mx, vi ? R.u[i] : 0u);
    }
    const uint32_t cw = wave_sum_u32((uint32_t)__popc(R.vmask));
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (l == 0) {
      sm.red[wv] = cw;
      sm.red[16 + wv] = mn;
      sm.red[32 + wv] = mx;
    }
    for (int i = tid; i < 2048; i += nt) {
      sm.hist[i] = 0;
      sm.hist2[i] = 0;
    }
    if (tid == 0) sm.st[4] = 0;
    lds_barrier();
    uint32_t C;
    {
      const int nw = nt >> 6;
      C = wave_sum_u32(l < nw ? sm.red[l] : 0u);
      mn = wave_min_u32(l < nw ? sm.red[16 + l] : 0xffffffffu);
      mx = wave_max_u32(l < nw ? sm.red[32 + l] : 0u);
    }
    lds_barrier();  // red[] is reused below
    if (C >= k) {
      uint32_t tau_u;
      int32_t tau_j;
      union_threshold(sm, R, k, mn, mx, &tau_u, &tau_j);
      // ---- certification: every partly reported tile ends at or below
      // theta (checked in the same block exchange as the ranks) ----
      bool bad = false;
      if (tid < ntiles) {
        const uint32_t wu = sm.wu[tid], wj = sm.wj[tid];
        const bool complete = wj >> 31;
        const int32_t wpos = (int32_t)(wj & 0x7fffffffu);
        bad = !complete && !((wu < tau_u) || (wu == tau_u && wpos >= tau_j));
      }
      uint32_t smask = 0;
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        const bool si = ((R.vmask >> i) & 1u) &&
                        ((R.u[i] > tau_u) || (R.u[i] == tau_u && R.j[i] <= tau_j));
        smask |= (uint32_t)si << i;
      }
      uint32_t rk[kSlots], total;
      bool any_bad = false;
      ordered_ranks(sm, smask, rk, &total, bad, &any_bad);
      ok = !any_bad;
      if (ok) {
        // stage in LDS, then store coalesced
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
          if (((smask >> i) & 1u) && rk[i] < k) sm.stage[rk[i]] = R.j[i];
        lds_barrier();
        for (int i = tid; i < K; i += nt) out[i] = sm.stage[i];
        if (stats && tid == 0) atomicAdd(&stats[0], 1u);
      }
    }
  }
  if (!ok) {
    // ---- exact fallback straight from the score row ----
    const float* row = scores + (int64_t)t * ld;
    auto get = [&](int64_t i, uint32_t* uu, int32_t* jj) {
      *uu = order_key(row[i]);
      *jj = (int32_t)i;
    };
    exact_threshold(sm, n, k, get);
    const uint32_t tau_u = sm.st[2];
    const int32_t tau_j = (int32_t)sm.st[3];
    uint32_t base = 0;
    for (int64_t r0 = 0; r0 < n; r0 += nt) {
      int64_t i = r0 + tid;
      uint32_t f = 0;
      if (i < n) {
        uint32_t uu = order_key(row[i]);
        f = (uu > tau_u) || (uu == tau_u && (int32_t)i <= tau_j);
      }
      uint32_t tot;
      uint32_t ex = block_excl_scan(f, sm.scan, &tot);
      if (f && base + ex < k) out[base + ex] = (int32_t)i;
      base += tot;
    }
    if (stats && tid == 0) atomicAdd(&stats[1], 1u);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
// Tile size: a power of two in [64, 2048] with at most kResolveTiles tiles
// per row and about four of the row's top K expected per tile, so that a
// tile rarely holds more than kRep of them (which would send the row to
// the exact fallback).
int topk_tile_for(int max_ctx, int K) {
  const int64_t k = K > 0 ? K : 1;
  const int64_t per4 = (4LL * max_ctx) / k;  // about four winners per tile
  const int64_t by_tiles = ((int64_t)max_ctx + kResolveTiles - 1) / kResolveTiles;
  int tile = 64;
  while (tile < kMaxTile && 2LL * tile <= per4) tile <<= 1;   // round down
  while (tile < kMaxTile && tile < by_tiles) tile <<= 1;      // tile-count cap
  return tile;
}

size_t topk_report_bytes(int T, int max_ctx, int K) {
  const int tile = topk_tile_for(max_ctx, K);
  const int64_t ntiles = (max_ctx + tile - 1) / tile;
  return (size_t)T * ntiles * (sizeof(RepHeader) + kRep * 8);
}

TopkWs topk_ws_carve(void* ws, int T, int max_ctx, int K) {
  TopkWs w;
  w.tile = topk_tile_for(max_ctx, K);
  w.ntiles_max = (max_ctx + w.tile - 1) / w.tile;
  const size_t nslot = (size_t)T * w.ntiles_max;
  char* p = static_cast<char*>(ws);
  w.hdr = reinterpret_cast<RepHeader*>(p);
  p += nslot * sizeof(RepHeader);
  w.rep_u = reinterpret_cast<uint32_t*>(p);
  p += nslot * kRep * sizeof(uint32_t);
  w.rep_j = reinterpret_cast<int32_t*>(p);
  return w;
}

hipError_t launch_tile_reports(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int max_ctx,
                               const TopkWs& w, hipStream_t stream) {
  dim3 grid(w.ntiles_max, T);
  switch (w.tile) {
#define DSA_TILE_CASE(T_)                                                                       \
  case T_:                                                                                      \
    hipLaunchKernelGGL(tile_report_kernel<T_>, grid, dim3(64), 0, stream, scores, ld, cu_q,    \
                       ctx_len, B, w.ntiles_max, w.hdr, w.rep_u, w.rep_j);                     \
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

hipError_t launch_topk_resolve(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int K, const TopkWs& w,
                               int32_t* idx, uint32_t* stats, hipStream_t stream) {
  // one thread per tile (16 report slots each), 64 .. 1024 threads
  int nt = ((w.ntiles_max + 63) / 64) * 64;
  nt = nt < 64 ? 64 : (nt > kResolveThreads ? kResolveThreads : nt);
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(T), dim3(nt), 0, stream, scores, ld,
                     cu_q, ctx_len, B, K, w.tile, w.ntiles_max, w.hdr, w.rep_u, w.rep_j, idx,
                     stats);
  return hipGetLastError();
}

}  // namespace dsa
