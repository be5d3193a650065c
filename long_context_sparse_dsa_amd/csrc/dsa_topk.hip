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
constexpr int kResolveCap = 16384;  // candidates held in LDS

__global__ __launch_bounds__(256) void tile_report_kernel(const float* __restrict__ scores,
                                                          int64_t ld, const int32_t* cu_q,
                                                          const int32_t* ctx_len, int B, int tile,
                                                          int ntiles_max, RepHeader* hdr,
                                                          uint32_t* rep_u, int32_t* rep_j) {
  __shared__ uint32_t su[kMaxTile];
  __shared__ TileReportSmem sm;
  const int t = blockIdx.y, ti = blockIdx.x;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t j0 = (int64_t)ti * tile;
  if (j0 > ri.p) return;
  const int n = (int)min<int64_t>(tile, ri.p + 1 - j0);
  const float* row = scores + (int64_t)t * ld + j0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) su[i] = order_key(row[i]);
  __syncthreads();
  const int64_t slot = (int64_t)t * ntiles_max + ti;
  tile_report(su, n, j0, sm, hdr + slot, rep_u + slot * kRepMax, rep_j + slot * kRepMax);
}

// ---------------------------------------------------------------------------
// Radix select helpers for the resolve kernel (1024 threads, 2048 bins).
// ---------------------------------------------------------------------------
struct ResolveSmem {
  uint32_t cu[kResolveCap];
  int32_t cj[kResolveCap];
  uint32_t hist[2048];
  uint32_t toff[1025];
  uint32_t scan[20];
  uint32_t st[8];
};

// Given hist[2048] of the current bucket and `above` elements strictly above
// it, find digit d with above+gt(d) < k <= above+gt(d)+hist[d].  Writes
// st[0] = d, st[1] = above + gt(d).  Every thread calls it.
__device__ void find_digit(ResolveSmem& sm, uint32_t above, uint32_t k) {
  const int tid = threadIdx.x;
  // thread tid owns digits 2*tid, 2*tid+1
  uint32_t h0 = sm.hist[2 * tid], h1 = sm.hist[2 * tid + 1];
  uint32_t tot;
  uint32_t excl = block_excl_scan(h0 + h1, sm.scan, &tot);
  uint32_t gt1 = tot - excl - h0 - h1;  // above digit 2*tid+1
  uint32_t gt0 = gt1 + h1;              // above digit 2*tid
  if (above + gt1 < k && above + gt1 + h1 >= k) {
    sm.st[0] = 2 * tid + 1;
    sm.st[1] = above + gt1;
  }
  if (above + gt0 < k && above + gt0 + h0 >= k) {
    sm.st[0] = 2 * tid;
    sm.st[1] = above + gt0;
  }
  __syncthreads();
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
    __syncthreads();
    for (int64_t i = tid; i < n; i += nt) {
      uint32_t u;
      int32_t j;
      get(i, &u, &j);
      bool in = pass == 0 ? true : (pass == 1 ? (u >> 21) == prefix : (u >> 10) == prefix);
      if (in) atomicAdd(&sm.hist[(u >> sh) & masks[pass]], 1u);
    }
    __syncthreads();
    find_digit(sm, above, k);
    const uint32_t d = sm.st[0];
    above = sm.st[1];
    prefix = pass == 0 ? d : (pass == 1 ? ((prefix << 11) | d) : ((prefix << 10) | d));
    __syncthreads();
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
  __syncthreads();
}

__global__ __launch_bounds__(kResolveThreads) void topk_resolve_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
    int B, int K, int tile, int ntiles_max, const RepHeader* __restrict__ hdr,
    const uint32_t* __restrict__ rep_u, const int32_t* __restrict__ rep_j, int32_t* idx,
    uint32_t* stats) {
  __shared__ ResolveSmem sm;
  const int t = blockIdx.x, tid = threadIdx.x, nt = blockDim.x;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t n = ri.p + 1;
  int32_t* out = idx + (int64_t)t * K;
  if (n <= K) {
    for (int i = tid; i < K; i += nt) out[i] = i < n ? i : -1;
    return;
  }
  const uint32_t k = (uint32_t)K;
  const int ntiles = (int)((n + tile - 1) / tile);
  const int64_t slot0 = (int64_t)t * ntiles_max;
  // ---- tile offsets ----
  bool fits = ntiles <= kResolveThreads;
  uint32_t C = 0;
  if (fits) {
    uint32_t c = tid < ntiles ? hdr[slot0 + tid].count : 0u;
    uint32_t tot;
    uint32_t ex = block_excl_scan(c, sm.scan, &tot);
    if (tid < ntiles) sm.toff[tid] = ex;
    if (tid == 0) sm.toff[ntiles] = tot;
    __syncthreads();
    C = sm.toff[ntiles];
    fits = C <= (uint32_t)kResolveCap && C >= k;
  }
  bool ok = false;
  if (fits) {
    // ---- gather the union into LDS in ascending position order ----
    for (int64_t s = tid; s < (int64_t)ntiles * kRepMax; s += nt) {
      int ti = (int)(s / kRepMax), e = (int)(s % kRepMax);
      uint32_t off = sm.toff[ti], cnt = sm.toff[ti + 1] - off;
      if ((uint32_t)e < cnt) {
        sm.cu[off + e] = rep_u[(slot0 + ti) * kRepMax + e];
        sm.cj[off + e] = rep_j[(slot0 + ti) * kRepMax + e];
      }
    }
    __syncthreads();
    exact_threshold(sm, (int64_t)C, k, [&](int64_t i, uint32_t* u, int32_t* j) {
      *u = sm.cu[i];
      *j = sm.cj[i];
    });
    const uint32_t tau_u = sm.st[2];
    const int32_t tau_j = (int32_t)sm.st[3];
    // ---- certification ----
    int bad = 0;
    for (int ti = tid; ti < ntiles; ti += nt) {
      RepHeader h = hdr[slot0 + ti];
      if (!h.complete) {
        bool fine = (h.worst_u < tau_u) || (h.worst_u == tau_u && h.worst_j >= tau_j);
        bad |= !fine;
      }
    }
    ok = !__syncthreads_or(bad);
    if (ok) {
      const int per = (int)((C + nt - 1) / nt);
      const int lo = tid * per, hi = min((int)C, lo + per);
      uint32_t cnt = 0;
      for (int i = lo; i < hi; ++i) {
        uint32_t u = sm.cu[i];
        cnt += (u > tau_u) || (u == tau_u && sm.cj[i] <= tau_j);
      }
      uint32_t tot;
      uint32_t pos = block_excl_scan(cnt, sm.scan, &tot);
      for (int i = lo; i < hi; ++i) {
        uint32_t u = sm.cu[i];
        if ((u > tau_u) || (u == tau_u && sm.cj[i] <= tau_j)) {
          if (pos < k) out[pos] = sm.cj[i];
          ++pos;
        }
      }
      if (stats && tid == 0) atomicAdd(&stats[0], 1u);
    }
  }
  if (!ok) {
    // ---- exact fallback straight from the score row ----
    const float* row = scores + (int64_t)t * ld;
    auto get = [&](int64_t i, uint32_t* u, int32_t* j) {
      *u = order_key(row[i]);
      *j = (int32_t)i;
    };
    exact_threshold(sm, n, k, get);
    const uint32_t tau_u = sm.st[2];
    const int32_t tau_j = (int32_t)sm.st[3];
    uint32_t base = 0;
    for (int64_t r0 = 0; r0 < n; r0 += nt) {
      int64_t i = r0 + tid;
      uint32_t f = 0;
      if (i < n) {
        uint32_t u = order_key(row[i]);
        f = (u > tau_u) || (u == tau_u && (int32_t)i <= tau_j);
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
int topk_tile_for(int max_ctx) {
  int tile = 256;
  while (tile < kMaxTile && (int64_t)tile * 512 < (int64_t)max_ctx) tile <<= 1;
  return tile;
}

size_t topk_report_bytes(int T, int max_ctx) {
  const int tile = topk_tile_for(max_ctx);
  const int64_t ntiles = (max_ctx + tile - 1) / tile;
  return (size_t)T * ntiles * (sizeof(RepHeader) + kRepMax * 8);
}

TopkWs topk_ws_carve(void* ws, int T, int max_ctx) {
  TopkWs w;
  w.tile = topk_tile_for(max_ctx);
  w.ntiles_max = (max_ctx + w.tile - 1) / w.tile;
  const size_t nslot = (size_t)T * w.ntiles_max;
  char* p = static_cast<char*>(ws);
  w.hdr = reinterpret_cast<RepHeader*>(p);
  p += nslot * sizeof(RepHeader);
  w.rep_u = reinterpret_cast<uint32_t*>(p);
  p += nslot * kRepMax * sizeof(uint32_t);
  w.rep_j = reinterpret_cast<int32_t*>(p);
  return w;
}

hipError_t launch_tile_reports(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int max_ctx,
                               const TopkWs& w, hipStream_t stream) {
  dim3 grid(w.ntiles_max, T);
  hipLaunchKernelGGL(tile_report_kernel, grid, dim3(256), 0, stream, scores, ld, cu_q, ctx_len,
                     B, w.tile, w.ntiles_max, w.hdr, w.rep_u, w.rep_j);
  return hipGetLastError();
}

hipError_t launch_topk_resolve(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int K, const TopkWs& w,
                               int32_t* idx, uint32_t* stats, hipStream_t stream) {
  hipLaunchKernelGGL(topk_resolve_kernel, dim3(T), dim3(kResolveThreads), 0, stream, scores, ld,
                     cu_q, ctx_len, B, K, w.tile, w.ntiles_max, w.hdr, w.rep_u, w.rep_j, idx,
                     stats);
  return hipGetLastError();
}

}  // namespace dsa
