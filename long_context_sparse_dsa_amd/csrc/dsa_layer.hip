// dsa_layer.hip -- small layer-level kernels around the three steps.
//
// chunk_desc_kernel: a prefill call whose workspace cannot hold the score
// array of all its query rows runs them in consecutive sub-chunks.  Every
// step of the layer is row-wise (a query row's scores, selection and
// attention depend on that row and the caches only), so a sub-chunk is a
// call of its own over rows [t0, t0 + tc) with a batch descriptor that
// keeps each row's position: for sequence b with n_q queries at positions
// ctx_len - n_q .. ctx_len - 1, the rows in the range are queries
// i0 .. i0 + n' - 1, which a descriptor with n' queries and context length
// ctx_len - n_q + i0 + n' places at the same positions.
//
// cache_append_kernel: the new tokens' rows into the caches.
// check_index_rows_kernel: the debug check of index rows.
#include "dsa_kernels.h"
#include "dsa_device.h"

namespace dsa {

__global__ void chunk_desc_kernel(const int32_t* __restrict__ cu_q,
                                  const int32_t* __restrict__ ctx_len, int B, int t0, int tc,
                                  int32_t* __restrict__ cu_q_c, int32_t* __restrict__ ctx_len_c) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > B) return;
  const int q0 = cu_q[b];
  const int lo = min(max(q0 - t0, 0), tc);
  cu_q_c[b] = lo;
  if (b == B) return;
  const int q1 = cu_q[b + 1];
  const int hi = min(max(q1 - t0, 0), tc);
  const int nq = q1 - q0, nc = hi - lo;
  const int i0 = t0 + lo - q0;  // query index (within the sequence) of the range's first row
  ctx_len_c[b] = nc > 0 ? ctx_len[b] - nq + i0 + nc : 0;
}

hipError_t launch_chunk_desc(const int32_t* cu_q, const int32_t* ctx_len, int B, int t0, int tc,
                             int32_t* cu_q_c, int32_t* ctx_len_c, hipStream_t stream) {
  const int n = B + 1;
  hipLaunchKernelGGL(chunk_desc_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cu_q, ctx_len,
                     B, t0, tc, cu_q_c, ctx_len_c);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Cache append: the new tokens' rows go into the caches at their positions
// (fp8 indexer keys quantised by e4m3_row_pair, dsa_device.h).
// ---------------------------------------------------------------------------
// One wave per new token row t, written to cache row cu_ctx[b] + p_t.
template <int DI, bool FP8>
__global__ __launch_bounds__(64) void cache_append_kernel(
    const uint16_t* __restrict__ k_idx_new, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int D, const int32_t* cu_q, const int32_t* ctx_len,
    const int64_t* cu_ctx, int B, uint8_t* __restrict__ k_idx_cache,
    float* __restrict__ k_scale_cache, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache) {
  const int t = blockIdx.x, l = lane_id();
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t row = cu_ctx[ri.b] + ri.p;
  if (k_idx_new) {
    if constexpr (FP8) {
      // DI / 2 lanes hold two elements each; the rest hold zeros (no effect on the maximum)
      uint32_t pair = 0;
      if (2 * l < DI) pair = *reinterpret_cast<const uint32_t*>(k_idx_new + (int64_t)t * DI + 2 * l);
      float sigma;
      const uint32_t codes = e4m3_row_pair(bf16_to_f32((uint16_t)(pair & 0xffffu)),
                                           bf16_to_f32((uint16_t)(pair >> 16)), &sigma);
      if (2 * l < DI)
        *reinterpret_cast<uint16_t*>(k_idx_cache + row * DI + 2 * l) = (uint16_t)codes;
      if (l == 0) k_scale_cache[row] = sigma;
    } else {
      constexpr int NC = DI / 8;  // 16-byte chunks of a bf16 row
      if (l < NC)
        *reinterpret_cast<u32x4*>(k_idx_cache + row * 2 * DI + 16 * l) =
            ld16(k_idx_new + (int64_t)t * DI + 8 * l);
    }
  }
  // K and V rows: one 16-byte chunk per lane, K in the low lanes, V above
  const int nc = D / 8;
  const bool is_v = l >= nc;
  const int c = is_v ? l - nc : l;
  const uint16_t* src = is_v ? v_new : k_new;
  uint16_t* dst = is_v ? v_cache : k_cache;
  if (l < 2 * nc && src != nullptr)
    *reinterpret_cast<u32x4*>(dst + row * D + 8 * c) = ld16(src + (int64_t)t * D + 8 * c);
}

hipError_t launch_cache_append(const void* k_idx_new, int d_I, const void* k_new,
                               const void* v_new, int D, const int32_t* cu_q,
                               const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                               void* k_idx_cache, int k_dtype, float* k_scale_cache,
                               void* k_cache, void* v_cache, hipStream_t stream) {
  auto ki = static_cast<const uint16_t*>(k_idx_new);
  auto kn = static_cast<const uint16_t*>(k_new);
  auto vn = static_cast<const uint16_t*>(v_new);
  auto kic = static_cast<uint8_t*>(k_idx_cache);
  auto kc = static_cast<uint16_t*>(k_cache);
  auto vc = static_cast<uint16_t*>(v_cache);
  const bool fp8 = k_dtype == 1;
#define DSA_APPEND(DI_, F_)                                                                   \
  hipLaunchKernelGGL((cache_append_kernel<DI_, F_>), dim3(T), dim3(64), 0, stream, ki, kn, vn, \
                     D, cu_q, ctx_len, cu_ctx, B, kic, k_scale_cache, kc, vc)
  if (d_I == 128) {
    if (fp8) DSA_APPEND(128, true); else DSA_APPEND(128, false);
  } else if (d_I == 64) {
    if (fp8) DSA_APPEND(64, true); else DSA_APPEND(64, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef DSA_APPEND
  return hipGetLastError();
}

// check_index_rows_kernel: one workgroup per index row t (K entries), p its
// query's position.  Counts in c[0] the entries outside [0, p] other than
// -1; with `full` (a Top-K output: K_eff = min(K, p + 1) ascending
// positions, then -1 padding) also, in c[1], the neighbouring pairs that
// break that order (a -1 before a position, or positions not increasing)
// and, in c[2], the rows whose count of positions is not K_eff; c[3]
// counts the rows checked.  Reads only idx and the batch descriptor.
__global__ __launch_bounds__(256) void check_index_rows_kernel(const int32_t* __restrict__ idx,
                                                               int K, const int32_t* cu_q,
                                                               const int32_t* ctx_len, int B,
                                                               int full, uint32_t* c) {
  __shared__ uint32_t nvalid;
  const int t = blockIdx.x;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int32_t* row = idx + (int64_t)t * K;
  if (threadIdx.x == 0) nvalid = 0;
  __syncthreads();
  uint32_t bad = 0, order = 0, valid = 0;
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    const int32_t j = row[i];
    bad += (j < -1 || (int64_t)j > ri.p) ? 1u : 0u;
    valid += j >= 0 ? 1u : 0u;
    if (full && i + 1 < K) {
      const int32_t n = row[i + 1];
      order += ((j < 0 && n >= 0) || (j >= 0 && n >= 0 && n <= j)) ? 1u : 0u;
    }
  }
  if (bad) atomicAdd(&c[0], bad);
  if (order) atomicAdd(&c[1], order);
  atomicAdd(&nvalid, valid);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t keff = ri.p + 1 < (int64_t)K ? ri.p + 1 : (int64_t)K;
    if (full && (int64_t)nvalid != keff) atomicAdd(&c[2], 1u);
    atomicAdd(&c[3], 1u);
  }
}

hipError_t launch_check_index_rows(const int32_t* idx, int K, const int32_t* cu_q,
                                   const int32_t* ctx_len, int B, int T, bool full,
                                   uint32_t* counters, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_index_rows_kernel, dim3(T), dim3(256), 0, stream, idx, K, cu_q,
                     ctx_len, B, full ? 1 : 0, counters);
  return hipGetLastError();
}

}  // namespace dsa
