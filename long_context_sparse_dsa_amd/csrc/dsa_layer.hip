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
#include "dsa_kernels.h"

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

}  // namespace dsa
