// dsa_attn.hip -- gated sparse attention over gathered K/V rows.
//
// For query row t and head h, over the selected positions S (one index row
// per query shared by every head; one shared K/V head):
//   o = softmax_{j in S}(c * q[t,h,:] . K[j,:]) @ V[S,:],  out = o * sigmoid(g)
// ("Open-Source LLM Architecture Evolution ...", Technical Deep Dive item 2:
// scores and softmax over only the selected 2048; Architecture Breakdown
// item 2 and the deployment page section 2: gated layers.)  With idx == NULL
// the set is the sliding window {p-W+1 .. p} (the naive-n0-5-flash page).
//
// Kernel layout (gfx950, wave64, 4 waves per workgroup):
//   - a workgroup takes `rows_per_split` consecutive entries of the query's
//     index row; wave (hb, rb) handles head block hb (32 heads) and row block
//     rb (32 rows) of each 32*RB-row step, keeping its own running softmax
//     state (max, sum, O^T accumulators); the waves' states are merged at
//     the end through LDS;
//   - S^T = K_rows . q^T on MFMA: the gathered K rows are loaded straight
//     into A-operand registers (16-byte chunks of each 256-byte row), q is
//     the B operand held in registers for the whole kernel;
//   - in the S^T accumulator layout each lane holds one head and 16 rows, so
//     the per-head max / sum need one cross-half exchange, and P^T is
//     already in B-operand layout (the k slots of the PV product are taken in
//     the order the accumulator rows come in);
//   - V rows are written transposed into a per-wave LDS tile so the A
//     operand of O^T = V^T . P^T is two 8-byte LDS reads per k step;
//   - with several splits per query the workgroups write partial (m, l, O)
//     and a combine kernel merges them and applies the gate.
#include "dsa_kernels.h"
#include "dsa_device.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + __expf(-x)); }

template <int D, int HB>
__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ idx, int K, int window,
    const uint16_t* __restrict__ gate, float scale_log2, int Hq, const int32_t* cu_q,
    const int32_t* ctx_len, const int64_t* cu_ctx, int B, int rows_per_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part, int nsplit) {
  constexpr int KS = D / 16;   // k-steps of q . K
  constexpr int DB = D / 32;   // 32-wide blocks of the output dim
  constexpr int RB = 4 / HB;   // row-block waves per head block
  constexpr int VTS = 32 + 4;  // padded row count of the transposed V tile (bf16)
  constexpr int MO_FLOATS = (RB - 1) * HB * 32 * (D + 2);
  constexpr int VT_HALFS = 4 * D * VTS;
  constexpr int SMEM_BYTES = (MO_FLOATS * 4 > VT_HALFS * 2) ? MO_FLOATS * 4 : VT_HALFS * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_BYTES];
  uint16_t* vt = reinterpret_cast<uint16_t*>(smem);
  float* mo = reinterpret_cast<float*>(smem);

  const int t = blockIdx.y, split = blockIdx.x;
  const int l = lane_id(), g = l >> 5, wv = wave_id();
  const int hb = wv % HB, rb = wv / HB;
  const RowInfo ri = row_info(t, cu_q, ctx_len, B);
  const int64_t row0 = cu_ctx[ri.b];
  const int nlist = idx ? K : (int)min<int64_t>(window, ri.p + 1);
  const int64_t jw0 = ri.p - nlist + 1;  // window mode: first position
  const int lo = split * rows_per_split;
  const int hi = min(nlist, lo + rows_per_split);

  const int head = 32 * hb + (l & 31);
  const bool head_ok = head < Hq;
  bf16x8 qb[KS];
  {
    // clamped address instead of a branch: every load is in flight at once
    const int hc = min(head, Hq - 1);
    u32x4 qv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qv[s] = ld16(q + ((int64_t)t * Hq + hc) * D + 16 * s + 8 * g);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (!head_ok) qv[s] = u32x4{0u, 0u, 0u, 0u};
      qb[s] = as_bf16x8(qv[s]);
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};

  uint16_t* myvt = vt + wv * (D * VTS);
#pragma unroll 1
  for (int base = lo; base < hi; base += 32 * RB) {
    const int lp = base + 32 * rb + (l & 31);
    bool valid = lp < hi;
    int64_t j = 0;
    if (valid) {
      j = idx ? (int64_t)idx[(int64_t)t * K + lp] : jw0 + lp;
      valid = j >= 0;
    }
    const int64_t row = row0 + (valid ? j : 0);
    u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = ld16(kc + row * D + 16 * s + 8 * g);
#pragma unroll
    for (int s = 0; s < KS; ++s) vf[s] = ld16(vc + row * D + 16 * s + 8 * g);
    const uint32_t vmask = (uint32_t)__ballot(valid);
    // V^T into this wave's LDS tile: element (d, r) at myvt[d*VTS + r]
    lds_barrier();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * s + 8 * g + e;
        const uint32_t word = vf[s][e >> 1];
        myvt[d * VTS + (l & 31)] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
      }
    }
    // S^T = K . q^T
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = mfma32(as_bf16x8(kf[s]), qb[s], sacc);
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + 4 * g + (r & 3);
      const bool ok = (vmask >> ir) & 1u;
      sv[r] = ok ? sacc[r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = (sv[r] == -INFINITY) ? 0.f : exp2f(sv[r] - m_new);
      psum += sv[r];
    }
    l_run = l_run * alpha + xor32_add(psum);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[s2][e] = static_cast<__bf16>(sv[8 * s2 + e]);
    lds_barrier();
    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* vrow = myvt + (32 * db + (l & 31)) * VTS;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow + 16 * s2 + 4 * g);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + 16 * s2 + 8 + 4 * g);
        const u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
        o[db] = mfma32(as_bf16x8(av), pb[s2], o[db]);
      }
    }
  }
  // ---- merge the RB row-block waves of each head block ----
  lds_barrier();
  if (rb > 0) {
    float* my = mo + ((rb - 1) * HB + hb) * 32 * (D + 2);
    const int hl = l & 31;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
        my[hl * (D + 2) + d] = o[db][r];
      }
    if (g == 0) {
      my[hl * (D + 2) + D] = m_run;
      my[hl * (D + 2) + D + 1] = l_run;
    }
  }
  lds_barrier();
  if (rb != 0) return;
  const int hl = l & 31;
  float M = m_run;
#pragma unroll
  for (int k = 1; k < RB; ++k) M = fmaxf(M, mo[((k - 1) * HB + hb) * 32 * (D + 2) + hl * (D + 2) + D]);
  const float a_self = (M == -INFINITY) ? 0.f : exp2f(m_run - M);
  float Lsum = l_run * a_self;
  float ak[RB];
  ak[0] = a_self;
#pragma unroll
  for (int k = 1; k < RB; ++k) {
    const float* other = mo + ((k - 1) * HB + hb) * 32 * (D + 2) + hl * (D + 2);
    ak[k] = (M == -INFINITY) ? 0.f : exp2f(other[D] - M);
    Lsum += other[D + 1] * ak[k];
  }
  if (!head_ok) return;
  const bool final_out = nsplit == 1;
  const float inv = (Lsum > 0.f) ? 1.f / Lsum : 0.f;
  float* pp = part + (((int64_t)t * nsplit + split) * Hq + head) * (D + 2);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float vals[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * r4 + e;
        const int d = 32 * db + 8 * r4 + 4 * g + e;
        float acc = o[db][r] * ak[0];
#pragma unroll
        for (int k = 1; k < RB; ++k)
          acc += mo[((k - 1) * HB + hb) * 32 * (D + 2) + hl * (D + 2) + d] * ak[k];
        vals[e] = acc;
      }
      const int d0 = 32 * db + 8 * r4 + 4 * g;
      if (final_out) {
        const uint16_t* gp = gate ? gate + ((int64_t)t * Hq + head) * D + d0 : nullptr;
        uint16_t ob[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = vals[e] * inv;
          if (gp) v *= sigmoidf(bf16_to_f32(gp[e]));
          ob[e] = f32_to_bf16(v);
        }
        uint16_t* op = out + ((int64_t)t * Hq + head) * D + d0;
        *reinterpret_cast<u32x2*>(op) = u32x2{(uint32_t)ob[0] | ((uint32_t)ob[1] << 16),
                                             (uint32_t)ob[2] | ((uint32_t)ob[3] << 16)};
      } else {
        *reinterpret_cast<f32x4*>(pp + d0) = f32x4{vals[0], vals[1], vals[2], vals[3]};
      }
    }
  }
  if (g == 0) {
    if (final_out) {
      if (lse) lse[(int64_t)t * Hq + head] = (Lsum > 0.f) ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
    } else {
      pp[D] = M;
      pp[D + 1] = Lsum;
    }
  }
}

// Merge split partials: grid (T, Hq), D threads.  All loads of a block are
// independent: first every split's (m, l), then every split's O[d].
constexpr int kMaxSplit = 64;

template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float* __restrict__ part, int nsplit,
                                                         int Hq, const uint16_t* __restrict__ gate,
                                                         uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  __shared__ float sm_m[kMaxSplit], sm_l[kMaxSplit], sm_w[kMaxSplit];
  __shared__ float sm_ML[2];
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const float* pp = part + ((int64_t)t * nsplit * Hq + h) * (D + 2);
  const int64_t stride = (int64_t)Hq * (D + 2);
  for (int s = d; s < nsplit; s += D) {
    sm_m[s] = pp[s * stride + D];
    sm_l[s] = pp[s * stride + D + 1];
  }
  float g = 0.f;
  const int64_t off = ((int64_t)t * Hq + h) * D + d;
  if (gate) g = bf16_to_f32(gate[off]);
  lds_barrier();
  if (d < 64) {
    float M = -INFINITY;
    for (int s = d; s < nsplit; s += 64) M = fmaxf(M, sm_m[s]);
    M = wave_max_f32(M);
    float L = 0.f;
    for (int s = d; s < nsplit; s += 64) {
      const float a = (M == -INFINITY) ? 0.f : exp2f(sm_m[s] - M);
      sm_w[s] = a;
      L += a * sm_l[s];
    }
    L = wave_sum_f32(L);
    if (d == 0) {
      sm_ML[0] = M;
      sm_ML[1] = L;
    }
  }
  lds_barrier();
  const float L = sm_ML[1];
  float acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) acc += sm_w[s] * pp[s * stride + d];
  float v = L > 0.f ? acc / L : 0.f;
  if (gate) v *= sigmoidf(g);
  out[off] = f32_to_bf16(v);
  if (lse && d == 0) lse[(int64_t)t * Hq + h] = L > 0.f ? (sm_ML[0] + log2f(L)) * kLn2 : -INFINITY;
}

AttnPlan attn_plan(int T, int K, int window, int Hq, int D) {
  AttnPlan p;
  const int nlist = K > 0 ? K : window;
  const int hb = (Hq + 31) / 32;
  const int step = 32 * (4 / (hb > 2 ? 2 : hb));
  // a step per workgroup when few queries, otherwise whole rows
  int rows = step;
  if ((int64_t)T * ((nlist + step - 1) / step) > 2048) rows = nlist > 0 ? nlist : step;
  while ((nlist + rows - 1) / rows > kMaxSplit) rows *= 2;
  p.rows_per_split = rows;
  p.nsplit = (nlist + rows - 1) / rows;
  if (p.nsplit < 1) p.nsplit = 1;
  p.ws_bytes = p.nsplit > 1 ? (size_t)T * p.nsplit * Hq * (D + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, int K, int window, const void* gate,
                              float sm_scale, int Hq, int D, const int32_t* cu_q,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                              void* out, float* lse, void* ws, const AttnPlan& plan,
                              hipStream_t stream) {
  const float scale = (sm_scale != 0.f ? sm_scale : 1.f / sqrtf((float)D)) * kLog2e;
  auto qp = static_cast<const uint16_t*>(q);
  auto kp = static_cast<const uint16_t*>(k_cache);
  auto vp = static_cast<const uint16_t*>(v_cache);
  auto gp = static_cast<const uint16_t*>(gate);
  auto op = static_cast<uint16_t*>(out);
  float* part = static_cast<float*>(ws);
  dim3 grid(plan.nsplit, T);
  if (D == 128 && Hq == 64) {
    hipLaunchKernelGGL((sparse_attn_kernel<128, 2>), grid, dim3(256), 0, stream, qp, kp, vp, idx,
                       K, window, gp, scale, Hq, cu_q, ctx_len, cu_ctx, B, plan.rows_per_split,
                       op, lse, part, plan.nsplit);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(T, Hq), dim3(128), 0, stream, part,
                         plan.nsplit, Hq, gp, op, lse);
  } else if (D == 64 && Hq == 8) {
    hipLaunchKernelGGL((sparse_attn_kernel<64, 1>), grid, dim3(256), 0, stream, qp, kp, vp, idx,
                       K, window, gp, scale, Hq, cu_q, ctx_len, cu_ctx, B, plan.rows_per_split,
                       op, lse, part, plan.nsplit);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL((attn_combine_kernel<64>), dim3(T, Hq), dim3(64), 0, stream, part,
                         plan.nsplit, Hq, gp, op, lse);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
