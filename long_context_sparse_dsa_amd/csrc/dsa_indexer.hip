// dsa_indexer.hip -- Indexer scores on gfx950 MFMA.
//
// The Indexer is a lightweight multi-head scorer of every causal past
// position ("Open-Source LLM Architecture Evolution ...", Architecture
// Breakdown item 2; "Fine-Grained Sparse Attention ...", 2.2: no RoPE, 2.3:
// 32 heads x 128 dim; the naive-n0-5-flash page: 16-head indexer):
//
//   s[t, j] = sum_h w[t,h] * max(0, sigma_j * q_idx[t,h,:] . k_idx[j,:])
//
// Both kernels run the per-head dot products as bf16 MFMA contractions with
// fp32 accumulation (v_mfma_f32_32x32x16_bf16).  fp8 e4m3fn keys are widened
// to bf16 in registers (exact), so fp8 only changes the bytes streamed.
//
// Decode (one query per sequence): HBM-bound stream of the key cache.
//   A = the query's heads (32 rows, zero-padded), B = 32 keys per block.
//   Each lane loads its key row's 16-byte chunks straight into MFMA operand
//   registers (no LDS round trip); C holds one key per lane column, so the
//   ReLU / head-weight / head-sum epilogue is 16 fused multiply-adds in
//   registers plus one cross-half add.  The workgroup's tile of scores is
//   then kept in LDS for the Top-K candidate report (dsa_topk_tile.h).
//
// Prefill (a chunk of queries per sequence): MFMA-bound dense contraction.
//   A = (query, head) rows of several queries, B = key tile staged in LDS
//   and shared by the four waves; rows are assigned so that every lane's 16
//   accumulator rows are whole queries, keeping the head sum in registers.
//   Key tiles past the last visible position of the workgroup's queries are
//   skipped; the diagonal tile is masked.
#include "dsa_kernels.h"
#include "dsa_topk_tile.h"

namespace dsa {

// Offset (in elements) of the 8 consecutive dims a lane of half `g` feeds
// into k-step s.  bf16 rows: natural order.  fp8 rows: each lane reads one
// 16-byte chunk covering two k-steps.
template <bool FP8>
__device__ __forceinline__ int kslot_dim(int s, int g) {
  return FP8 ? (32 * (s >> 1) + 16 * g + 8 * (s & 1)) : (16 * s + 8 * g);
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------
template <int DI, bool FP8, int TILE, bool REPORT>
__global__ __launch_bounds__(256) void index_decode_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w, int64_t w_ld,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale, int H_I,
    const int32_t* __restrict__ ctx_len, const int64_t* __restrict__ cu_ctx,
    float* __restrict__ scores, int64_t ld, RepHeader* hdr, uint32_t* rep_u, int32_t* rep_j,
    int ntiles_max) {
  constexpr int KS = DI / 16;            // MFMA k-steps
  constexpr int ROWB = FP8 ? DI : 2 * DI; // bytes per key row
  constexpr int KPW = TILE / 4;          // keys per wave
  constexpr int NB = KPW / 32;           // 32-key blocks per wave
  constexpr int NLD = FP8 ? KS / 2 : KS; // 16-byte loads per lane per block
  constexpr int PF = NB < 4 ? NB : 4;    // blocks loaded ahead together

  __shared__ uint32_t su[TILE];
  __shared__ TileReportSmem sm;

  const int b = blockIdx.y, ti = blockIdx.x;
  const int64_t p = (int64_t)ctx_len[b] - 1;
  const int64_t j0 = (int64_t)ti * TILE;
  if (j0 > p) return;
  const int n_valid = (int)min<int64_t>(TILE, p + 1 - j0);
  const int l = lane_id(), g = l >> 5, wv = wave_id();
  const int64_t row0 = cu_ctx[b];

  // A operand: query heads (rows), zero beyond H_I.
  bf16x8 qa[KS];
  {
    const int head = l & 31;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < H_I) v = ld16(q_idx + ((int64_t)b * H_I + head) * DI + kslot_dim<FP8>(s, g));
      qa[s] = as_bf16x8(v);
    }
  }
  // Head weights of the 16 accumulator rows this lane holds.
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int head = 8 * (r >> 2) + 4 * g + (r & 3);
    wr[r] = head < H_I ? bf16_to_f32(w[(int64_t)b * w_ld + head]) : 0.f;
  }

#pragma unroll 1
  for (int blk0 = 0; blk0 < NB; blk0 += PF) {
    u32x4 kv[PF][NLD];
    float sig[PF];
    int jr[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      jr[u] = wv * KPW + (blk0 + u) * 32 + (l & 31);
      const int64_t jl = min<int64_t>(j0 + jr[u], p);  // clamp: never read past the context
      const uint8_t* rowp = k_idx + (row0 + jl) * ROWB;
#pragma unroll
      for (int c = 0; c < NLD; ++c) kv[u][c] = ld16(rowp + 32 * c + 16 * g);
      sig[u] = FP8 ? k_scale[row0 + jl] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      f32x16 acc = {};
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < NLD; ++c) {
          acc = mfma32(qa[2 * c], fp8x8_to_bf16x8(kv[u][c][0], kv[u][c][1]), acc);
          acc = mfma32(qa[2 * c + 1], fp8x8_to_bf16x8(kv[u][c][2], kv[u][c][3]), acc);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NLD; ++c) acc = mfma32(qa[c], as_bf16x8(kv[u][c]), acc);
      }
      float sl = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sl += wr[r] * fmaxf(sig[u] * acc[r], 0.f);
      const float sc = xor32_add(sl);
      if (g == 0 && jr[u] < n_valid) {
        scores[(int64_t)b * ld + j0 + jr[u]] = sc;
        su[jr[u]] = order_key(sc);
      }
    }
  }
  if constexpr (!REPORT) return;
  __syncthreads();
  const int64_t slot = (int64_t)b * ntiles_max + ti;
  tile_report(su, n_valid, j0, sm, hdr + slot, rep_u + slot * kRepMax, rep_j + slot * kRepMax);
}

template <int DI, bool FP8, bool REPORT>
static hipError_t launch_decode_tiled(int tile, const uint16_t* q, const uint16_t* w,
                                      int64_t w_ld, const uint8_t* k, const float* ks, int H_I,
                                      const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                      int max_ctx, float* scores, int64_t ld, RepHeader* hdr,
                                      uint32_t* ru, int32_t* rj, int ntiles_max,
                                      hipStream_t st) {
  dim3 grid((max_ctx + tile - 1) / tile, B);
#define DSA_DECODE_TILE(T_)                                                                    \
  case T_:                                                                                     \
    hipLaunchKernelGGL((index_decode_kernel<DI, FP8, T_, REPORT>), grid, dim3(256), 0, st, q,  \
                       w, w_ld, k, ks, H_I, ctx_len, cu_ctx, scores, ld, hdr, ru, rj,          \
                       ntiles_max);                                                            \
    break;
  switch (tile) {
    DSA_DECODE_TILE(256)
    DSA_DECODE_TILE(512)
    DSA_DECODE_TILE(1024)
    DSA_DECODE_TILE(2048)
    default:
      return hipErrorInvalidValue;
  }
#undef DSA_DECODE_TILE
  return hipGetLastError();
}

template <int DI, bool FP8>
static hipError_t launch_decode_any(bool report, int tile, const uint16_t* q, const uint16_t* w,
                                    int64_t w_ld, const uint8_t* k, const float* ks, int H_I,
                                    const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                    int max_ctx, float* scores, int64_t ld, RepHeader* hdr,
                                    uint32_t* ru, int32_t* rj, int ntiles_max, hipStream_t st) {
  return report ? launch_decode_tiled<DI, FP8, true>(tile, q, w, w_ld, k, ks, H_I, ctx_len,
                                                     cu_ctx, B, max_ctx, scores, ld, hdr, ru, rj,
                                                     ntiles_max, st)
                : launch_decode_tiled<DI, FP8, false>(tile, q, w, w_ld, k, ks, H_I, ctx_len,
                                                      cu_ctx, B, max_ctx, scores, ld, hdr, ru,
                                                      rj, ntiles_max, st);
}

hipError_t launch_index_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_ctx,
                               float* scores, int64_t ld, const TopkWs* reports,
                               hipStream_t stream) {
  const int tile = reports ? reports->tile : topk_tile_for(max_ctx);
  RepHeader* hdr = reports ? reports->hdr : nullptr;
  uint32_t* ru = reports ? reports->rep_u : nullptr;
  int32_t* rj = reports ? reports->rep_j : nullptr;
  const int ntm = reports ? reports->ntiles_max : 0;
  auto q = static_cast<const uint16_t*>(q_idx);
  auto wp = static_cast<const uint16_t*>(w);
  auto k = static_cast<const uint8_t*>(k_idx);
  const bool fp8 = k_dtype == 1;
  const bool rep = reports != nullptr;
  if (d_I == 128 && !fp8)
    return launch_decode_any<128, false>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len,
                                         cu_ctx, B, max_ctx, scores, ld, hdr, ru, rj, ntm, stream);
  if (d_I == 128 && fp8)
    return launch_decode_any<128, true>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len, cu_ctx,
                                        B, max_ctx, scores, ld, hdr, ru, rj, ntm, stream);
  if (d_I == 64 && !fp8)
    return launch_decode_any<64, false>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len, cu_ctx,
                                        B, max_ctx, scores, ld, hdr, ru, rj, ntm, stream);
  if (d_I == 64 && fp8)
    return launch_decode_any<64, true>(rep, tile, q, wp, w_ld, k, k_scale, H_I, ctx_len, cu_ctx,
                                       B, max_ctx, scores, ld, hdr, ru, rj, ntm, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------
// Row i of a 32-row MFMA block <-> (query within block, head).  Chosen so
// that the 16 accumulator rows of each lane are whole queries.
template <int HI>
struct RowMap {
  static constexpr int QPB = 32 / HI;  // queries per 32-row block
  __device__ static int query_of_row(int i) {
    return HI == 4 ? (i >> 2) : (HI == 16 ? ((i >> 2) & 1) : 0);
  }
  __device__ static int head_of_row(int i) {
    return HI == 4 ? (i & 3) : (HI == 16 ? (4 * (i >> 3) + (i & 3)) : i);
  }
};

template <int DI, int HI, bool FP8, int MB>
__global__ __launch_bounds__(256) void index_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w, int64_t w_ld,
    const uint8_t* __restrict__ k_idx, const float* __restrict__ k_scale,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ ctx_len,
    const int64_t* __restrict__ cu_ctx, float* __restrict__ scores, int64_t ld, int nsplit) {
  constexpr int KS = DI / 16;
  constexpr int ROWB = FP8 ? DI : 2 * DI;
  constexpr int NBK = 2;                     // 32-key blocks per stage
  constexpr int KT = 32 * NBK;               // keys per stage
  constexpr int LROW = ROWB + 16;            // padded LDS row (bytes)
  constexpr int QPB = RowMap<HI>::QPB;
  constexpr int QW = MB * QPB;               // queries per wave
  constexpr int QWG = 4 * QW;                // queries per workgroup
  constexpr int CH = ROWB / 16;              // 16-byte chunks per key row
  constexpr int LDPT = KT * CH / 256;        // chunks per thread per stage

  __shared__ __attribute__((aligned(16))) uint8_t kt_lds[KT * LROW];
  __shared__ float sig_lds[KT];

  const int b = blockIdx.z, qt = blockIdx.y, split = blockIdx.x;
  const int nq = cu_q[b + 1] - cu_q[b];
  const int qbase = qt * QWG;
  if (qbase >= nq) return;
  const int64_t L = ctx_len[b];
  const int64_t pos0 = L - nq;               // position of query 0 of the sequence
  const int64_t row0 = cu_ctx[b];
  const int64_t t0 = cu_q[b];
  const int l = lane_id(), g = l >> 5, wv = wave_id();

  // Query tile of this wave and its A fragments.
  const int wq0 = qbase + wv * QW;
  bf16x8 qa[MB][KS];
  float wr[MB][16];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int i = l & 31;
    const int qq = wq0 + m * QPB + RowMap<HI>::query_of_row(i);
    const int hh = RowMap<HI>::head_of_row(i);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qq < nq) v = ld16(q_idx + ((t0 + qq) * HI + hh) * DI + kslot_dim<FP8>(s, g));
      qa[m][s] = as_bf16x8(v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ir = 8 * (r >> 2) + 4 * g + (r & 3);
      const int q2 = wq0 + m * QPB + RowMap<HI>::query_of_row(ir);
      wr[m][r] = q2 < nq ? bf16_to_f32(w[(t0 + q2) * w_ld + RowMap<HI>::head_of_row(ir)]) : 0.f;
    }
  }
  // Visible key range of this workgroup: [0, last position of its queries].
  const int qlast = min(nq, qbase + QWG) - 1;
  const int64_t kend = pos0 + qlast + 1;
  const int64_t nst = (kend + KT - 1) / KT;
  const int64_t st_lo = nst * split / nsplit, st_hi = nst * (split + 1) / nsplit;

#pragma unroll 1
  for (int64_t st = st_lo; st < st_hi; ++st) {
    const int64_t k0 = st * KT;
    // ---- stage key tile into LDS ----
    __syncthreads();
#pragma unroll
    for (int c = 0; c < LDPT; ++c) {
      const int e = threadIdx.x + 256 * c;
      const int kr = e / CH, kc = e % CH;
      const int64_t j = min<int64_t>(k0 + kr, L - 1);
      u32x4 v = ld16(k_idx + (row0 + j) * ROWB + 16 * kc);
      *reinterpret_cast<u32x4*>(kt_lds + kr * LROW + 16 * kc) = v;
    }
    if (FP8 && threadIdx.x < KT) sig_lds[threadIdx.x] = k_scale[row0 + min<int64_t>(k0 + threadIdx.x, L - 1)];
    __syncthreads();
    // ---- MFMA ----
    f32x16 acc[MB][NBK];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < NBK; ++n) acc[m][n] = f32x16{};
#pragma unroll
    for (int n = 0; n < NBK; ++n) {
      const uint8_t* kr = kt_lds + (32 * n + (l & 31)) * LROW;
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < KS / 2; ++c) {
          u32x4 v = *reinterpret_cast<const u32x4*>(kr + 32 * c + 16 * g);
          bf16x8 b0 = fp8x8_to_bf16x8(v[0], v[1]), b1 = fp8x8_to_bf16x8(v[2], v[3]);
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            acc[m][n] = mfma32(qa[m][2 * c], b0, acc[m][n]);
            acc[m][n] = mfma32(qa[m][2 * c + 1], b1, acc[m][n]);
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          bf16x8 bb = as_bf16x8(*reinterpret_cast<const u32x4*>(kr + 32 * s + 16 * g));
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[m][n] = mfma32(qa[m][s], bb, acc[m][n]);
        }
      }
    }
    // ---- epilogue: ReLU, head weights, head sum, causal mask, store ----
#pragma unroll
    for (int n = 0; n < NBK; ++n) {
      const int64_t j = k0 + 32 * n + (l & 31);
      const float sg = FP8 ? sig_lds[32 * n + (l & 31)] : 1.f;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if constexpr (HI == 4) {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            float s = 0.f;
#pragma unroll
            for (int r = 4 * c4; r < 4 * c4 + 4; ++r) s += wr[m][r] * fmaxf(sg * acc[m][n][r], 0.f);
            const int qq = wq0 + m * QPB + 2 * c4 + g;
            if (qq < nq && j <= pos0 + qq) scores[(t0 + qq) * ld + j] = s;
          }
        } else {
          float s = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) s += wr[m][r] * fmaxf(sg * acc[m][n][r], 0.f);
          int qq;
          if constexpr (HI == 32) {
            s = xor32_add(s);
            qq = (g == 0) ? wq0 + m : nq;  // one half writes
          } else {
            qq = wq0 + m * QPB + g;
          }
          if (qq < nq && j <= pos0 + qq) scores[(t0 + qq) * ld + j] = s;
        }
      }
    }
  }
}

template <int DI, int HI, bool FP8>
static hipError_t launch_prefill_t(const uint16_t* q, const uint16_t* w, int64_t w_ld,
                                   const uint8_t* k, const float* ks, const int32_t* cu_q,
                                   const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                   int max_q, int max_ctx, float* scores, int64_t ld,
                                   hipStream_t st) {
  constexpr int MB = 2;
  constexpr int QWG = 4 * MB * (32 / HI);
  const int qtiles = (max_q + QWG - 1) / QWG;
  // enough workgroups to fill the chip: split the key range when needed
  int nsplit = 1;
  while ((int64_t)qtiles * B * nsplit < 1024 && nsplit < 64 &&
         (int64_t)max_ctx / (nsplit * 2) >= 1024)
    nsplit *= 2;
  dim3 grid(nsplit, qtiles, B);
  hipLaunchKernelGGL((index_prefill_kernel<DI, HI, FP8, MB>), grid, dim3(256), 0, st, q, w, w_ld,
                     k, ks, cu_q, ctx_len, cu_ctx, scores, ld, nsplit);
  return hipGetLastError();
}

hipError_t launch_index_prefill(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                                int k_dtype, const float* k_scale, int H_I, int d_I,
                                const int32_t* cu_q, const int32_t* ctx_len,
                                const int64_t* cu_ctx, int B, int max_q, int max_ctx,
                                float* scores, int64_t ld, hipStream_t stream) {
  auto q = static_cast<const uint16_t*>(q_idx);
  auto wp = static_cast<const uint16_t*>(w);
  auto k = static_cast<const uint8_t*>(k_idx);
  const bool fp8 = k_dtype == 1;
#define DSA_PREFILL_CASE(DI_, HI_)                                                              \
  if (d_I == DI_ && H_I == HI_) {                                                               \
    return fp8 ? launch_prefill_t<DI_, HI_, true>(q, wp, w_ld, k, k_scale, cu_q, ctx_len,      \
                                                  cu_ctx, B, max_q, max_ctx, scores, ld,      \
                                                  stream)                                      \
               : launch_prefill_t<DI_, HI_, false>(q, wp, w_ld, k, k_scale, cu_q, ctx_len,     \
                                                   cu_ctx, B, max_q, max_ctx, scores, ld,     \
                                                   stream);                                    \
  }
  DSA_PREFILL_CASE(128, 32)
  DSA_PREFILL_CASE(128, 16)
  DSA_PREFILL_CASE(64, 4)
#undef DSA_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace dsa
