// dsa_kernels.h -- internal launcher interface between the C ABI (dsa_api.cpp)
// and the kernels.  Not installed; the public interface is include/dsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct RepHeader;

constexpr int kMaxTile = 2048;

// Workspace of the Top-K candidate reports.
struct TopkWs {
  int tile;     // positions per report-writing workgroup
  int ntiles;   // such tiles per row of max_ctx positions
  int stride;   // report entries (sub-tiles) per row
  int max_ctx;
  int K;
  RepHeader* hdr;
  uint32_t* rep_u;
  int32_t* rep_j;
};

int topk_tile_for(int max_ctx, int K);
int topk_report_stride(int max_ctx, int K);
size_t topk_report_bytes(int T, int max_ctx, int K);
TopkWs topk_ws_carve(void* ws, int T, int max_ctx, int K);

hipError_t launch_tile_reports(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int K, const TopkWs& w,
                               hipStream_t stream);
// Many rows (T >= a threshold): each row selected by sweeps over its scores,
// no candidate reports (topk_report_bytes is then 0).
bool topk_use_rows(int T);
hipError_t launch_topk_rows(const float* scores, int64_t ld, const int32_t* cu_q,
                            const int32_t* ctx_len, int B, int T, int K, int32_t* idx,
                            uint32_t* stats, hipStream_t stream);
hipError_t launch_topk_resolve(const float* scores, int64_t ld, const int32_t* cu_q,
                               const int32_t* ctx_len, int B, int T, int K, const TopkWs& w,
                               int32_t* idx, uint32_t* stats, hipStream_t stream);

// New rows of a fused decode cache append (one new token per sequence, at
// position ctx_len - 1): bf16 sources and the caches they go into.
struct DecodeAppend {
  const uint16_t* k_idx_new;  // [B, d_I]
  const uint16_t* k_new;      // [B, D] or null
  const uint16_t* v_new;      // [B, D] or null
  uint8_t* k_idx_cache;       // the indexer key cache (bf16 or fp8 codes)
  float* k_scale_cache;       // fp8 scales, or null
  uint16_t* k_cache;
  uint16_t* v_cache;
  int D;
};

// Indexer, one query per sequence.  When `reports` is non-null the kernel
// also writes the Top-K candidate reports of its tiles (tile = reports->tile).
// With `app`, it also appends each sequence's new token to the caches.
// With events, the dispatch records ev0 / ev1 at the kernel's start / end.
hipError_t launch_index_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_ctx,
                               float* scores, int64_t ld, const TopkWs* reports,
                               const DecodeAppend* app, hipStream_t stream,
                               hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Indexer, a chunk of queries per sequence (dense MFMA contraction).  Query
// heads bf16 (q_dtype 0) or E4M3FN codes with q_scale (q_dtype 1, fp8 keys).
hipError_t launch_index_prefill(const void* q_idx, int q_dtype, const float* q_scale,
                                const void* w, int64_t w_ld, const void* k_idx, int k_dtype,
                                const float* k_scale, int H_I, int d_I, const int32_t* cu_q,
                                const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_q,
                                int max_ctx, float* scores, int64_t ld, hipStream_t stream);

// Sparse attention.
struct AttnPlan {
  int nsplit;        // workgroups per query row
  int rows_per_split;
  size_t ws_bytes;   // partial (m, l, o) buffers when nsplit > 1
};
AttnPlan attn_plan(int T, int K, int window, int Hq, int D);

// Merge of split partials (m, l, O) into the gated bf16 output (and lse).
hipError_t launch_attn_combine(int T, int Hq, int D, const float* part, int nsplit,
                               const void* gate, int gstride, void* out, float* lse,
                               hipStream_t stream);

// Decode (one query per sequence, few sequences, Hq = 64, D = 128, index
// rows of 64 per split): the Top-K selection from the candidate reports and
// the split attention in one launch; every workgroup of a sequence repeats
// the selection in its own LDS and attends over its 64 selected rows.
// Writes idx [B, K] (split 0 of each sequence) and the partials `part`,
// merged afterwards by launch_attn_combine.  select_attend_fits tells
// whether a call of B sequences and nsplit splits may take it.
bool select_attend_fits(int B, int K, int nsplit, int rows_per_split, int Hq, int D);
hipError_t launch_select_attend(const float* scores, int64_t ld, const int32_t* ctx_len, int B,
                                int K, const TopkWs& w, int32_t* idx, uint32_t* stats,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int64_t* cu_ctx, float sm_scale, float* part,
                                int nsplit, hipStream_t stream);

// Several attention layers over one batch descriptor in one launch (grid z
// = layer): layer z reads q[z], k_cache[z], v_cache[z], gate[z] and writes
// out[z] in place of the single-layer pointers.
constexpr int kMaxAttnLayers = 8;
struct AttnLayers {
  int n;  // 0: a single layer (the plain pointers)
  const uint16_t* q[kMaxAttnLayers];
  const uint16_t* kc[kMaxAttnLayers];
  const uint16_t* vc[kMaxAttnLayers];
  const uint16_t* gate[kMaxAttnLayers];
  uint16_t* out[kMaxAttnLayers];
};

hipError_t launch_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, int K, int window, const void* gate,
                              int gate_stride_d, float sm_scale, int Hq, int D,
                              const int32_t* cu_q,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                              void* out, float* lse, void* ws, const AttnPlan& plan,
                              hipStream_t stream, const AttnLayers* layers = nullptr);

// Batch descriptor of query rows [t0, t0 + tc) of a prefill call, as a call
// of its own whose row 0 is global row t0: cu_q_c [B+1] and ctx_len_c [B]
// (a sequence without rows in the range gets none; positions are kept).
hipError_t launch_chunk_desc(const int32_t* cu_q, const int32_t* ctx_len, int B, int t0, int tc,
                             int32_t* cu_q_c, int32_t* ctx_len_c, hipStream_t stream);

// New tokens' rows into the caches: query row t goes to cache row
// cu_ctx[b] + p_t (indexer key: bf16 copy, or E4M3FN codes + fp32 scale).
hipError_t launch_cache_append(const void* k_idx_new, int d_I, const void* k_new,
                               const void* v_new, int D, const int32_t* cu_q,
                               const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                               void* k_idx_cache, int k_dtype, float* k_scale_cache,
                               void* k_cache, void* v_cache, hipStream_t stream);

// Debug check of T index rows of K entries (counters: see dsa.h,
// dsa_check_index_rows).  full: the rows are Top-K outputs.
hipError_t launch_check_index_rows(const int32_t* idx, int K, const int32_t* cu_q,
                                   const int32_t* ctx_len, int B, int T, bool full,
                                   uint32_t* counters, hipStream_t stream);

}  // namespace dsa
