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

// Indexer, one query per sequence.  When `reports` is non-null the kernel
// also writes the Top-K candidate reports of its tiles (tile = reports->tile).
// With events, the dispatch records ev0 / ev1 at the kernel's start / end.
hipError_t launch_index_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_ctx,
                               float* scores, int64_t ld, const TopkWs* reports,
                               hipStream_t stream, hipEvent_t ev0 = nullptr,
                               hipEvent_t ev1 = nullptr);

// Indexer, a chunk of queries per sequence (dense MFMA contraction).
hipError_t launch_index_prefill(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                                int k_dtype, const float* k_scale, int H_I, int d_I,
                                const int32_t* cu_q, const int32_t* ctx_len,
                                const int64_t* cu_ctx, int B, int max_q, int max_ctx,
                                float* scores, int64_t ld, hipStream_t stream);

// Sparse attention.
struct AttnPlan {
  int nsplit;        // workgroups per query row
  int rows_per_split;
  size_t ws_bytes;   // partial (m, l, o) buffers when nsplit > 1
};
AttnPlan attn_plan(int T, int K, int window, int Hq, int D);
hipError_t launch_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, int K, int window, const void* gate,
                              float sm_scale, int Hq, int D, const int32_t* cu_q,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                              void* out, float* lse, void* ws, const AttnPlan& plan,
                              hipStream_t stream);

}  // namespace dsa
