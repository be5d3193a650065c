// dsa_api.cpp -- the C ABI of libdsa.so (declared in include/dsa.h).
//
// Host-side argument validation, workspace carving and kernel dispatch.
// Validation never touches the GPU, so the library loads and rejects bad
// arguments on a host without a device.  Every launch is asynchronous on
// the caller's stream.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "dsa_kernels.h"
#include "dsa_topk_tile.h"

namespace {

thread_local char g_err[512] = "";

dsa_status_t fail(dsa_status_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

dsa_status_t ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define DSA_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define DSA_PTR(p, name)                                                                   \
  do {                                                                                     \
    if ((p) == nullptr) return fail(DSA_ERR_INVALID_ARG, "%s must not be NULL", name);     \
    if (!aligned16(p)) return fail(DSA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name); \
  } while (0)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ws_ld(int max_ctx) { return (int64_t)align_up((size_t)max_ctx, 64); }

bool indexer_shape_ok(int H_I, int d_I) {
  return (H_I == 4 && d_I == 64) || (H_I == 16 && d_I == 128) || (H_I == 32 && d_I == 128);
}

bool attn_shape_ok(int Hq, int D) { return (Hq == 8 && D == 64) || (Hq == 64 && D == 128); }

dsa_status_t check_batch(const int32_t* cu_q, const int32_t* ctx_len, const int64_t* cu_ctx,
                         bool need_cu_ctx, int B, int T, int max_q, int max_ctx) {
  DSA_REQUIRE(B >= 1, DSA_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  DSA_REQUIRE(T >= 1, DSA_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
  DSA_REQUIRE(max_ctx >= 1, DSA_ERR_INVALID_ARG, "max_ctx must be >= 1 (got %d)", max_ctx);
  DSA_REQUIRE(ctx_len != nullptr, DSA_ERR_INVALID_ARG, "ctx_len must not be NULL");
  if (need_cu_ctx) DSA_REQUIRE(cu_ctx != nullptr, DSA_ERR_INVALID_ARG, "cu_ctx must not be NULL");
  if (cu_q == nullptr) {
    DSA_REQUIRE(T == B, DSA_ERR_INVALID_ARG,
                "cu_q == NULL means one query per sequence: T (%d) must equal B (%d)", T, B);
  } else {
    DSA_REQUIRE(max_q >= 1 && max_q <= max_ctx, DSA_ERR_INVALID_ARG,
                "max_q must be in [1, max_ctx] (got %d)", max_q);
  }
  return DSA_OK;
}

struct DecodeWs {
  float* scores;
  int64_t ld;
  dsa::TopkWs topk;
  int32_t* idx;
  void* attn;
};

size_t decode_ws_layout(int B, int max_ctx, int K, int Hq, int D, char* base, DecodeWs* out) {
  const int64_t ld = ws_ld(max_ctx);
  size_t off = 0;
  const size_t s_scores = align_up((size_t)B * ld * sizeof(float), 256);
  const size_t s_rep = align_up(dsa::topk_report_bytes(B, max_ctx, K), 256);
  const size_t s_idx = align_up((size_t)B * K * sizeof(int32_t), 256);
  const dsa::AttnPlan plan = dsa::attn_plan(B, K, 0, Hq, D);
  const size_t s_attn = align_up(plan.ws_bytes, 256);
  if (out) {
    out->ld = ld;
    out->scores = reinterpret_cast<float*>(base + off);
    out->topk = dsa::topk_ws_carve(base + off + s_scores, B, max_ctx, K);
    out->idx = reinterpret_cast<int32_t*>(base + off + s_scores + s_rep);
    out->attn = base + off + s_scores + s_rep + s_idx;
  }
  return s_scores + s_rep + s_idx + s_attn;
}

size_t prefill_ws_layout(int T, int max_ctx, int K, int Hq, int D, char* base, DecodeWs* out) {
  const int64_t ld = ws_ld(max_ctx);
  const size_t s_scores = align_up((size_t)T * ld * sizeof(float), 256);
  const size_t s_rep = align_up(dsa::topk_report_bytes(T, max_ctx, K), 256);
  const size_t s_idx = align_up((size_t)T * K * sizeof(int32_t), 256);
  const dsa::AttnPlan plan = dsa::attn_plan(T, K, 0, Hq, D);
  const size_t s_attn = align_up(plan.ws_bytes, 256);
  if (out) {
    out->ld = ld;
    out->scores = reinterpret_cast<float*>(base);
    out->topk = dsa::topk_ws_carve(base + s_scores, T, max_ctx, K);
    out->idx = reinterpret_cast<int32_t*>(base + s_scores + s_rep);
    out->attn = base + s_scores + s_rep + s_idx;
  }
  return s_scores + s_rep + s_idx + s_attn;
}

}  // namespace

// Caller-owned Top-K path counters (this thread), or null.
thread_local uint32_t* t_topk_counters = nullptr;

extern "C" {

const char* dsa_version(void) { return "dsa-mi355x 0.1.0 gfx950"; }

const char* dsa_last_error(void) { return g_err; }

dsa_status_t dsa_index_scores(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I,
                              const int32_t* cu_q, const int32_t* ctx_len, const int64_t* cu_ctx,
                              int B, int T, int max_q, int max_ctx, float* scores, int64_t ld,
                              void* stream) {
  DSA_PTR(q_idx, "q_idx");
  DSA_PTR(w, "w");
  DSA_PTR(k_idx, "k_idx");
  DSA_PTR(scores, "scores");
  dsa_status_t st = check_batch(cu_q, ctx_len, cu_ctx, true, B, T, max_q, max_ctx);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(k_dtype == DSA_KEY_BF16 || k_dtype == DSA_KEY_FP8_E4M3, DSA_ERR_INVALID_ARG,
              "k_dtype must be DSA_KEY_BF16 or DSA_KEY_FP8_E4M3 (got %d)", k_dtype);
  if (k_dtype == DSA_KEY_FP8_E4M3)
    DSA_REQUIRE(k_scale != nullptr, DSA_ERR_INVALID_ARG, "fp8 keys need k_scale");
  else
    DSA_REQUIRE(k_scale == nullptr, DSA_ERR_INVALID_ARG, "bf16 keys take no k_scale");
  DSA_REQUIRE(indexer_shape_ok(H_I, d_I), DSA_ERR_UNSUPPORTED,
              "unsupported indexer shape H_I=%d d_I=%d (supported: 4x64, 16x128, 32x128)", H_I,
              d_I);
  DSA_REQUIRE(w_ld == 0 || w_ld >= H_I, DSA_ERR_INVALID_ARG, "w_ld must be 0 or >= H_I");
  DSA_REQUIRE(ld >= max_ctx, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= max_ctx (%d)",
              (long long)ld, max_ctx);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (cu_q == nullptr)
    e = dsa::launch_index_decode(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, ctx_len,
                                 cu_ctx, B, max_ctx, scores, ld, nullptr, s);
  else
    e = dsa::launch_index_prefill(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, cu_q,
                                  ctx_len, cu_ctx, B, max_q, max_ctx, scores, ld, s);
  return hip_status(e, "dsa_index_scores");
}

size_t dsa_topk_workspace_size(int B, int T, int max_ctx, int K) {
  (void)B;
  if (T < 1 || max_ctx < 1 || K < 1) return 0;
  return dsa::topk_report_bytes(T, max_ctx, K);
}

dsa_status_t dsa_topk(const float* scores, int64_t ld, const int32_t* cu_q,
                      const int32_t* ctx_len, int B, int T, int max_q, int max_ctx, int K,
                      int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  DSA_PTR(scores, "scores");
  DSA_PTR(idx, "idx");
  dsa_status_t st = check_batch(cu_q, ctx_len, nullptr, false, B, T, max_q, max_ctx);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(K >= 1 && K <= 4096, DSA_ERR_UNSUPPORTED, "K must be in [1, 4096] (got %d)", K);
  DSA_REQUIRE(ld >= max_ctx, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= max_ctx (%d)",
              (long long)ld, max_ctx);
  const size_t need = dsa_topk_workspace_size(B, T, max_ctx, K);
  DSA_REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes",
              ws_bytes, need);
  DSA_PTR(ws, "ws");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dsa::TopkWs w = dsa::topk_ws_carve(ws, T, max_ctx, K);
  hipError_t e;
  if (dsa::topk_use_rows(T)) {
    e = dsa::launch_topk_rows(scores, ld, cu_q, ctx_len, B, T, K, idx, t_topk_counters, s);
    return hip_status(e, "dsa_topk");
  }
  e = dsa::launch_tile_reports(scores, ld, cu_q, ctx_len, B, T, K, w, s);
  if (e == hipSuccess) e = dsa::launch_topk_resolve(scores, ld, cu_q, ctx_len, B, T, K, w, idx,
                                                    t_topk_counters, s);
  return hip_status(e, "dsa_topk");
}

size_t dsa_sparse_attn_workspace_size(int B, int T, int K, int window, int Hq, int D) {
  (void)B;
  if (T < 1) return 0;
  return dsa::attn_plan(T, K, window, Hq, D).ws_bytes;
}

dsa_status_t dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* idx, int K, int window, const void* gate,
                             float sm_scale, int Hq, int D, const int32_t* cu_q,
                             const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                             int max_q, int max_ctx, void* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  DSA_PTR(q, "q");
  DSA_PTR(k_cache, "k_cache");
  DSA_PTR(v_cache, "v_cache");
  DSA_PTR(out, "out");
  if (gate) DSA_PTR(gate, "gate");
  if (idx) DSA_PTR(idx, "idx");
  dsa_status_t st = check_batch(cu_q, ctx_len, cu_ctx, true, B, T, max_q, max_ctx);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(attn_shape_ok(Hq, D), DSA_ERR_UNSUPPORTED,
              "unsupported attention shape Hq=%d D=%d (supported: 8x64, 64x128)", Hq, D);
  if (idx) {
    DSA_REQUIRE(K >= 1 && K <= 4096, DSA_ERR_UNSUPPORTED, "K must be in [1, 4096] (got %d)", K);
  } else {
    DSA_REQUIRE(window >= 1 && window <= 4096, DSA_ERR_UNSUPPORTED,
                "window must be in [1, 4096] when idx is NULL (got %d)", window);
    K = 0;
  }
  DSA_REQUIRE(sm_scale >= 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be >= 0");
  const dsa::AttnPlan plan = dsa::attn_plan(T, K, idx ? 0 : window, Hq, D);
  DSA_REQUIRE(ws_bytes >= plan.ws_bytes, DSA_ERR_WORKSPACE,
              "workspace too small: %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  if (plan.ws_bytes) DSA_PTR(ws, "ws");
  hipError_t e = dsa::launch_sparse_attn(q, k_cache, v_cache, idx, K, idx ? 0 : window, gate,
                                         sm_scale, Hq, D, cu_q, ctx_len, cu_ctx, B, T, out, lse,
                                         ws, plan, static_cast<hipStream_t>(stream));
  return hip_status(e, "dsa_sparse_attn");
}

size_t dsa_layer_decode_workspace_size(int B, int max_ctx, int K, int Hq, int D) {
  if (B < 1 || max_ctx < 1 || K < 1) return 0;
  return decode_ws_layout(B, max_ctx, K, Hq, D, nullptr, nullptr);
}

// Caller-owned events recorded around the indexer launch (this thread).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

dsa_status_t dsa_set_topk_counters(uint32_t* counters) {
  t_topk_counters = counters;
  return DSA_OK;
}

dsa_status_t dsa_set_indexer_events(void* start, void* stop) {
  DSA_REQUIRE((start == nullptr) == (stop == nullptr), DSA_ERR_INVALID_ARG,
              "start and stop events must both be set or both be NULL");
  t_ev_start = static_cast<hipEvent_t>(start);
  t_ev_stop = static_cast<hipEvent_t>(stop);
  return DSA_OK;
}

dsa_status_t dsa_layer_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I, const void* q,
                              const void* k_cache, const void* v_cache, const void* gate,
                              float sm_scale, int Hq, int D, int K, const int32_t* ctx_len,
                              const int64_t* cu_ctx, int B, int max_ctx, void* out,
                              int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  DSA_PTR(q_idx, "q_idx");
  DSA_PTR(w, "w");
  DSA_PTR(k_idx, "k_idx");
  DSA_PTR(q, "q");
  DSA_PTR(k_cache, "k_cache");
  DSA_PTR(v_cache, "v_cache");
  DSA_PTR(out, "out");
  if (gate) DSA_PTR(gate, "gate");
  if (idx_out) DSA_PTR(idx_out, "idx_out");
  dsa_status_t st = check_batch(nullptr, ctx_len, cu_ctx, true, B, B, 1, max_ctx);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(k_dtype == DSA_KEY_BF16 || k_dtype == DSA_KEY_FP8_E4M3, DSA_ERR_INVALID_ARG,
              "k_dtype must be DSA_KEY_BF16 or DSA_KEY_FP8_E4M3 (got %d)", k_dtype);
  if (k_dtype == DSA_KEY_FP8_E4M3)
    DSA_REQUIRE(k_scale != nullptr, DSA_ERR_INVALID_ARG, "fp8 keys need k_scale");
  else
    DSA_REQUIRE(k_scale == nullptr, DSA_ERR_INVALID_ARG, "bf16 keys take no k_scale");
  DSA_REQUIRE(indexer_shape_ok(H_I, d_I), DSA_ERR_UNSUPPORTED,
              "unsupported indexer shape H_I=%d d_I=%d (supported: 4x64, 16x128, 32x128)", H_I,
              d_I);
  DSA_REQUIRE(w_ld == 0 || w_ld >= H_I, DSA_ERR_INVALID_ARG, "w_ld must be 0 or >= H_I");
  DSA_REQUIRE(attn_shape_ok(Hq, D), DSA_ERR_UNSUPPORTED,
              "unsupported attention shape Hq=%d D=%d (supported: 8x64, 64x128)", Hq, D);
  DSA_REQUIRE(K >= 1 && K <= 4096, DSA_ERR_UNSUPPORTED, "K must be in [1, 4096] (got %d)", K);
  DSA_REQUIRE(sm_scale >= 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be >= 0");
  const size_t need = decode_ws_layout(B, max_ctx, K, Hq, D, nullptr, nullptr);
  DSA_REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes",
              ws_bytes, need);
  DSA_PTR(ws, "ws");
  DecodeWs L;
  decode_ws_layout(B, max_ctx, K, Hq, D, static_cast<char*>(ws), &L);
  int32_t* idx = idx_out ? idx_out : L.idx;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // few rows: the indexer writes candidate reports for the resolve; many
  // rows: plain scores, each row selected by sweeps
  const bool rows = dsa::topk_use_rows(B);
  hipError_t e = dsa::launch_index_decode(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I,
                                          ctx_len, cu_ctx, B, max_ctx, L.scores, L.ld,
                                          rows ? nullptr : &L.topk, s, t_ev_start, t_ev_stop);
  if (e == hipSuccess)
    e = rows ? dsa::launch_topk_rows(L.scores, L.ld, nullptr, ctx_len, B, B, K, idx,
                                     t_topk_counters, s)
             : dsa::launch_topk_resolve(L.scores, L.ld, nullptr, ctx_len, B, B, K, L.topk, idx,
                                        t_topk_counters, s);
  if (e == hipSuccess) {
    const dsa::AttnPlan plan = dsa::attn_plan(B, K, 0, Hq, D);
    e = dsa::launch_sparse_attn(q, k_cache, v_cache, idx, K, 0, gate, sm_scale, Hq, D, nullptr,
                                ctx_len, cu_ctx, B, B, out, nullptr, L.attn, plan, s);
  }
  return hip_status(e, "dsa_layer_decode");
}

size_t dsa_layer_prefill_workspace_size(int B, int T, int max_ctx, int K, int Hq, int D) {
  (void)B;
  if (T < 1 || max_ctx < 1 || K < 1) return 0;
  return prefill_ws_layout(T, max_ctx, K, Hq, D, nullptr, nullptr);
}

dsa_status_t dsa_layer_prefill(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const void* q, const void* k_cache, const void* v_cache,
                               const void* gate, float sm_scale, int Hq, int D, int K,
                               const int32_t* cu_q, const int32_t* ctx_len,
                               const int64_t* cu_ctx, int B, int T, int max_q, int max_ctx,
                               void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                               void* stream) {
  DSA_PTR(q_idx, "q_idx");
  DSA_PTR(w, "w");
  DSA_PTR(k_idx, "k_idx");
  DSA_PTR(q, "q");
  DSA_PTR(k_cache, "k_cache");
  DSA_PTR(v_cache, "v_cache");
  DSA_PTR(out, "out");
  if (gate) DSA_PTR(gate, "gate");
  if (idx_out) DSA_PTR(idx_out, "idx_out");
  DSA_REQUIRE(cu_q != nullptr, DSA_ERR_INVALID_ARG, "prefill needs cu_q");
  dsa_status_t st = check_batch(cu_q, ctx_len, cu_ctx, true, B, T, max_q, max_ctx);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(k_dtype == DSA_KEY_BF16 || k_dtype == DSA_KEY_FP8_E4M3, DSA_ERR_INVALID_ARG,
              "k_dtype must be DSA_KEY_BF16 or DSA_KEY_FP8_E4M3 (got %d)", k_dtype);
  if (k_dtype == DSA_KEY_FP8_E4M3)
    DSA_REQUIRE(k_scale != nullptr, DSA_ERR_INVALID_ARG, "fp8 keys need k_scale");
  else
    DSA_REQUIRE(k_scale == nullptr, DSA_ERR_INVALID_ARG, "bf16 keys take no k_scale");
  DSA_REQUIRE(indexer_shape_ok(H_I, d_I), DSA_ERR_UNSUPPORTED,
              "unsupported indexer shape H_I=%d d_I=%d (supported: 4x64, 16x128, 32x128)", H_I,
              d_I);
  DSA_REQUIRE(w_ld == 0 || w_ld >= H_I, DSA_ERR_INVALID_ARG, "w_ld must be 0 or >= H_I");
  DSA_REQUIRE(attn_shape_ok(Hq, D), DSA_ERR_UNSUPPORTED,
              "unsupported attention shape Hq=%d D=%d (supported: 8x64, 64x128)", Hq, D);
  DSA_REQUIRE(K >= 1 && K <= 4096, DSA_ERR_UNSUPPORTED, "K must be in [1, 4096] (got %d)", K);
  DSA_REQUIRE(sm_scale >= 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be >= 0");
  const size_t need = prefill_ws_layout(T, max_ctx, K, Hq, D, nullptr, nullptr);
  DSA_REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes",
              ws_bytes, need);
  DSA_PTR(ws, "ws");
  DecodeWs L;
  prefill_ws_layout(T, max_ctx, K, Hq, D, static_cast<char*>(ws), &L);
  int32_t* idx = idx_out ? idx_out : L.idx;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dsa::launch_index_prefill(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I,
                                           cu_q, ctx_len, cu_ctx, B, max_q, max_ctx, L.scores,
                                           L.ld, s);
  if (e == hipSuccess && dsa::topk_use_rows(T)) {
    e = dsa::launch_topk_rows(L.scores, L.ld, cu_q, ctx_len, B, T, K, idx, t_topk_counters, s);
  } else {
    if (e == hipSuccess)
      e = dsa::launch_tile_reports(L.scores, L.ld, cu_q, ctx_len, B, T, K, L.topk, s);
    if (e == hipSuccess)
      e = dsa::launch_topk_resolve(L.scores, L.ld, cu_q, ctx_len, B, T, K, L.topk, idx,
                                   t_topk_counters, s);
  }
  if (e == hipSuccess) {
    const dsa::AttnPlan plan = dsa::attn_plan(T, K, 0, Hq, D);
    e = dsa::launch_sparse_attn(q, k_cache, v_cache, idx, K, 0, gate, sm_scale, Hq, D, cu_q,
                                ctx_len, cu_ctx, B, T, out, nullptr, L.attn, plan, s);
  }
  return hip_status(e, "dsa_layer_prefill");
}

}  // extern "C"
