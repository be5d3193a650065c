// dsa_api.cpp -- the C ABI of libdsa.so (declared in include/dsa.h).
//
// Host-side argument validation, workspace carving and kernel dispatch.
// Validation never touches the GPU, so the library loads and rejects bad
// arguments on a host without a device.  Every launch is asynchronous on
// the caller's stream.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <dlfcn.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <algorithm>
#include <atomic>
#include <mutex>

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

// Optional roctx ranges (DSA_TRACE=1 in the environment): each entry point
// that enqueues GPU work brackets its host side, so a profiler's marker
// trace shows which call launched which kernels.  The marker library is
// opened on first use, not linked.
struct Roctx {
  int (*push)(const char*);
  int (*pop)();
};

const Roctx* roctx() {
  static const Roctx* r = []() -> const Roctx* {
    const char* e = std::getenv("DSA_TRACE");
    if (e == nullptr || e[0] == '\0' || e[0] == '0') return nullptr;
    // the profiler SDK's marker library (what rocprofv3 --marker-trace
    // records), else the older roctracer one
    void* h = nullptr;
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so",
                            "/opt/rocm/lib/librocprofiler-sdk-roctx.so", "libroctx64.so",
                            "/opt/rocm/lib/libroctx64.so"}) {
      h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (h != nullptr) break;
    }
    if (h == nullptr) return nullptr;
    static Roctx t;
    t.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    t.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    return (t.push && t.pop) ? &t : nullptr;
  }();
  return r;
}

class TraceRange {
 public:
  explicit TraceRange(const char* name) : r_(roctx()) {
    if (r_) r_->push(name);
  }
  ~TraceRange() {
    if (r_) r_->pop();
  }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;

 private:
  const Roctx* r_;
};

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

dsa_status_t check_query_dtype(int q_dtype, const float* q_scale, int k_dtype) {
  DSA_REQUIRE(q_dtype == DSA_QUERY_BF16 || q_dtype == DSA_QUERY_FP8_E4M3, DSA_ERR_INVALID_ARG,
              "q_dtype must be DSA_QUERY_BF16 or DSA_QUERY_FP8_E4M3 (got %d)", q_dtype);
  if (q_dtype == DSA_QUERY_FP8_E4M3) {
    DSA_REQUIRE(q_scale != nullptr, DSA_ERR_INVALID_ARG, "fp8 query heads need q_scale");
    DSA_REQUIRE(k_dtype == DSA_KEY_FP8_E4M3, DSA_ERR_UNSUPPORTED,
                "fp8 query heads need an fp8 key cache (the fp8 MFMA takes both operands)");
  } else {
    DSA_REQUIRE(q_scale == nullptr, DSA_ERR_INVALID_ARG, "bf16 query heads take no q_scale");
  }
  return DSA_OK;
}

// Device descriptor of one prefill sub-chunk: cu_q [B+1] and ctx_len [B]
// (int32), each 256-byte aligned.
size_t prefill_chunk_desc_bytes(int B) {
  return align_up((size_t)B + 1, 64) * 4 + align_up((size_t)B * 4, 256);
}

}  // namespace

// Caller-owned Top-K path counters (this thread), or null.
thread_local uint32_t* t_topk_counters = nullptr;
// Caller-owned index-row check counters (this thread), or null.
thread_local uint32_t* t_idx_checks = nullptr;

namespace {

// The debug check of freshly selected index rows, while enabled.
hipError_t check_selected(const int32_t* idx, int K, const int32_t* cu_q, const int32_t* ctx_len,
                          int B, int T, hipStream_t s) {
  if (t_idx_checks == nullptr) return hipSuccess;
  return dsa::launch_check_index_rows(idx, K, cu_q, ctx_len, B, T, true, t_idx_checks, s);
}

}  // namespace

namespace {

// Indexer -> Top-K -> attention for T query rows in the workspace carved as
// L for T_plan >= T rows: the Top-K path and the attention split plan are
// those of T_plan, so the carve holds their scratch for any T <= T_plan.
hipError_t prefill_pass(const void* q_idx, int q_dtype, const float* q_scale, const void* w,
                        int64_t w_ld, const void* k_idx, int k_dtype, const float* k_scale,
                        int H_I, int d_I, const void* q,
                        const void* k_cache, const void* v_cache, const void* gate, int gstride,
                        float sm_scale, int Hq, int D, int K, const int32_t* cu_q,
                        const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T, int T_plan,
                        int max_q, int max_ctx, void* out, int32_t* idx, const DecodeWs& L,
                        hipStream_t s) {
  hipError_t e = dsa::launch_index_prefill(q_idx, q_dtype, q_scale, w, w_ld, k_idx, k_dtype,
                                           k_scale, H_I, d_I, cu_q, ctx_len, cu_ctx, B, max_q,
                                           max_ctx, L.scores, L.ld, s);
  if (e == hipSuccess && dsa::topk_use_rows(T_plan)) {
    e = dsa::launch_topk_rows(L.scores, L.ld, cu_q, ctx_len, B, T, K, idx, t_topk_counters, s);
  } else {
    if (e == hipSuccess)
      e = dsa::launch_tile_reports(L.scores, L.ld, cu_q, ctx_len, B, T, K, L.topk, s);
    if (e == hipSuccess)
      e = dsa::launch_topk_resolve(L.scores, L.ld, cu_q, ctx_len, B, T, K, L.topk, idx,
                                   t_topk_counters, s);
  }
  if (e == hipSuccess) e = check_selected(idx, K, cu_q, ctx_len, B, T, s);
  if (e == hipSuccess) {
    const dsa::AttnPlan plan = dsa::attn_plan(T_plan, K, 0, Hq, D);
    e = dsa::launch_sparse_attn(q, k_cache, v_cache, idx, K, 0, gate, gstride, sm_scale, Hq, D,
                                cu_q, ctx_len, cu_ctx, B, T, out, nullptr, L.attn, plan, s);
  }
  return e;
}

// Largest row count c in [1, T - 1] whose prefill layout fits `avail`
// bytes, or 0.  The layout grows with c except where a call of more rows
// drops a scratch region (Top-K reports below the row-sweep threshold,
// attention partials while the split plan is in use), so each stretch
// between those two break points is searched on its own, from the top.
int prefill_chunk_rows(int T, int max_ctx, int K, int Hq, int D, size_t avail) {
  auto fits = [&](int c) {
    return prefill_ws_layout(c, max_ctx, K, Hq, D, nullptr, nullptr) <= avail;
  };
  // break points: the last c with Top-K reports and the last c with
  // attention partials (both predicates hold for every smaller c)
  auto last_true = [&](auto pred) {
    int lo = 0, hi = T;
    while (lo < hi) {
      const int mid = lo + (hi - lo + 1) / 2;
      if (pred(mid)) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  const int b_rep = last_true([](int c) { return !dsa::topk_use_rows(c); });
  const int b_att = last_true([&](int c) { return dsa::attn_plan(c, K, 0, Hq, D).ws_bytes > 0; });
  int cuts[4] = {T - 1, b_rep, b_att, 0};
  std::sort(cuts, cuts + 4, [](int a, int b) { return a > b; });
  for (int i = 0; i < 3; ++i) {
    int hi = std::min(cuts[i], T - 1), lo = cuts[i + 1] + 1;
    if (hi < lo || hi < 1) continue;
    lo = std::max(lo, 1);
    if (!fits(lo)) continue;
    while (lo < hi) {  // the layout grows with c inside the stretch
      const int mid = lo + (hi - lo + 1) / 2;
      if (fits(mid)) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  return 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode entry point: one fixed array in each
// GPU's memory, held until the process ends.  In host code `scratch` is only
// a host-side handle; its device address (one per GPU) comes from
// hipGetSymbolAddress on the entry point's first call on that GPU, with the
// GPU current, and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current GPU (looked up once per GPU).
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* dsa_version(void) { return "dsa-mi355x 0.1.0 gfx950"; }

const char* dsa_last_error(void) { return g_err; }

dsa_status_t dsa_index_scores(const void* q_idx, int q_dtype, const float* q_scale,
                              const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I,
                              const int32_t* cu_q, const int32_t* ctx_len, const int64_t* cu_ctx,
                              int B, int T, int max_q, int max_ctx, float* scores, int64_t ld,
                              void* stream) {
  TraceRange tr("dsa_index_scores");
  DSA_PTR(q_idx, "q_idx");
  {
    const dsa_status_t qs = check_query_dtype(q_dtype, q_scale, k_dtype);
    if (qs != DSA_OK) return qs;
  }
  DSA_REQUIRE(q_dtype == DSA_QUERY_BF16 || cu_q != nullptr, DSA_ERR_UNSUPPORTED,
              "fp8 query heads are scored by the prefill contraction: pass cu_q");
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
                                 cu_ctx, B, max_ctx, scores, ld, nullptr, nullptr, s);
  else
    e = dsa::launch_index_prefill(q_idx, q_dtype, q_scale, w, w_ld, k_idx, k_dtype, k_scale, H_I,
                                  d_I, cu_q, ctx_len, cu_ctx, B, max_q, max_ctx, scores, ld, s);
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
  TraceRange tr("dsa_topk");
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
  } else {
    e = dsa::launch_tile_reports(scores, ld, cu_q, ctx_len, B, T, K, w, s);
    if (e == hipSuccess) e = dsa::launch_topk_resolve(scores, ld, cu_q, ctx_len, B, T, K, w, idx,
                                                      t_topk_counters, s);
  }
  if (e == hipSuccess) e = check_selected(idx, K, cu_q, ctx_len, B, T, s);
  return hip_status(e, "dsa_topk");
}

dsa_status_t dsa_cache_append(const void* k_idx_new, int d_I, const void* k_new,
                              const void* v_new, int D, const int32_t* cu_q,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                              void* k_idx_cache, int k_dtype, float* k_scale_cache,
                              void* k_cache, void* v_cache, void* stream) {
  TraceRange tr("dsa_cache_append");
  DSA_REQUIRE(B >= 1 && T >= 1, DSA_ERR_INVALID_ARG, "B and T must be >= 1 (got %d, %d)", B, T);
  DSA_REQUIRE(ctx_len != nullptr && cu_ctx != nullptr, DSA_ERR_INVALID_ARG,
              "ctx_len and cu_ctx must not be NULL");
  DSA_REQUIRE(cu_q != nullptr || T == B, DSA_ERR_INVALID_ARG,
              "cu_q == NULL means one new token per sequence: T (%d) must equal B (%d)", T, B);
  if (k_idx_new) {
    DSA_PTR(k_idx_new, "k_idx_new");
    DSA_PTR(k_idx_cache, "k_idx_cache");
    DSA_REQUIRE(d_I == 64 || d_I == 128, DSA_ERR_UNSUPPORTED, "d_I must be 64 or 128 (got %d)",
                d_I);
    DSA_REQUIRE(k_dtype == DSA_KEY_BF16 || k_dtype == DSA_KEY_FP8_E4M3, DSA_ERR_INVALID_ARG,
                "k_dtype must be DSA_KEY_BF16 or DSA_KEY_FP8_E4M3 (got %d)", k_dtype);
    if (k_dtype == DSA_KEY_FP8_E4M3)
      DSA_REQUIRE(k_scale_cache != nullptr, DSA_ERR_INVALID_ARG, "an fp8 key cache needs k_scale_cache");
  }
  if (k_new || v_new) {
    DSA_REQUIRE(D == 64 || D == 128, DSA_ERR_UNSUPPORTED, "D must be 64 or 128 (got %d)", D);
    if (k_new) {
      DSA_PTR(k_new, "k_new");
      DSA_PTR(k_cache, "k_cache");
    }
    if (v_new) {
      DSA_PTR(v_new, "v_new");
      DSA_PTR(v_cache, "v_cache");
    }
  }
  if (!k_idx_new && !k_new && !v_new) return ok();
  hipError_t e = dsa::launch_cache_append(k_idx_new, d_I, k_new, v_new, D, cu_q, ctx_len, cu_ctx,
                                          B, T, k_idx_cache, k_dtype, k_scale_cache, k_cache,
                                          v_cache, static_cast<hipStream_t>(stream));
  return hip_status(e, "dsa_cache_append");
}

size_t dsa_sparse_attn_workspace_size(int B, int T, int K, int window, int Hq, int D) {
  (void)B;
  if (T < 1) return 0;
  return dsa::attn_plan(T, K, window, Hq, D).ws_bytes;
}

dsa_status_t dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* idx, int K, int window, const void* gate,
                             int64_t gate_stride_d, float sm_scale, int Hq, int D,
                             const int32_t* cu_q,
                             const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                             int max_q, int max_ctx, void* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  TraceRange tr("dsa_sparse_attn");
  DSA_PTR(q, "q");
  DSA_PTR(k_cache, "k_cache");
  DSA_PTR(v_cache, "v_cache");
  DSA_PTR(out, "out");
  if (gate) DSA_PTR(gate, "gate");
  if (idx) DSA_PTR(idx, "idx");
  DSA_REQUIRE(gate_stride_d == 0 || gate_stride_d == 1, DSA_ERR_INVALID_ARG,
              "gate_stride_d must be 1 (elementwise gate) or 0 (one gate per head), got %lld",
              (long long)gate_stride_d);
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (idx && t_idx_checks)  // the caller's rows, before they are gathered with
    e = dsa::launch_check_index_rows(idx, K, cu_q, ctx_len, B, T, false, t_idx_checks, s);
  if (e == hipSuccess)
    e = dsa::launch_sparse_attn(q, k_cache, v_cache, idx, K, idx ? 0 : window, gate,
                                (int)gate_stride_d, sm_scale, Hq, D, cu_q, ctx_len, cu_ctx, B, T,
                                out, lse, ws, plan, s);
  return hip_status(e, "dsa_sparse_attn");
}

dsa_status_t dsa_swa_decode_layers(int n_layers, const void* const* q, const void* const* k_cache,
                                   const void* const* v_cache, const void* const* gate,
                                   int64_t gate_stride_d, int window, float sm_scale, int Hq,
                                   int D, const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                   int max_ctx, void* const* out, void* stream) {
  TraceRange tr("dsa_swa_decode_layers");
  DSA_REQUIRE(n_layers >= 1 && n_layers <= dsa::kMaxAttnLayers, DSA_ERR_UNSUPPORTED,
              "n_layers must be in [1, %d] (got %d)", dsa::kMaxAttnLayers, n_layers);
  DSA_REQUIRE(q && k_cache && v_cache && out, DSA_ERR_INVALID_ARG,
              "q, k_cache, v_cache and out must be arrays of n_layers pointers");
  DSA_REQUIRE(gate_stride_d == 0 || gate_stride_d == 1, DSA_ERR_INVALID_ARG,
              "gate_stride_d must be 1 (elementwise gate) or 0 (one gate per head), got %lld",
              (long long)gate_stride_d);
  dsa::AttnLayers lay;
  lay.n = n_layers;
  for (int i = 0; i < n_layers; ++i) {
    DSA_PTR(q[i], "q[layer]");
    DSA_PTR(k_cache[i], "k_cache[layer]");
    DSA_PTR(v_cache[i], "v_cache[layer]");
    DSA_PTR(out[i], "out[layer]");
    const void* g = gate ? gate[i] : nullptr;
    if (g) DSA_PTR(g, "gate[layer]");
    lay.q[i] = static_cast<const uint16_t*>(q[i]);
    lay.kc[i] = static_cast<const uint16_t*>(k_cache[i]);
    lay.vc[i] = static_cast<const uint16_t*>(v_cache[i]);
    lay.gate[i] = static_cast<const uint16_t*>(g);
    lay.out[i] = static_cast<uint16_t*>(out[i]);
  }
  dsa_status_t st = check_batch(nullptr, ctx_len, cu_ctx, true, B, B, 1, max_ctx);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(attn_shape_ok(Hq, D), DSA_ERR_UNSUPPORTED,
              "unsupported attention shape Hq=%d D=%d (supported: 8x64, 64x128)", Hq, D);
  DSA_REQUIRE(window >= 1 && window <= 4096, DSA_ERR_UNSUPPORTED,
              "window must be in [1, 4096] (got %d)", window);
  DSA_REQUIRE(sm_scale >= 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be >= 0");
  // one workgroup per (layer, sequence) over its whole window
  dsa::AttnPlan plan;
  plan.nsplit = 1;
  plan.rows_per_split = window;
  plan.ws_bytes = 0;
  hipError_t e = dsa::launch_sparse_attn(lay.q[0], lay.kc[0], lay.vc[0], nullptr, 0, window,
                                         lay.gate[0], (int)gate_stride_d, sm_scale, Hq, D,
                                         nullptr, ctx_len, cu_ctx, B, B, lay.out[0], nullptr,
                                         nullptr, plan, static_cast<hipStream_t>(stream), &lay);
  return hip_status(e, "dsa_swa_decode_layers");
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

dsa_status_t dsa_set_index_checks(uint32_t* counters) {
  t_idx_checks = counters;
  return DSA_OK;
}

dsa_status_t dsa_check_index_rows(const int32_t* idx, int K, const int32_t* cu_q,
                                  const int32_t* ctx_len, int B, int T, int full,
                                  uint32_t* counters, void* stream) {
  TraceRange tr("dsa_check_index_rows");
  DSA_PTR(idx, "idx");
  DSA_PTR(counters, "counters");
  DSA_REQUIRE(ctx_len != nullptr, DSA_ERR_INVALID_ARG, "ctx_len must not be NULL");
  DSA_REQUIRE(B >= 1 && T >= 1, DSA_ERR_INVALID_ARG, "B and T must be >= 1 (got %d, %d)", B, T);
  DSA_REQUIRE(cu_q != nullptr || T == B, DSA_ERR_INVALID_ARG,
              "cu_q == NULL means one row per sequence: T (%d) must equal B (%d)", T, B);
  DSA_REQUIRE(K >= 1, DSA_ERR_INVALID_ARG, "K must be >= 1 (got %d)", K);
  const hipError_t e = dsa::launch_check_index_rows(idx, K, cu_q, ctx_len, B, T, full != 0,
                                                    counters, static_cast<hipStream_t>(stream));
  return hip_status(e, "dsa_check_index_rows");
}

dsa_status_t dsa_set_indexer_events(void* start, void* stop) {
  DSA_REQUIRE((start == nullptr) == (stop == nullptr), DSA_ERR_INVALID_ARG,
              "start and stop events must both be set or both be NULL");
  t_ev_start = static_cast<hipEvent_t>(start);
  t_ev_stop = static_cast<hipEvent_t>(stop);
  return DSA_OK;
}

static dsa_status_t layer_decode_impl(
    const void* q_idx, const void* w, int64_t w_ld, const void* k_idx, int k_dtype,
    const float* k_scale, int H_I, int d_I, const void* q, const void* k_cache,
    const void* v_cache, const void* gate, int64_t gate_stride_d, float sm_scale, int Hq, int D,
    int K, const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_ctx, void* out,
    int32_t* idx_out, void* ws, size_t ws_bytes, const dsa::DecodeAppend* app, void* stream,
    const char* fn) {
  DSA_PTR(q_idx, "q_idx");
  DSA_PTR(w, "w");
  DSA_PTR(k_idx, "k_idx");
  DSA_PTR(q, "q");
  DSA_PTR(k_cache, "k_cache");
  DSA_PTR(v_cache, "v_cache");
  DSA_PTR(out, "out");
  if (gate) DSA_PTR(gate, "gate");
  if (idx_out) DSA_PTR(idx_out, "idx_out");
  DSA_REQUIRE(gate_stride_d == 0 || gate_stride_d == 1, DSA_ERR_INVALID_ARG,
              "gate_stride_d must be 1 (elementwise gate) or 0 (one gate per head), got %lld",
              (long long)gate_stride_d);
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
  if (app) {
    DSA_PTR(app->k_idx_new, "k_idx_new");
    if (app->k_new) DSA_PTR(app->k_new, "k_new");
    if (app->v_new) DSA_PTR(app->v_new, "v_new");
  }
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
                                          rows ? nullptr : &L.topk, app, s, t_ev_start,
                                          t_ev_stop);
  const dsa::AttnPlan plan = dsa::attn_plan(B, K, 0, Hq, D);
  if (!rows && dsa::select_attend_fits(B, K, plan.nsplit, plan.rows_per_split, Hq, D)) {
    // few sequences: the selection runs inside the split attention's launch
    // (each split repeats it in its own LDS), then the combine
    if (e == hipSuccess)
      e = dsa::launch_select_attend(L.scores, L.ld, ctx_len, B, K, L.topk, idx, t_topk_counters,
                                    q, k_cache, v_cache, cu_ctx, sm_scale,
                                    static_cast<float*>(L.attn), plan.nsplit, s);
    if (e == hipSuccess) e = check_selected(idx, K, nullptr, ctx_len, B, B, s);
    if (e == hipSuccess)
      e = dsa::launch_attn_combine(B, Hq, D, static_cast<const float*>(L.attn), plan.nsplit, gate,
                                   (int)gate_stride_d, out, nullptr, s);
    return hip_status(e, fn);
  }
  if (e == hipSuccess)
    e = rows ? dsa::launch_topk_rows(L.scores, L.ld, nullptr, ctx_len, B, B, K, idx,
                                     t_topk_counters, s)
             : dsa::launch_topk_resolve(L.scores, L.ld, nullptr, ctx_len, B, B, K, L.topk, idx,
                                        t_topk_counters, s);
  if (e == hipSuccess) e = check_selected(idx, K, nullptr, ctx_len, B, B, s);
  if (e == hipSuccess)
    e = dsa::launch_sparse_attn(q, k_cache, v_cache, idx, K, 0, gate, (int)gate_stride_d,
                                sm_scale, Hq, D, nullptr, ctx_len, cu_ctx, B, B, out, nullptr,
                                L.attn, plan, s);
  return hip_status(e, fn);
}

dsa_status_t dsa_layer_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I, const void* q,
                              const void* k_cache, const void* v_cache, const void* gate,
                              int64_t gate_stride_d, float sm_scale, int Hq, int D, int K,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int max_ctx,
                              void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                              void* stream) {
  TraceRange tr("dsa_layer_decode");
  return layer_decode_impl(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, q, k_cache,
                           v_cache, gate, gate_stride_d, sm_scale, Hq, D, K, ctx_len, cu_ctx, B,
                           max_ctx, out, idx_out, ws, ws_bytes, nullptr, stream,
                           "dsa_layer_decode");
}

dsa_status_t dsa_layer_decode_append(const void* q_idx, const void* w, int64_t w_ld, void* k_idx,
                                     int k_dtype, float* k_scale, int H_I, int d_I, const void* q,
                                     void* k_cache, void* v_cache, const void* gate,
                                     int64_t gate_stride_d, float sm_scale, int Hq, int D, int K,
                                     const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                     int max_ctx, const void* k_idx_new, const void* k_new,
                                     const void* v_new, void* out, int32_t* idx_out, void* ws,
                                     size_t ws_bytes, void* stream) {
  TraceRange tr("dsa_layer_decode_append");
  dsa::DecodeAppend app;
  app.k_idx_new = static_cast<const uint16_t*>(k_idx_new);
  app.k_new = static_cast<const uint16_t*>(k_new);
  app.v_new = static_cast<const uint16_t*>(v_new);
  app.k_idx_cache = static_cast<uint8_t*>(k_idx);
  app.k_scale_cache = k_scale;
  app.k_cache = static_cast<uint16_t*>(k_cache);
  app.v_cache = static_cast<uint16_t*>(v_cache);
  app.D = D;
  return layer_decode_impl(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, q, k_cache,
                           v_cache, gate, gate_stride_d, sm_scale, Hq, D, K, ctx_len, cu_ctx, B,
                           max_ctx, out, idx_out, ws, ws_bytes, &app, stream,
                           "dsa_layer_decode_append");
}

size_t dsa_layer_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

dsa_status_t dsa_layer_decode_noalloc(const void* q_idx, const void* w, int64_t w_ld,
                                      const void* k_idx, int k_dtype, const float* k_scale,
                                      int H_I, int d_I, const void* q, const void* k_cache,
                                      const void* v_cache, const void* gate,
                                      int64_t gate_stride_d, float sm_scale, int Hq, int D, int K,
                                      const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                      int max_ctx, void* out, int32_t* idx_out, void* stream) {
  TraceRange tr("dsa_layer_decode_noalloc");
  // the size check comes first: an oversize call is refused without
  // touching the GPU
  DSA_REQUIRE(B >= 1 && max_ctx >= 1 && K >= 1, DSA_ERR_INVALID_ARG,
              "B, max_ctx and K must be >= 1 (got %d, %d, %d)", B, max_ctx, K);
  const size_t need = (K <= 4096 && attn_shape_ok(Hq, D))
                          ? decode_ws_layout(B, max_ctx, K, Hq, D, nullptr, nullptr)
                          : 0;
  DSA_REQUIRE(need <= kNoAllocScratchBytes, DSA_ERR_WORKSPACE,
              "dsa_layer_decode_noalloc: this call needs %zu bytes of scratch, more than the "
              "library's fixed %zu (B * max_ctx too large; use dsa_layer_decode with a "
              "caller workspace)",
              need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = scratch_for_current_device(&ws);
  if (e != hipSuccess) return hip_status(e, "dsa_layer_decode_noalloc: scratch lookup");
  return dsa_layer_decode(q_idx, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, q, k_cache, v_cache,
                          gate, gate_stride_d, sm_scale, Hq, D, K, ctx_len, cu_ctx, B, max_ctx,
                          out, idx_out, ws, kNoAllocScratchBytes, stream);
}

size_t dsa_layer_prefill_workspace_size(int B, int T, int max_ctx, int K, int Hq, int D) {
  (void)B;
  if (T < 1 || max_ctx < 1 || K < 1) return 0;
  return prefill_ws_layout(T, max_ctx, K, Hq, D, nullptr, nullptr);
}

size_t dsa_layer_prefill_min_workspace_size(int B, int max_ctx, int K, int Hq, int D) {
  if (B < 1 || max_ctx < 1 || K < 1) return 0;
  return prefill_chunk_desc_bytes(B) + prefill_ws_layout(1, max_ctx, K, Hq, D, nullptr, nullptr);
}

dsa_status_t dsa_layer_prefill(const void* q_idx, int q_dtype, const float* q_scale,
                               const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const void* q, const void* k_cache, const void* v_cache,
                               const void* gate, int64_t gate_stride_d, float sm_scale, int Hq,
                               int D, int K, const int32_t* cu_q, const int32_t* ctx_len,
                               const int64_t* cu_ctx, int B, int T, int max_q, int max_ctx,
                               void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                               void* stream) {
  TraceRange tr("dsa_layer_prefill");
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
  {
    const dsa_status_t qs = check_query_dtype(q_dtype, q_scale, k_dtype);
    if (qs != DSA_OK) return qs;
  }
  DSA_REQUIRE(gate_stride_d == 0 || gate_stride_d == 1, DSA_ERR_INVALID_ARG,
              "gate_stride_d must be 1 (elementwise gate) or 0 (one gate per head), got %lld",
              (long long)gate_stride_d);
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
  DSA_PTR(ws, "ws");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t full = prefill_ws_layout(T, max_ctx, K, Hq, D, nullptr, nullptr);
  if (ws_bytes >= full) {
    DecodeWs L;
    prefill_ws_layout(T, max_ctx, K, Hq, D, static_cast<char*>(ws), &L);
    const hipError_t e = prefill_pass(q_idx, q_dtype, q_scale, w, w_ld, k_idx, k_dtype, k_scale,
                                      H_I, d_I, q,
                                      k_cache, v_cache, gate, (int)gate_stride_d, sm_scale, Hq, D,
                                      K, cu_q, ctx_len, cu_ctx, B, T, T, max_q, max_ctx, out,
                                      idx_out ? idx_out : L.idx, L, s);
    return hip_status(e, "dsa_layer_prefill");
  }
  // Sub-chunks of tc rows: the largest tc whose layout fits next to the
  // chunk descriptor.  (The layout is not monotone in the row count: calls
  // of many rows skip the Top-K reports and the attention partials.)
  const size_t desc = prefill_chunk_desc_bytes(B);
  const size_t need_min = desc + prefill_ws_layout(1, max_ctx, K, Hq, D, nullptr, nullptr);
  DSA_REQUIRE(ws_bytes >= need_min, DSA_ERR_WORKSPACE,
              "workspace too small: %zu < %zu bytes (the least that runs one query row at a "
              "time; %zu bytes run all %d rows in one pass)",
              ws_bytes, need_min, full, T);
  const int tc = prefill_chunk_rows(T, max_ctx, K, Hq, D, ws_bytes - desc);
  DSA_REQUIRE(tc >= 1, DSA_ERR_WORKSPACE, "workspace too small: %zu bytes", ws_bytes);
  char* base = static_cast<char*>(ws);
  int32_t* cu_q_c = reinterpret_cast<int32_t*>(base);
  int32_t* ctx_len_c = cu_q_c + align_up((size_t)B + 1, 64);
  DecodeWs L;
  prefill_ws_layout(tc, max_ctx, K, Hq, D, base + desc, &L);
  const int64_t gate_row = (int64_t)Hq * (gate_stride_d ? D : 1);
  hipError_t e = hipSuccess;
  for (int t0 = 0; t0 < T && e == hipSuccess; t0 += tc) {
    const int n = T - t0 < tc ? T - t0 : tc;
    e = dsa::launch_chunk_desc(cu_q, ctx_len, B, t0, n, cu_q_c, ctx_len_c, s);
    if (e != hipSuccess) break;
    // every per-row input and output is row-major in the query rows
    e = prefill_pass(
        static_cast<const uint8_t*>(q_idx) + (int64_t)t0 * H_I * d_I * (q_dtype ? 1 : 2),
        q_dtype, q_scale ? q_scale + (int64_t)t0 * H_I : nullptr,
        static_cast<const uint16_t*>(w) + (int64_t)t0 * w_ld, w_ld, k_idx, k_dtype, k_scale,
        H_I, d_I, static_cast<const uint16_t*>(q) + (int64_t)t0 * Hq * D, k_cache, v_cache,
        gate ? static_cast<const uint16_t*>(gate) + t0 * gate_row : nullptr, (int)gate_stride_d,
        sm_scale, Hq, D, K, cu_q_c, ctx_len_c, cu_ctx, B, n, tc, max_q < n ? max_q : n, max_ctx,
        static_cast<uint16_t*>(out) + (int64_t)t0 * Hq * D,
        idx_out ? idx_out + (int64_t)t0 * K : L.idx, L, s);
  }
  return hip_status(e, "dsa_layer_prefill");
}

}  // extern "C"
