/*
 * dsa.h -- C ABI of the MI355X (gfx950) Gated DSA library, libdsa.so.
 *
 * The Gated DSA layer (DeepSeek Sparse Attention with an output gate) has
 * three steps, as the pages describe it:
 *   1. a lightweight multi-head Indexer scores every causal past position
 *      for each query ("Open-Source LLM Architecture Evolution ...",
 *      Architecture Breakdown, item 2; "Fine-Grained Sparse Attention in
 *      Ultra-Large Parameter Models", sections 2.1-2.3: 32 heads x 128 dim,
 *      no RoPE);
 *   2. a per-query Top-K keeps the K best positions (same item; K = 2048);
 *   3. softmax attention runs over the gathered K/V rows of those positions
 *      only ("Technical Deep Dive", item 2) and a gate is applied to its
 *      output ("Gated" DSA; the deployment page, section 2).
 *
 * Score, selection and gate readings (the pages print no formula):
 *   score  s[t,j] = sum_h w[t,h] * max(0, sigma_j * dot(qI[t,h,:], kI[j,:]))
 *   select the K_eff = min(K, p+1) best positions j <= p, ties to the lower
 *          position, -0.0 == +0.0, emitted in ascending order, padded with -1
 *   attend o[t,h,:] = softmax_j(c * dot(q[t,h,:], K[j,:])) @ V[j,:]
 *   gate   out[t,h,d] = o[t,h,d] * sigmoid(g[t,h,d])
 *
 * Conventions (all entry points):
 *   - Every tensor argument is a DEVICE pointer owned by the caller; the
 *     library never allocates or frees device memory.  Scratch memory is a
 *     caller-provided device buffer (ws, ws_bytes) sized by the matching
 *     *_workspace_size() call.
 *   - Every call is asynchronous on the caller's HIP stream (hipStream_t
 *     passed as void*; NULL is the default stream) and never synchronises.
 *   - Tensors are dense and row-major.  Device pointers must be 16-byte
 *     aligned.  bf16 is IEEE binary32 truncated to its upper 16 bits; fp8 is
 *     OCP E4M3FN.
 *   - Batch descriptor: B sequences, T query rows in total.
 *       cu_q    device int32 [B+1], query-row offsets per sequence; NULL
 *               means one query per sequence (decode: T == B, row t is
 *               sequence t).
 *       ctx_len device int32 [B], context length of each sequence including
 *               its new queries.
 *       cu_ctx  device int64 [B+1], first cache row of each sequence in the
 *               packed caches.
 *       max_q, max_ctx are host upper bounds of the per-sequence query count
 *       and of ctx_len (grid sizing only).
 *     Query i of sequence b sits at position p = ctx_len[b] - n_q[b] + i and
 *     sees positions 0..p (its own row is already in the cache).  Returned
 *     positions are relative to the sequence (0 .. ctx_len[b]-1).
 *   - Errors: every call validates its host-side arguments before touching
 *     the GPU.  DSA_ERR_INVALID_ARG / DSA_ERR_UNSUPPORTED / DSA_ERR_WORKSPACE
 *     mean nothing was launched.  DSA_ERR_HIP means a HIP call failed.  The
 *     text of the last error of the calling thread is dsa_last_error().
 *     Device-side values (descriptor contents, indices) are trusted; indices
 *     outside 0..p or duplicated are the caller's error.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE = 3,
  DSA_ERR_HIP = 4
} dsa_status_t;

typedef enum dsa_key_dtype {
  DSA_KEY_BF16 = 0,     /* indexer keys bf16 [rows, d_I]; k_scale must be NULL      */
  DSA_KEY_FP8_E4M3 = 1  /* indexer keys fp8 e4m3fn [rows, d_I] + fp32 scale [rows] */
} dsa_key_dtype_t;

/* Library version string, e.g. "dsa-mi355x 0.1.0 gfx950".  Never fails. */
const char* dsa_version(void);

/* Text of the last error raised on the calling thread ("" if none). */
const char* dsa_last_error(void);

/* ------------------------------------------------------------------------ */
/* Step 1: Indexer scores.                                                   */
/* Pages: "Open-Source LLM Architecture Evolution ...", Architecture         */
/* Breakdown item 2 (Indexer: multi-head, fast global scan of historical     */
/* positions); "Fine-Grained Sparse Attention ...", 2.2 (no RoPE) and 2.3    */
/* (32 heads x 128 dim); the naive-n0-5-flash page (16-head indexer).        */
/*                                                                           */
/*   scores[t, j] = sum_h w[t*w_ld + h] *                                    */
/*                  max(0, sigma_j * sum_d q_idx[t,h,d] * k_idx[row(j), d])  */
/* for j = 0..p_t, with sigma_j = k_scale[row(j)] for fp8 keys, 1 for bf16.  */
/* Entries j > p_t of each score row are left untouched.                     */
/*                                                                           */
/*   q_idx   bf16 [T, H_I, d_I]                                              */
/*   w       bf16 head weights; row t at w + t*w_ld (w_ld == 0: one row     */
/*           shared by every query, i.e. static per-layer weights)           */
/*   k_idx   indexer key cache [sum ctx_len, d_I], bf16 or fp8 e4m3fn        */
/*   k_scale fp32 [sum ctx_len] per-token scale for fp8 keys, else NULL      */
/*   scores  fp32 [T, ld], ld >= max_ctx                                     */
/* Supported (H_I, d_I): (4,64), (16,128), (32,128).                         */
/* ------------------------------------------------------------------------ */
dsa_status_t dsa_index_scores(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I,
                              const int32_t* cu_q, const int32_t* ctx_len, const int64_t* cu_ctx,
                              int B, int T, int max_q, int max_ctx, float* scores, int64_t ld,
                              void* stream);

/* ------------------------------------------------------------------------ */
/* Step 2: exact Top-K of each score row.                                    */
/* Pages: "Open-Source LLM Architecture Evolution ...", Architecture         */
/* Breakdown item 2 (keep the K highest-scoring positions, K = 2048);        */
/* "Fine-Grained Sparse Attention ...", 2.1.                                 */
/*                                                                           */
/* For row t, keeps the K_eff = min(K, p_t + 1) best positions of            */
/* scores[t, 0..p_t] by (score descending, position ascending), with -0.0   */
/* equal to +0.0, writes them to idx[t, 0..K_eff-1] in ascending order and  */
/* fills idx[t, K_eff..K-1] with -1.  Deterministic; bit-identical to the   */
/* plain definition for any finite fp32 input (NaN rows are unspecified).    */
/*                                                                           */
/*   scores fp32 [T, ld];  idx int32 [T, K];  1 <= K <= 4096.                */
/* ------------------------------------------------------------------------ */
size_t dsa_topk_workspace_size(int B, int T, int max_ctx, int K);
dsa_status_t dsa_topk(const float* scores, int64_t ld, const int32_t* cu_q,
                      const int32_t* ctx_len, int B, int T, int max_q, int max_ctx, int K,
                      int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Step 3: gated sparse attention over the selected rows.                    */
/* Pages: "Open-Source LLM Architecture Evolution ...", Technical Deep Dive  */
/* item 2 (scores and softmax over the 2048 selected elements only) and      */
/* Architecture Breakdown item 2 (gating unit); the deployment page,         */
/* section 2 (gated DSA layers); sliding-window mode: the naive-n0-5-flash   */
/* page (SWA layers with a 128-token window).                                */
/*                                                                           */
/* For query row t and head h (all Hq heads share one K/V head and one       */
/* index row):                                                               */
/*   S = idx[t, :] without -1 entries   (idx != NULL), or                    */
/*   S = {max(0, p_t - window + 1) .. p_t}   (idx == NULL, window >= 1)      */
/*   o = softmax_{j in S}(c * q[t,h,:] . K[row(j),:]) @ V[row(j),:]          */
/*   out[t,h,:] = o * sigmoid(gate[t,h,:])   (gate == NULL: out = o)         */
/* c = sm_scale, or 1/sqrt(D) when sm_scale == 0.  lse (optional, fp32       */
/* [T, Hq]) receives log(sum_j exp(c * q.K_j)).  An empty S gives out = 0.   */
/*                                                                           */
/*   q, gate, out  bf16 [T, Hq, D];  k_cache, v_cache bf16 [sum ctx_len, D]  */
/*   idx int32 [T, K] or NULL                                                */
/* Supported (Hq, D): (8, 64), (64, 128); K <= 4096; window <= 4096.         */
/* ------------------------------------------------------------------------ */
size_t dsa_sparse_attn_workspace_size(int B, int T, int K, int window, int Hq, int D);
dsa_status_t dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* idx, int K, int window, const void* gate,
                             float sm_scale, int Hq, int D, const int32_t* cu_q,
                             const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                             int max_q, int max_ctx, void* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Whole layer, decode: one new query per sequence (T == B).                 */
/* Steps 1 -> 2 -> 3 above on the caller's stream, with the step-1 kernel   */
/* also emitting the per-tile candidate lists that step 2 certifies (the     */
/* selection is still exact).  Arguments are those of the three steps;       */
/* idx_out (int32 [B, K], or NULL) receives the selected positions, which   */
/* otherwise stay in the workspace.                                          */
/* ------------------------------------------------------------------------ */
size_t dsa_layer_decode_workspace_size(int B, int max_ctx, int K, int Hq, int D);
dsa_status_t dsa_layer_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I, const void* q,
                              const void* k_cache, const void* v_cache, const void* gate,
                              float sm_scale, int Hq, int D, int K, const int32_t* ctx_len,
                              const int64_t* cu_ctx, int B, int max_ctx, void* out,
                              int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* Measurement hook: on the calling thread, every later dsa_layer_decode    */
/* call launches its step-1 indexer kernel with `start` and `stop` (both    */
/* hipEvent_t) attached to the dispatch, which records them when that       */
/* kernel starts and ends, so the caller can time it inside a running       */
/* sequence of layer calls.  The events stay owned by the caller and must   */
/* outlive their use; pass NULL, NULL to stop.                              */
/* Returns DSA_ERR_INVALID_ARG if exactly one of them is NULL.               */
dsa_status_t dsa_set_indexer_events(void* start, void* stop);

/* Diagnostic hook: on the calling thread, every later Top-K selection     */
/* (dsa_topk, dsa_layer_decode, dsa_layer_prefill) adds, per row, 1 to one  */
/* of the first four of five caller-owned device counters (uint32 [5],     */
/* zeroed by the caller) naming the path that produced the row: [0] the     */
/* union of the row's sub-tile candidate reports, certified exact; [1] the  */
/* exact radix select over the whole score row (certification failed, or a  */
/* key shared by too many positions); [2] the direct select of a row of at  */
/* most 16384 positions; [3] the collection sweep over the row's scores     */
/* used when a call has 1024 rows or more.  [4] counts the rows of [3]      */
/* whose collection threshold came from a sample of the row (one sweep      */
/* instead of histogram sweeps first).  Rows with at most K positions take  */
/* none of them.  Pass NULL to stop.  Always DSA_OK.                        */
dsa_status_t dsa_set_topk_counters(uint32_t* counters);

/* ------------------------------------------------------------------------ */
/* Whole layer, prefill: a chunk of new queries per sequence (cu_q given).   */
/* Same steps; the indexer runs as a dense bf16 MFMA contraction of the      */
/* chunk's query heads against the key cache with causal tile skipping.      */
/* ------------------------------------------------------------------------ */
size_t dsa_layer_prefill_workspace_size(int B, int T, int max_ctx, int K, int Hq, int D);
dsa_status_t dsa_layer_prefill(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const void* q, const void* k_cache, const void* v_cache,
                               const void* gate, float sm_scale, int Hq, int D, int K,
                               const int32_t* cu_q, const int32_t* ctx_len,
                               const int64_t* cu_ctx, int B, int T, int max_q, int max_ctx,
                               void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
