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

/* Indexer query heads: bf16 [T, H_I, d_I] (q_scale NULL), or E4M3FN codes   */
/* [T, H_I, d_I] with one positive fp32 scale per query and head, q_scale    */
/* [T, H_I], which multiplies that head's dot product like the key scale.    */
/* fp8 query heads need an fp8 key cache and run on the fp8 MFMA; they are   */
/* taken by the prefill contraction (cu_q given), not by the decode kernel.  */
/* The fp8 MFMA epilogue assumes both scales positive (what a quantiser's    */
/* absolute-maximum scale is); other scales give unspecified scores.        */
typedef enum dsa_query_dtype {
  DSA_QUERY_BF16 = 0,
  DSA_QUERY_FP8_E4M3 = 1
} dsa_query_dtype_t;

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
/*                  max(0, rho_th * sigma_j *                                */
/*                         sum_d q_idx[t,h,d] * k_idx[row(j), d])            */
/* for j = 0..p_t, with sigma_j = k_scale[row(j)] for fp8 keys, 1 for bf16, */
/* and rho_th = q_scale[t, h] for fp8 query heads, 1 for bf16.               */
/* Entries j > p_t of each score row are left untouched.                     */
/*                                                                           */
/*   q_idx   [T, H_I, d_I], bf16 or E4M3FN codes (q_dtype, q_scale: above)   */
/*   w       bf16 head weights; row t at w + t*w_ld (w_ld == 0: one row     */
/*           shared by every query, i.e. static per-layer weights)           */
/*   k_idx   indexer key cache [sum ctx_len, d_I], bf16 or fp8 e4m3fn        */
/*   k_scale fp32 [sum ctx_len] per-token scale for fp8 keys, else NULL      */
/*   scores  fp32 [T, ld], ld >= max_ctx                                     */
/* Supported (H_I, d_I): (4,64), (16,128), (32,128).                         */
/* ------------------------------------------------------------------------ */
dsa_status_t dsa_index_scores(const void* q_idx, int q_dtype, const float* q_scale,
                              const void* w, int64_t w_ld, const void* k_idx,
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
/* Cache append: the new tokens' rows go into the caches before the layer    */
/* reads them (the naive-n0-5-flash page, Key Capabilities: FP8 mixed        */
/* precision; an fp8 indexer key cache holds E4M3FN codes and one fp32      */
/* scale per token).  For query row t of the batch descriptor (position p_t */
/* of sequence b), cache row r = cu_ctx[b] + p_t receives:                  */
/*   k_idx_cache[r, :]  bf16 cache: k_idx_new[t, :] as is;                   */
/*                      fp8 cache: codes of y_d = k_idx_new[t, d] / s,       */
/*                      rounded to the nearest E4M3FN value (ties to even)   */
/*                      after clamping to +-448, with s = max_d |k_idx_new|  */
/*                      / 448 in fp32 (1 for an all-zero row);               */
/*   k_scale_cache[r]   s (fp8 cache only);                                  */
/*   k_cache[r, :], v_cache[r, :]  k_new[t, :], v_new[t, :].                 */
/* Any of k_idx_new, k_new, v_new may be NULL (that cache is left alone).    */
/* Call it with the descriptor of the layer call that follows (decode:       */
/* cu_q = NULL, the new token at ctx_len[b] - 1).                            */
/*   k_idx_new bf16 [T, d_I], d_I in {64, 128};  k_new, v_new bf16 [T, D],  */
/*   D in {64, 128}.                                                         */
/* ------------------------------------------------------------------------ */
dsa_status_t dsa_cache_append(const void* k_idx_new, int d_I, const void* k_new,
                              const void* v_new, int D, const int32_t* cu_q,
                              const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                              void* k_idx_cache, int k_dtype, float* k_scale_cache,
                              void* k_cache, void* v_cache, void* stream);

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
/*   S = the entries of idx[t, :] in [0, p_t]   (idx != NULL; -1 padding,   */
/*       and any other entry outside that range, is skipped), or            */
/*   S = {max(0, p_t - window + 1) .. p_t}   (idx == NULL, window >= 1)      */
/*   o = softmax_{j in S}(c * q[t,h,:] . K[row(j),:]) @ V[row(j),:]          */
/*   out[t,h,:] = o * sigmoid(gate[t,h,:])   (gate == NULL: out = o)         */
/* c = sm_scale, or 1/sqrt(D) when sm_scale == 0.  lse (optional, fp32       */
/* [T, Hq]) receives log(sum_j exp(c * q.K_j)).  An empty S gives out = 0.   */
/*                                                                           */
/*   q, out  bf16 [T, Hq, D];  k_cache, v_cache bf16 [sum ctx_len, D]        */
/*   gate    bf16 [T, Hq, D] with gate_stride_d == 1 (one gate value per     */
/*           output element), or [T, Hq] with gate_stride_d == 0 (one value  */
/*           per head, applied to all D dims of it); ignored when NULL       */
/*   idx int32 [T, K] or NULL                                                */
/* Supported (Hq, D): (8, 64), (64, 128); K <= 4096; window <= 4096.         */
/* gate_stride_d other than 0 or 1 is DSA_ERR_INVALID_ARG.                   */
/* ------------------------------------------------------------------------ */
size_t dsa_sparse_attn_workspace_size(int B, int T, int K, int window, int Hq, int D);
dsa_status_t dsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* idx, int K, int window, const void* gate,
                             int64_t gate_stride_d, float sm_scale, int Hq, int D,
                             const int32_t* cu_q,
                             const int32_t* ctx_len, const int64_t* cu_ctx, int B, int T,
                             int max_q, int max_ctx, void* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The sliding-window layers of a hybrid decode step, in one launch: the     */
/* naive-n0-5-flash page (Key Capabilities) interleaves five sliding-window  */
/* attention layers (128-token window) with each DSA layer.  For each of the */
/* n_layers layers L (1 <= n_layers <= 8), each with its own tensors, and   */
/* each sequence b of the shared descriptor (one new query at p = ctx_len[b] */
/* - 1; every layer's caches packed the same way by cu_ctx):                */
/*   out[L][b] = dsa_sparse_attn over S = {max(0, p - window + 1) .. p}      */
/*               of q[L][b] against k_cache[L], v_cache[L],                  */
/*               gated by gate[L] when gate != NULL and gate[L] != NULL.     */
/* q, k_cache, v_cache, out (and gate, if not NULL) are host arrays of       */
/* n_layers device pointers.  One workgroup per (layer, sequence) takes the  */
/* whole window; no workspace.  Results equal n_layers dsa_sparse_attn       */
/* calls in window mode up to the order of the softmax sums.                 */
/* Supported: (Hq, D) as dsa_sparse_attn; 1 <= window <= 4096.               */
/* ------------------------------------------------------------------------ */
dsa_status_t dsa_swa_decode_layers(int n_layers, const void* const* q, const void* const* k_cache,
                                   const void* const* v_cache, const void* const* gate,
                                   int64_t gate_stride_d, int window, float sm_scale, int Hq,
                                   int D, const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                   int max_ctx, void* const* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Whole layer, decode: one new query per sequence (T == B).                 */
/* Steps 1 -> 2 -> 3 above on the caller's stream, with the step-1 kernel   */
/* also emitting the per-tile candidate lists that step 2 certifies (the     */
/* selection is still exact).  Arguments are those of the three steps;       */
/* idx_out (int32 [B, K], or NULL) receives the selected positions, which   */
/* otherwise stay in the workspace.                                          */
/* Workspace contents after the call (a diagnostic contract): its first      */
/* B * ld fp32 values, ld = max_ctx rounded up to a multiple of 64, are the  */
/* step-1 scores the selection was made from (row b at offset b * ld,       */
/* positions 0 .. ctx_len[b]-1 written).                                     */
/* ------------------------------------------------------------------------ */
size_t dsa_layer_decode_workspace_size(int B, int max_ctx, int K, int Hq, int D);
dsa_status_t dsa_layer_decode(const void* q_idx, const void* w, int64_t w_ld, const void* k_idx,
                              int k_dtype, const float* k_scale, int H_I, int d_I, const void* q,
                              const void* k_cache, const void* v_cache, const void* gate,
                              int64_t gate_stride_d, float sm_scale, int Hq, int D, int K,
                              const int32_t* ctx_len,
                              const int64_t* cu_ctx, int B, int max_ctx, void* out,
                              int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* Whole layer, decode, with the new token appended first (the cache-append */
/* step of dsa_cache_append fused into the layer's first kernel): for each   */
/* sequence b, cache row cu_ctx[b] + ctx_len[b] - 1 receives k_idx_new[b]    */
/* (bf16 [B, d_I]; an fp8 key cache gets its E4M3FN codes and k_scale its    */
/* scale, exactly as dsa_cache_append computes them), k_new[b] and v_new[b] */
/* (bf16 [B, D], either may be NULL), and the layer then runs on the updated */
/* caches, the new position included.  Results and cache contents are       */
/* bit-identical to dsa_cache_append followed by dsa_layer_decode.  The      */
/* caches are therefore writable here.                                      */
dsa_status_t dsa_layer_decode_append(const void* q_idx, const void* w, int64_t w_ld, void* k_idx,
                                     int k_dtype, float* k_scale, int H_I, int d_I, const void* q,
                                     void* k_cache, void* v_cache, const void* gate,
                                     int64_t gate_stride_d, float sm_scale, int Hq, int D, int K,
                                     const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                     int max_ctx, const void* k_idx_new, const void* k_new,
                                     const void* v_new, void* out, int32_t* idx_out, void* ws,
                                     size_t ws_bytes, void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory   */
/* (code under HIP graph capture, tight serving loops, harnesses that forbid */
/* allocation): dsa_layer_decode with its workspace in a fixed scratch array */
/* the library keeps in each GPU's memory until the process ends            */
/* (dsa_layer_decode_noalloc_max_bytes() bytes, 64 MiB).  It never calls    */
/* hipMalloc or hipFree.  A call whose workspace                            */
/* (dsa_layer_decode_workspace_size) exceeds that size returns              */
/* DSA_ERR_WORKSPACE without touching the GPU.  Every call on one GPU uses  */
/* the same array: calls that overlap on one GPU (other streams, other host */
/* threads) race and must be ordered by the caller.  No step needs the      */
/* array cleared, so the previous call's contents are harmless.  Results    */
/* are bit-identical to dsa_layer_decode's.                                 */
size_t dsa_layer_decode_noalloc_max_bytes(void);
dsa_status_t dsa_layer_decode_noalloc(const void* q_idx, const void* w, int64_t w_ld,
                                      const void* k_idx, int k_dtype, const float* k_scale,
                                      int H_I, int d_I, const void* q, const void* k_cache,
                                      const void* v_cache, const void* gate,
                                      int64_t gate_stride_d, float sm_scale, int Hq, int D, int K,
                                      const int32_t* ctx_len, const int64_t* cu_ctx, int B,
                                      int max_ctx, void* out, int32_t* idx_out, void* stream);

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
/* of six caller-owned device counters (uint32 [6], zeroed by the caller)   */
/* naming the path that produced the row: [0] the union of the row's        */
/* sub-tile candidate reports, certified exact; [1] the exact radix select  */
/* over the whole score row (a key shared by too many positions, or keys    */
/* too many for [5]); [2] the direct select of a row of at most 16384       */
/* positions; [3] the collection sweep over the row's scores used when a    */
/* call has 1024 rows or more; [5] a report union whose certification       */
/* failed, resolved by one collection sweep of the row's keys at or above   */
/* the union's K-th best key.  [4] counts the rows of [3] whose collection  */
/* threshold came from a sample of the row (one sweep instead of histogram  */
/* sweeps first).  Rows with at most K positions take none of them.  Pass   */
/* NULL to stop.  Always DSA_OK.                                            */
dsa_status_t dsa_set_topk_counters(uint32_t* counters);

/* Debug check of index rows (the Top-K output rows of the Architecture     */
/* Breakdown's selection step, and the index rows the sparse attention     */
/* gathers with).  For T rows of K int32 entries `idx` [T, K] on the        */
/* device, with the batch descriptor giving each row's query position p,   */
/* adds to four caller-owned device counters (uint32 [4], zeroed by the    */
/* caller): [0] the entries outside [0, p] other than -1; with full != 0   */
/* (rows that are Top-K outputs: K_eff = min(K, p + 1) positions ascending, */
/* then -1 padding) [1] the neighbouring pairs that break that order and  */
/* [2] the rows whose count of positions is not K_eff; [3] the rows        */
/* checked.  Reads only idx and the descriptor (cu_q NULL: one row per     */
/* sequence, at p = ctx_len[b] - 1).  Asynchronous on `stream`.             */
/* Returns DSA_ERR_INVALID_ARG for a NULL or misaligned pointer, T or B    */
/* out of range, or K < 1.                                                  */
dsa_status_t dsa_check_index_rows(const int32_t* idx, int K, const int32_t* cu_q,
                                  const int32_t* ctx_len, int B, int T, int full,
                                  uint32_t* counters, void* stream);

/* Debug hook: on the calling thread, every later selection (dsa_topk,      */
/* dsa_layer_decode and its variants, dsa_layer_prefill) runs              */
/* dsa_check_index_rows(full = 1) on the rows it selected, and every later  */
/* dsa_sparse_attn call with index rows runs it (full = 0) on the caller's */
/* rows before the attention, adding into `counters` (device uint32 [4],   */
/* as above).  One extra small kernel per call while set.  Pass NULL to    */
/* stop.  Always DSA_OK.                                                   */
dsa_status_t dsa_set_index_checks(uint32_t* counters);

/* ------------------------------------------------------------------------ */
/* Whole layer, prefill: a chunk of new queries per sequence (cu_q given).   */
/* Same steps; the indexer runs as a dense MFMA contraction of the chunk's   */
/* query heads against the key cache with causal tile skipping (bf16, or fp8 */
/* with fp8 query heads and keys).                                           */
/*                                                                           */
/* Workspace: dsa_layer_prefill_workspace_size() bytes run the T query rows */
/* in one pass (the fp32 score array alone is T x max_ctx).  Any smaller     */
/* workspace of at least dsa_layer_prefill_min_workspace_size() bytes is     */
/* used by running the rows in consecutive sub-chunks of as many rows as    */
/* fit (same results: every step is row-wise); below that the call returns   */
/* DSA_ERR_WORKSPACE.  After a one-pass call the first T * ld fp32 values of */
/* the workspace (ld = max_ctx rounded up to a multiple of 64) are the       */
/* step-1 scores the selection was made from; after a sub-chunked call they */
/* hold the last sub-chunk's rows.                                           */
/* ------------------------------------------------------------------------ */
size_t dsa_layer_prefill_workspace_size(int B, int T, int max_ctx, int K, int Hq, int D);
size_t dsa_layer_prefill_min_workspace_size(int B, int max_ctx, int K, int Hq, int D);
dsa_status_t dsa_layer_prefill(const void* q_idx, int q_dtype, const float* q_scale,
                               const void* w, int64_t w_ld, const void* k_idx,
                               int k_dtype, const float* k_scale, int H_I, int d_I,
                               const void* q, const void* k_cache, const void* v_cache,
                               const void* gate, int64_t gate_stride_d, float sm_scale, int Hq,
                               int D, int K,
                               const int32_t* cu_q, const int32_t* ctx_len,
                               const int64_t* cu_ctx, int B, int T, int max_q, int max_ctx,
                               void* out, int32_t* idx_out, void* ws, size_t ws_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
