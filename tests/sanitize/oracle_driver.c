/* Drives every entry point of oracle/dsa_oracle.c on small ragged inputs,
 * several threads each, for a build with -fsanitize=address,undefined: any
 * out-of-bounds access, leak, misaligned or overflowing operation in the
 * oracle aborts the run.  The values are not checked here (the oracle's
 * pins do that); the driver only exercises every code path: bf16 and fp8
 * keys, bf16 and fp8 query heads, Top-K on fp64 and fp32 rows (rows longer
 * and shorter than K), attention in index and window modes, gated and
 * ungated, the whole layer, and the cache-append quantiser. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_index_scores(const void* q_idx, int q_dtype, const float* q_scale, const uint16_t* w,
                     int64_t w_ld, const void* k_idx, int k_dtype, const float* k_scale, int H_I,
                     int d_I, const int32_t* cu_q, const int32_t* ctx_len, const int64_t* cu_ctx,
                     int B, double* scores, int64_t ld, int nthreads);
int orc_quantize_e4m3_rows(const uint16_t* k, int64_t rows, int d, uint8_t* codes, float* scale);
int orc_topk_f64(const double* scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
                 int B, int K, int32_t* idx, int nthreads);
int orc_topk_f32(const float* scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
                 int B, int K, int32_t* idx, int nthreads);
int orc_sparse_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* idx, int K, int window, const uint16_t* gate, double sm_scale,
                    int Hq, int D, const int32_t* cu_q, const int32_t* ctx_len,
                    const int64_t* cu_ctx, int B, double* out, double* lse, int nthreads);
int orc_layer(const uint16_t* q_idx, const uint16_t* w, int64_t w_ld, const void* k_idx,
              int k_dtype, const float* k_scale, int H_I, int d_I, const uint16_t* q,
              const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* gate,
              double sm_scale, int Hq, int D, int K, const int32_t* cu_q, const int32_t* ctx_len,
              const int64_t* cu_ctx, int B, double* out, double* lse, double* scores_out,
              int32_t* idx_out, int64_t ld, int nthreads);

static uint64_t state = 0x243f6a8885a308d3ull;
static uint32_t next_u32(void) { /* xorshift64*, test data only */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}
/* a finite bf16 pattern of magnitude below 4 */
static uint16_t rand_bf16(void) {
  const uint32_t r = next_u32();
  const uint16_t exp = (uint16_t)(120 + r % 9);  /* 2^-7 .. 2^1 */
  return (uint16_t)(((r >> 8) & 1u) << 15 | exp << 7 | ((r >> 9) & 0x7fu));
}
static uint8_t rand_e4m3(void) { /* any finite code (0x7f / 0xff are NaN) */
  uint8_t c;
  do c = (uint8_t)next_u32(); while ((c & 0x7f) == 0x7f);
  return c;
}
static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

int main(void) {
  enum { B = 3, HI = 4, DI = 64, HQ = 8, D = 64, K = 48, NT = 3 };
  const int32_t lens[B] = {40, 130, 7}; /* longer and shorter than K */
  const int32_t nq[B] = {1, 3, 2};      /* a prefill-like ragged chunk */
  int32_t cu_q[B + 1], ctx_len[B];
  int64_t cu_ctx[B + 1];
  cu_q[0] = 0;
  cu_ctx[0] = 0;
  for (int b = 0; b < B; ++b) {
    ctx_len[b] = lens[b];
    cu_q[b + 1] = cu_q[b] + nq[b];
    cu_ctx[b + 1] = cu_ctx[b] + lens[b];
  }
  const int T = cu_q[B];
  const int64_t L = cu_ctx[B], ld = 136;

  uint16_t* q_idx = xmalloc(sizeof(uint16_t) * T * HI * DI);
  uint8_t* q8 = xmalloc((size_t)T * HI * DI);
  float* q_scale = xmalloc(sizeof(float) * T * HI);
  uint16_t* w = xmalloc(sizeof(uint16_t) * T * HI);
  uint16_t* k_idx = xmalloc(sizeof(uint16_t) * L * DI);
  uint8_t* k8 = xmalloc((size_t)L * DI);
  float* k_scale = xmalloc(sizeof(float) * L);
  uint16_t* q = xmalloc(sizeof(uint16_t) * T * HQ * D);
  uint16_t* kc = xmalloc(sizeof(uint16_t) * L * D);
  uint16_t* vc = xmalloc(sizeof(uint16_t) * L * D);
  uint16_t* gate = xmalloc(sizeof(uint16_t) * T * HQ * D);
  for (int i = 0; i < T * HI * DI; ++i) q_idx[i] = rand_bf16();
  for (int i = 0; i < T * HI * DI; ++i) q8[i] = rand_e4m3();
  for (int i = 0; i < T * HI; ++i) q_scale[i] = 0.5f + (float)(next_u32() % 100) / 64.f;
  for (int i = 0; i < T * HI; ++i) w[i] = (uint16_t)(rand_bf16() & 0x7fffu);
  for (int64_t i = 0; i < L * DI; ++i) k_idx[i] = rand_bf16();
  for (int i = 0; i < T * HQ * D; ++i) q[i] = rand_bf16();
  for (int i = 0; i < T * HQ * D; ++i) gate[i] = rand_bf16();
  for (int64_t i = 0; i < L * D; ++i) kc[i] = rand_bf16();
  for (int64_t i = 0; i < L * D; ++i) vc[i] = rand_bf16();
  /* a zero row and a saturating row for the quantiser */
  memset(k_idx, 0, sizeof(uint16_t) * DI);
  for (int d = 0; d < DI; ++d) k_idx[DI + d] = (uint16_t)(0x4380u | (d & 1u) << 15);
  if (orc_quantize_e4m3_rows(k_idx, L, DI, k8, k_scale)) return 1;

  double* s = xmalloc(sizeof(double) * T * ld);
  float* s32 = xmalloc(sizeof(float) * T * ld);
  int32_t* idx = xmalloc(sizeof(int32_t) * T * K);
  double* out = xmalloc(sizeof(double) * T * HQ * D);
  double* lse = xmalloc(sizeof(double) * T * HQ);
  const int kd[2] = {0, 1};
  for (int a = 0; a < 2; ++a) {
    const void* keys = kd[a] ? (const void*)k8 : (const void*)k_idx;
    const float* ks = kd[a] ? k_scale : NULL;
    if (orc_index_scores(q_idx, 0, NULL, w, HI, keys, kd[a], ks, HI, DI, cu_q, ctx_len, cu_ctx,
                         B, s, ld, NT))
      return 1;
    if (orc_index_scores(q_idx, 0, NULL, w, 0, keys, kd[a], ks, HI, DI, cu_q, ctx_len, cu_ctx, B,
                         s, ld, NT))
      return 1;
  }
  if (orc_index_scores(q8, 1, q_scale, w, HI, k8, 1, k_scale, HI, DI, cu_q, ctx_len, cu_ctx, B, s,
                       ld, NT))
    return 1;
  if (orc_topk_f64(s, ld, cu_q, ctx_len, B, K, idx, NT)) return 1;
  for (int64_t i = 0; i < (int64_t)T * ld; ++i) s32[i] = (float)(s[i] == s[i] ? s[i] : 0.0);
  if (orc_topk_f32(s32, ld, cu_q, ctx_len, B, K, idx, NT)) return 1;
  if (orc_sparse_attn(q, kc, vc, idx, K, 0, gate, 0.0, HQ, D, cu_q, ctx_len, cu_ctx, B, out, lse,
                      NT))
    return 1;
  if (orc_sparse_attn(q, kc, vc, NULL, 0, 16, NULL, 0.0, HQ, D, cu_q, ctx_len, cu_ctx, B, out,
                      NULL, NT))
    return 1;
  if (orc_layer(q_idx, w, HI, k_idx, 0, NULL, HI, DI, q, kc, vc, gate, 0.0, HQ, D, K, cu_q,
                ctx_len, cu_ctx, B, out, lse, NULL, NULL, ld, NT))
    return 1;
  if (orc_layer(q_idx, w, HI, k8, 1, k_scale, HI, DI, q, kc, vc, NULL, 0.0, HQ, D, K, cu_q,
                ctx_len, cu_ctx, B, out, NULL, s, idx, ld, NT))
    return 1;

  free(q_idx); free(q8); free(q_scale); free(w); free(k_idx); free(k8); free(k_scale);
  free(q); free(kc); free(vc); free(gate); free(s); free(s32); free(idx); free(out); free(lse);
  printf("oracle driver ok\n");
  return 0;
}
