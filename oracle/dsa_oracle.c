/*
 * dsa_oracle.c -- plain fp64 CPU oracle for the Gated DSA layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The product path (the HIP library
 * and its Python binding) never links, loads or calls it, and it shares no
 * source, header, table or helper with that path.
 *
 * What it computes (sources are the five web pages on the subject; the page
 * titles are abbreviated as below):
 *   [OSLLM]  "Open-Source LLM Architecture Evolution: How Lightweight Sparse
 *            Attention Reshapes Long-Context Modeling Efficiency",
 *            section "Architecture Breakdown", item 2 (Indexer, Top-K, gate);
 *            section "Technical Deep Dive", item 2 (attention over the 2048).
 *   [FGSA]   "Fine-Grained Sparse Attention in Ultra-Large Parameter Models",
 *            section 2.1 (Indexer + Top-K, K = 2048), 2.2 (no RoPE in the
 *            indexer), 2.3 (32 heads x 128 dim).
 *   [N05]    the naive-n0-5-flash item page, "Key Capabilities" (16-head
 *            indexer, top-2048, 5:1 SWA with a 128-token window).
 * The pages give no formula; the readings taken where they are silent are
 * listed next to each function and in the design notes of the repository.
 *
 * Arithmetic: every input is widened exactly to double; every sum runs in
 * index order in double; nothing is blocked, fused or reordered.
 *
 * Parity pins: every exported function is pinned by CPU tests against
 * closed forms, library routines and brute force (see tests/test_oracle_*).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_KEY_BF16 0
#define ORC_KEY_FP8_E4M3 1

/* ---------------------------------------------------------------------- */
/* Input decoding (exact).                                                 */
/* ---------------------------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32: widening is exact. */
double orc_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits, no infinities, S.1111.111 is NaN, max 448. */
double orc_e4m3_to_f64(uint8_t code) {
  int s = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Position of query i of sequence b: the cache already holds the new
 * queries' own rows, so p = ctx_len - n_q + i (the query sees itself). */
static int64_t query_pos(const int32_t* cu_q, const int32_t* ctx_len, int b, int64_t t) {
  int64_t nq = (int64_t)cu_q[b + 1] - cu_q[b];
  return (int64_t)ctx_len[b] - nq + (t - cu_q[b]);
}

static int seq_of_row(const int32_t* cu_q, int B, int64_t t) {
  for (int b = 0; b < B; ++b)
    if (t >= cu_q[b] && t < cu_q[b + 1]) return b;
  return -1;
}

/* ---------------------------------------------------------------------- */
/* Thread pool helper: split [0, n) into contiguous ranges.               */
/* ---------------------------------------------------------------------- */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_tramp(void* a) {
  range_job* j = (range_job*)a;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < nthreads) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  range_job jobs[256];
  int started[256];
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].lo = n * i / nthreads;
    jobs[i].hi = n * (i + 1) / nthreads;
    started[i] = pthread_create(&th[i], NULL, range_tramp, &jobs[i]) == 0;
    if (!started[i]) fn(ctx, jobs[i].lo, jobs[i].hi);
  }
  for (int i = 0; i < nthreads; ++i)
    if (started[i]) pthread_join(th[i], NULL);
}

/* ---------------------------------------------------------------------- */
/* Indexer score ([OSLLM] Architecture Breakdown item 2; [FGSA] 2.1-2.3).  */
/*                                                                         */
/*   s[t, j] = sum_h w[t,h] * max(0, rho_th * sigma_j *                    */
/*                                   sum_d qI[t,h,d] * kI[j,d])            */
/*                                                                         */
/* for j = 0..p_t.  One indexer key row per position is shared by all      */
/* heads; positions are not rotated (no RoPE, [FGSA] 2.2); the per-head    */
/* dot products are combined by a ReLU and a per-query head weight; sigma  */
/* is the per-token fp32 scale of an fp8 key cache, 1 for bf16 keys.  The  */
/* query heads are bf16 (rho = 1) or, for the fp8 prefill contraction      */
/* ([N05] Key Capabilities: FP8; [OWD] sections 1 and 3: FP8 activations), */
/* E4M3FN codes with one fp32 scale rho_th per query and head: like the    */
/* key scale, it multiplies the dot product of the decoded codes.          */
/* ---------------------------------------------------------------------- */

typedef struct {
  const void* q;       /* [T, H, d] bf16 bits or E4M3FN codes */
  int q_dtype;
  const float* q_scale; /* [T, H] for E4M3FN queries */
  const uint16_t* w;   /* [T, w_ld] bf16 bits */
  int64_t w_ld;
  const void* k;       /* [sum L, d] bf16 bits or e4m3 codes */
  int k_dtype;
  const float* k_scale;
  int H, d;
  const int32_t* cu_q;
  const int32_t* ctx_len;
  const int64_t* cu_ctx;
  int B;
  double* scores;      /* [T, ld] */
  int64_t ld;
} score_ctx;

static double key_elem(const score_ctx* c, int64_t row, int dd) {
  if (c->k_dtype == ORC_KEY_BF16)
    return orc_bf16_to_f64(((const uint16_t*)c->k)[row * c->d + dd]);
  return orc_e4m3_to_f64(((const uint8_t*)c->k)[row * c->d + dd]);
}

/* Work unit u covers row t = u / SCORE_CHUNKS and one contiguous chunk of
 * its visible positions, so a single decode query still uses every thread.
 * Every s[t, j] is computed on its own; the split changes no arithmetic. */
#define SCORE_CHUNKS 64

static void score_units(void* vctx, int64_t lo, int64_t hi) {
  const score_ctx* c = (const score_ctx*)vctx;
  double* qd = (double*)malloc(sizeof(double) * (size_t)c->H * c->d);
  double* wd = (double*)malloc(sizeof(double) * (size_t)c->H);
  double* kd = (double*)malloc(sizeof(double) * (size_t)c->d);
  double* rho = (double*)malloc(sizeof(double) * (size_t)c->H);
  for (int64_t u = lo; u < hi; ++u) {
    int64_t t = u / SCORE_CHUNKS, part = u % SCORE_CHUNKS;
    int b = seq_of_row(c->cu_q, c->B, t);
    int64_t p = query_pos(c->cu_q, c->ctx_len, b, t);
    int64_t j0 = (p + 1) * part / SCORE_CHUNKS, j1 = (p + 1) * (part + 1) / SCORE_CHUNKS;
    for (int h = 0; h < c->H; ++h) {
      wd[h] = orc_bf16_to_f64(c->w[t * c->w_ld + h]);
      rho[h] = c->q_scale ? (double)c->q_scale[t * c->H + h] : 1.0;
      for (int dd = 0; dd < c->d; ++dd) {
        const int64_t qi = (t * c->H + h) * c->d + dd;
        qd[h * c->d + dd] = c->q_dtype == ORC_KEY_BF16
                                ? orc_bf16_to_f64(((const uint16_t*)c->q)[qi])
                                : orc_e4m3_to_f64(((const uint8_t*)c->q)[qi]);
      }
    }
    for (int64_t j = j0; j < j1; ++j) {
      int64_t row = c->cu_ctx[b] + j;
      double sigma = c->k_scale ? (double)c->k_scale[row] : 1.0;
      for (int dd = 0; dd < c->d; ++dd) kd[dd] = key_elem(c, row, dd);
      double s = 0.0;
      for (int h = 0; h < c->H; ++h) {
        double dot = 0.0;
        for (int dd = 0; dd < c->d; ++dd) dot += qd[h * c->d + dd] * kd[dd];
        double x = rho[h] * sigma * dot;
        s += wd[h] * (x > 0.0 ? x : 0.0);
      }
      c->scores[t * c->ld + j] = s;
    }
  }
  free(qd);
  free(wd);
  free(kd);
  free(rho);
}

int orc_index_scores(const void* q_idx, int q_dtype, const float* q_scale, const uint16_t* w,
                     int64_t w_ld, const void* k_idx, int k_dtype, const float* k_scale, int H_I,
                     int d_I, const int32_t* cu_q, const int32_t* ctx_len, const int64_t* cu_ctx,
                     int B, double* scores, int64_t ld, int nthreads) {
  score_ctx c = {q_idx, q_dtype, q_scale, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, cu_q,
                 ctx_len, cu_ctx, B, scores, ld};
  parallel_for((int64_t)cu_q[B] * SCORE_CHUNKS, nthreads, score_units, &c);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Cache append: quantisation of a new token's indexer key row to the fp8  */
/* key cache ([N05] Key Capabilities: FP8 mixed precision; the cache holds */
/* OCP E4M3FN codes plus one fp32 scale per token).  The pages give no     */
/* recipe; the reading taken is per-token absolute-maximum scaling:        */
/*   amax  = max_d |x_d|                     (x: the bf16 row, exact)      */
/*   sigma = amax / 448 in fp32 (1 for an all-zero row)                    */
/*   y_d   = x_d / sigma in fp32, clamped to [-448, 448]                   */
/*   code  = y_d rounded to the nearest E4M3FN value, ties to even         */
/* so that sigma * decode(code) approximates x_d.  The rounding decision   */
/* is taken on the fp32 value y_d (the precision the device computes in).  */
/* ---------------------------------------------------------------------- */

/* Nearest E4M3FN code of a finite fp32 value with |y| <= 448, ties to even.
 * Worked in double, where every step below is exact: subnormal codes are
 * multiples of 2^-9 below 2^-6; a normal code 1.mmm x 2^e has spacing
 * 2^(e-3). */
static uint8_t e4m3_nearest(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (a < ldexp(1.0, -6)) {
    double m = nearbyint(a * 512.0); /* 0..8; 8 is the smallest normal, code 0x08 */
    return (uint8_t)(sign | (uint8_t)m);
  }
  int ex;
  frexp(a, &ex);          /* a = f * 2^ex, f in [0.5, 1): a in [2^(ex-1), 2^ex) */
  int e = ex - 1;         /* a = 1.xxx * 2^e, e in [-6, 8] */
  double r = nearbyint(a / ldexp(1.0, e - 3));  /* 8..16 */
  if (r == 16.0) {
    e += 1;
    r = 8.0;
  }
  return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)(r - 8.0));
}

int orc_quantize_e4m3_rows(const uint16_t* k, int64_t rows, int d, uint8_t* codes,
                           float* scales) {
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.f;
    for (int i = 0; i < d; ++i) {
      float x = (float)orc_bf16_to_f64(k[r * d + i]);
      if (fabsf(x) > amax) amax = fabsf(x);
    }
    float sigma = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[r] = sigma;
    for (int i = 0; i < d; ++i) {
      float y = (float)orc_bf16_to_f64(k[r * d + i]) / sigma;
      if (y > 448.0f) y = 448.0f;
      if (y < -448.0f) y = -448.0f;
      codes[r * d + i] = e4m3_nearest(y);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Top-K select ([OSLLM] Architecture Breakdown item 2: keep the K best;   */
/* [FGSA] 2.1: K = 2048 historical positions).                             */
/*                                                                         */
/* Readings where the pages are silent: a query at p sees 0..p; when fewer */
/* than K positions are visible it keeps all of them and pads with -1;     */
/* equal scores go to the lower position; -0.0 equals +0.0; the kept       */
/* positions are emitted in ascending order.                               */
/* ---------------------------------------------------------------------- */

typedef struct {
  double s;
  int64_t j;
} sj_pair;

static int cmp_desc_score_asc_pos(const void* a, const void* b) {
  const sj_pair* x = (const sj_pair*)a;
  const sj_pair* y = (const sj_pair*)b;
  /* -0.0 == +0.0 under IEEE comparison, so they tie and fall to position. */
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

typedef struct {
  const double* s64;
  const float* s32;
  int64_t ld;
  const int32_t* cu_q;
  const int32_t* ctx_len;
  int B;
  int K;
  int32_t* idx;
} topk_ctx;

static void topk_rows(void* vctx, int64_t lo, int64_t hi) {
  const topk_ctx* c = (const topk_ctx*)vctx;
  for (int64_t t = lo; t < hi; ++t) {
    int b = seq_of_row(c->cu_q, c->B, t);
    int64_t p = query_pos(c->cu_q, c->ctx_len, b, t);
    int64_t n = p + 1;
    sj_pair* v = (sj_pair*)malloc(sizeof(sj_pair) * (size_t)n);
    for (int64_t j = 0; j < n; ++j) {
      v[j].s = c->s64 ? c->s64[t * c->ld + j] : (double)c->s32[t * c->ld + j];
      v[j].j = j;
    }
    qsort(v, (size_t)n, sizeof(sj_pair), cmp_desc_score_asc_pos);
    int64_t keff = n < c->K ? n : c->K;
    int32_t* out = c->idx + t * c->K;
    for (int64_t i = 0; i < keff; ++i) out[i] = (int32_t)v[i].j;
    qsort(out, (size_t)keff, sizeof(int32_t), cmp_i32);
    for (int64_t i = keff; i < c->K; ++i) out[i] = -1;
    free(v);
  }
}

/* Mode E: select on fp64 scores produced by orc_index_scores. */
int orc_topk_f64(const double* scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
                 int B, int K, int32_t* idx, int nthreads) {
  topk_ctx c = {scores, NULL, ld, cu_q, ctx_len, B, K, idx};
  parallel_for(cu_q[B], nthreads, topk_rows, &c);
  return 0;
}

/* Mode T: select on an fp32 score array, widened exactly. */
int orc_topk_f32(const float* scores, int64_t ld, const int32_t* cu_q, const int32_t* ctx_len,
                 int B, int K, int32_t* idx, int nthreads) {
  topk_ctx c = {NULL, scores, ld, cu_q, ctx_len, B, K, idx};
  parallel_for(cu_q[B], nthreads, topk_rows, &c);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Gated sparse attention ([OSLLM] Technical Deep Dive item 2: scores and  */
/* softmax over only the selected 2048; Architecture Breakdown item 2 and  */
/* the layer list of the deployment page: a gated layer).                  */
/*                                                                         */
/* For query t and head h, over the selected set S (one set per query,     */
/* shared by all heads; one shared K/V head):                              */
/*   z_j = c * sum_d q[t,h,d] K[j,d],  a = softmax(z),  o = sum_j a_j V[j] */
/*   out[t,h,d] = o[d] * sigmoid(g[t,h,d])   (no gate when g is absent)    */
/* with c = sm_scale, or 1/sqrt(D) when sm_scale is 0.  Window mode (the   */
/* sliding-window layers of the 5:1 hybrid, [N05]): S = {max(0,p-W+1)..p}. */
/* ---------------------------------------------------------------------- */

typedef struct {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* idx;
  int K;
  int window;
  const uint16_t* g;
  double scale;
  int Hq, D;
  const int32_t* cu_q;
  const int32_t* ctx_len;
  const int64_t* cu_ctx;
  int B;
  double* out;
  double* lse;
} attn_ctx;

/* Work unit u is the pair (t = u / Hq, h = u % Hq); each is independent. */
static void attn_units(void* vctx, int64_t lo, int64_t hi) {
  const attn_ctx* c = (const attn_ctx*)vctx;
  int nmax = c->idx ? c->K : c->window;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nmax > 0 ? nmax : 1));
  double* z = (double*)malloc(sizeof(double) * (size_t)(nmax > 0 ? nmax : 1));
  for (int64_t u = lo; u < hi; ++u) {
    int64_t t = u / c->Hq;
    int h = (int)(u % c->Hq);
    int b = seq_of_row(c->cu_q, c->B, t);
    int64_t p = query_pos(c->cu_q, c->ctx_len, b, t);
    int n = 0;
    if (c->idx) {
      for (int i = 0; i < c->K; ++i) {
        int32_t j = c->idx[t * c->K + i];
        if (j >= 0) rows[n++] = c->cu_ctx[b] + j;
      }
    } else {
      int64_t j0 = p - c->window + 1;
      if (j0 < 0) j0 = 0;
      for (int64_t j = j0; j <= p; ++j) rows[n++] = c->cu_ctx[b] + j;
    }
    const uint16_t* qh = c->q + (t * c->Hq + h) * c->D;
    double m = -INFINITY;
    for (int i = 0; i < n; ++i) {
      double dot = 0.0;
      for (int d = 0; d < c->D; ++d)
        dot += orc_bf16_to_f64(qh[d]) * orc_bf16_to_f64(c->kc[rows[i] * c->D + d]);
      z[i] = c->scale * dot;
      if (z[i] > m) m = z[i];
    }
    double l = 0.0;
    for (int i = 0; i < n; ++i) {
      z[i] = exp(z[i] - m);
      l += z[i];
    }
    double* o = c->out + (t * c->Hq + h) * c->D;
    for (int d = 0; d < c->D; ++d) {
      double acc = 0.0;
      for (int i = 0; i < n; ++i) acc += z[i] * orc_bf16_to_f64(c->vc[rows[i] * c->D + d]);
      double od = n > 0 ? acc / l : 0.0;
      if (c->g) {
        double gv = orc_bf16_to_f64(c->g[(t * c->Hq + h) * c->D + d]);
        od = od / (1.0 + exp(-gv));
      }
      o[d] = od;
    }
    if (c->lse) c->lse[t * c->Hq + h] = n > 0 ? m + log(l) : -INFINITY;
  }
  free(rows);
  free(z);
}

int orc_sparse_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                    const int32_t* idx, int K, int window, const uint16_t* gate,
                    double sm_scale, int Hq, int D, const int32_t* cu_q,
                    const int32_t* ctx_len, const int64_t* cu_ctx, int B, double* out,
                    double* lse, int nthreads) {
  attn_ctx c = {q, k_cache, v_cache, idx, K, window, gate,
                sm_scale != 0.0 ? sm_scale : 1.0 / sqrt((double)D), Hq, D, cu_q, ctx_len,
                cu_ctx, B, out, lse};
  parallel_for((int64_t)cu_q[B] * Hq, nthreads, attn_units, &c);
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Whole layer: indexer scores -> top-K -> gated sparse attention, for the */
/* queries of the batch descriptor (decode: one query per sequence).       */
/* scores_out / idx_out may be NULL; when given, they receive the fp64     */
/* scores [T, ld] and the selected positions [T, K].                       */
/* ---------------------------------------------------------------------- */

int orc_layer(const uint16_t* q_idx, const uint16_t* w, int64_t w_ld, const void* k_idx,
              int k_dtype, const float* k_scale, int H_I, int d_I, const uint16_t* q,
              const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* gate,
              double sm_scale, int Hq, int D, int K, const int32_t* cu_q,
              const int32_t* ctx_len, const int64_t* cu_ctx, int B, double* out, double* lse,
              double* scores_out, int32_t* idx_out, int64_t ld, int nthreads) {
  int64_t T = cu_q[B];
  double* s = scores_out;
  int32_t* id = idx_out;
  if (!s) s = (double*)malloc(sizeof(double) * (size_t)(T * ld));
  if (!id) id = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * K));
  if (!s || !id) return 1;
  orc_index_scores(q_idx, ORC_KEY_BF16, NULL, w, w_ld, k_idx, k_dtype, k_scale, H_I, d_I, cu_q,
                   ctx_len, cu_ctx, B, s, ld, nthreads);
  orc_topk_f64(s, ld, cu_q, ctx_len, B, K, id, nthreads);
  orc_sparse_attn(q, k_cache, v_cache, id, K, 0, gate, sm_scale, Hq, D, cu_q,
                  ctx_len, cu_ctx, B, out, lse, nthreads);
  if (!scores_out) free(s);
  if (!idx_out) free(id);
  return 0;
}
