/*
 * Plain CPU oracle of the DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may call, link or
 * load this file; only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code, header or table with the GPU library.
 *
 * Every quantity is computed by the definition, in double precision, with plain loops.
 * Threads only split independent query rows; each row is computed by the same loops a
 * single thread would run, so the thread count never changes a result.
 *
 * What it follows (page titles as given in the source pages):
 *   - "DSA ablation model card" (BananaMind/dsa-model-ablation), model list: a lightning
 *     indexer with ReLU and per-query heads scores keys and each query keeps its top-k
 *     keys; parameter count (1,530,496 vs 1,498,496) fixes one indexer key per token
 *     shared by the heads, and no bias.
 *   - same card, "Benchmarks" note: a prompt shorter than k selects every token, so DSA
 *     is then identical to dense attention.
 *   - "DSV2-Lite-IndexCache-Sparse-1250" model card, intro: causal key selection with a
 *     budget of 2048 tokens; FSS layer pattern in which full layers compute the routes
 *     reused by the shared layers that follow.
 *   - "IndexCache" (vLLM feature doc), "How It Works": F layers compute and store top-k
 *     indices, S layers receive the cached indices of the previous layer.
 *   - "DeepSeek-V2-Lite-Chat SIQ K4/K3" card, "Measured": MLA latent of 576 values per
 *     token (kv_lora_rank 512 plus 64 rotary), cached as fp8; same section: an nvfp4
 *     latent-cache backend exists only for sparse MLA on sparse-indexer models, a cache
 *     this oracle reads in the OCP Microscaling FP4 format (MXFP4, oracle_mxfp4_value).
 * Readings where the pages are silent (index score formula, tie rule, output order,
 * fp8 variant and scaling, fp4 row layout, softmax scale argument) are stated at each
 * function.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "dsa_oracle.h"

/* ---------- exact decoders of the storage formats ---------- */

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
double oracle_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit float E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals at exponent field 0, no infinities, NaN only at S.1111.111.
 * Value = (-1)^S * 2^(E-7) * (1 + M/8) for E > 0, (-1)^S * 2^(-6) * (M/8) for E = 0. */
double oracle_e4m3_to_double(uint8_t b) {
  int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element (low 4 bits of `c`): 1 sign,
 * 2 exponent bits (bias 1), 1 mantissa bit, no infinities or NaN.
 * Value = (-1)^S * 2^(E-1) * (1 + M/2) for E > 0, (-1)^S * (M/2) for E = 0. */
double oracle_e2m1_to_double(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = e == 0 ? (double)m / 2.0 : ldexp(1.0 + (double)m / 2.0, e - 1);
  return s ? -v : v;
}

/* Same spec, E8M0 shared scale: 2^(E-127), and NaN for E = 255. */
double oracle_e8m0_to_double(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* MXFP4 latent row of D values (D a multiple of 32, at most 1024): D/32 blocks of 32
 * values share one E8M0 scale; value d = e2m1 element * scale of block d/32.  Layout (a
 * reading: the pages name the cache, not its bytes), D/2 + 32 bytes:
 *   bytes [16j, 16j+16): the 32 elements of block j, element 2i in the low nibble of
 *     byte 16j + i and element 2i+1 in its high nibble;
 *   bytes [D/2, D/2 + 32): the scales, block j's at byte D/2 + 4*(j mod 8) + j/8;
 *     bytes no block names are ignored. */
int64_t oracle_mxfp4_row_bytes(int D) { return (int64_t)D / 2 + 32; }

double oracle_mxfp4_value(const uint8_t* row, int D, int d) {
  int j = d / 32, i = d % 32;
  uint8_t byte = row[16 * j + i / 2];
  uint8_t code = (i % 2 == 0) ? (uint8_t)(byte & 15) : (uint8_t)(byte >> 4);
  uint8_t e = row[D / 2 + 4 * (j % 8) + j / 8];
  return oracle_e2m1_to_double(code) * oracle_e8m0_to_double(e);
}

/* ---------- row-parallel driver ---------- */

typedef void (*row_fn)(void* ctx, int64_t row);
typedef struct {
  row_fn fn;
  void* ctx;
  int64_t begin, end;
} span_t;

static void* run_span(void* p) {
  span_t* s = (span_t*)p;
  for (int64_t r = s->begin; r < s->end; ++r) s->fn(s->ctx, r);
  return NULL;
}

static void for_rows(int64_t nrows, int nthreads, row_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  pthread_t th[256];
  span_t sp[256];
  for (int i = 0; i < nthreads; ++i) {
    sp[i].fn = fn;
    sp[i].ctx = ctx;
    sp[i].begin = nrows * i / nthreads;
    sp[i].end = nrows * (i + 1) / nthreads;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, run_span, &sp[i]);
  run_span(&sp[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* Position of query i of sequence b: p = kv_len[b] - Tq + i; it may attend keys 0..p.
 * (Causal selection, IndexCache model card intro; the query's own key is included.) */
static int64_t query_pos(const int32_t* kv_len, int b, int Tq, int Tk, int i) {
  int64_t L = kv_len ? kv_len[b] : Tk;
  return L - Tq + i;
}

/* ---------- 1. lightning-indexer scores ---------- */
/* I[t,s] = sum_j w[t,j] * max(0, sum_d q[t,j,d] * k[s,d]) for s <= p; -inf for s > p.
 * Computed in double and rounded once to float (C's conversion rounds to nearest even). */

typedef struct {
  const uint16_t *q, *k, *w;
  const int32_t* kv_len;
  int B, Tq, Tk, H, D;
  float* scores;
  int64_t ld;
} idx_ctx;

static void idx_row(void* c_, int64_t row) {
  idx_ctx* c = (idx_ctx*)c_;
  int b = (int)(row / c->Tq), i = (int)(row % c->Tq);
  int64_t p = query_pos(c->kv_len, b, c->Tq, c->Tk, i);
  const uint16_t* qrow = c->q + ((int64_t)b * c->Tq + i) * c->H * c->D;
  const uint16_t* wrow = c->w + ((int64_t)b * c->Tq + i) * c->H;
  float* out = c->scores + ((int64_t)b * c->Tq + i) * c->ld;
  for (int64_t s = 0; s < c->Tk; ++s) {
    if (s > p) {
      out[s] = -INFINITY;
      continue;
    }
    const uint16_t* krow = c->k + ((int64_t)b * c->Tk + s) * c->D;
    double total = 0.0;
    for (int j = 0; j < c->H; ++j) {
      double dot = 0.0;
      for (int d = 0; d < c->D; ++d)
        dot += oracle_bf16_to_double(qrow[j * c->D + d]) * oracle_bf16_to_double(krow[d]);
      double relu = dot > 0.0 ? dot : 0.0;
      total += oracle_bf16_to_double(wrow[j]) * relu;
    }
    out[s] = (float)total;
  }
}

int oracle_index_scores(const uint16_t* q, const uint16_t* k, const uint16_t* w,
                        const int32_t* kv_len, int B, int Tq, int Tk, int H, int D,
                        float* scores, int64_t ld, int nthreads) {
  if (!q || !k || !w || !scores || B < 0 || Tq < 0 || Tk < 0 || H < 1 || D < 1 || ld < Tk) return 1;
  idx_ctx c = {q, k, w, kv_len, B, Tq, Tk, H, D, scores, ld};
  for_rows((int64_t)B * Tq, nthreads, idx_row, &c);
  return 0;
}

/* ---------- 2. causal top-k ---------- */
/* Candidates of row i are keys 0..p.  If p+1 <= k all of them are kept (a prompt shorter
 * than k selects every token, DSA ablation card "Benchmarks").  Otherwise the k keys of
 * largest score are kept; between equal scores the lower key index is preferred
 * (reading: a deterministic rule; IEEE equality, so -0 equals +0).  Output: the kept
 * indices in ascending order, then -1 up to k entries (reading). */

typedef struct {
  float score;
  int32_t index;
} cand_t;

static int by_score_then_index(const void* a_, const void* b_) {
  const cand_t *a = (const cand_t*)a_, *b = (const cand_t*)b_;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->index > b->index) - (a->index < b->index);
}

static int by_index(const void* a_, const void* b_) {
  int32_t a = *(const int32_t*)a_, b = *(const int32_t*)b_;
  return (a > b) - (a < b);
}

typedef struct {
  const float* scores;
  int64_t ld;
  const int32_t* kv_len;
  int B, Tq, Tk, k;
  int32_t* idx;
} topk_ctx;

static void topk_row(void* c_, int64_t row) {
  topk_ctx* c = (topk_ctx*)c_;
  int b = (int)(row / c->Tq), i = (int)(row % c->Tq);
  int64_t p = query_pos(c->kv_len, b, c->Tq, c->Tk, i);
  int64_t n = p + 1;
  int32_t* out = c->idx + row * c->k;
  const float* s = c->scores + row * c->ld;
  int64_t kept = 0;
  if (n <= 0) {
    kept = 0;
  } else if (n <= c->k) {
    for (int64_t j = 0; j < n; ++j) out[j] = (int32_t)j;
    kept = n;
  } else {
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)n);
    for (int64_t j = 0; j < n; ++j) {
      cand[j].score = s[j];
      cand[j].index = (int32_t)j;
    }
    qsort(cand, (size_t)n, sizeof(cand_t), by_score_then_index);
    for (int j = 0; j < c->k; ++j) out[j] = cand[j].index;
    free(cand);
    qsort(out, (size_t)c->k, sizeof(int32_t), by_index);
    kept = c->k;
  }
  for (int64_t j = kept; j < c->k; ++j) out[j] = -1;
}

int oracle_topk(const float* scores, int64_t ld, const int32_t* kv_len, int B, int Tq, int Tk,
                int k, int32_t* idx, int nthreads) {
  if (!scores || !idx || B < 0 || Tq < 0 || Tk < 0 || k < 1 || ld < Tk) return 1;
  topk_ctx c = {scores, ld, kv_len, B, Tq, Tk, k, idx};
  for_rows((int64_t)B * Tq, nthreads, topk_row, &c);
  return 0;
}

/* ---------- 3. attention restricted to the selected keys ---------- */
/* For each query row and head h (kv head g = h*Hkv/H), over the valid entries s of the
 * row's index list (entries < 0 are skipped):
 *   z_s = sm_scale * sum_d q[h,d] * K[s,g,d]
 *   out[h,:] = sum_s exp(z_s - m) V[s,g,:] / sum_s exp(z_s - m),  m = max_s z_s
 *   lse[h]   = m + log(sum_s exp(z_s - m))
 * K is the bf16 key row, the fp8 e4m3 row times its per-token scale (kv_fmt 1), or the
 * decoded MXFP4 row (kv_fmt 2: rows of oracle_mxfp4_row_bytes(Dqk) bytes).  When v is
 * NULL, V is the first Dv columns of the same row (MLA: one shared latent row per token
 * whose first 512 values are the compressed KV and last 64 the rotary part).
 * A row with no valid entry yields out = 0 and lse = -inf. */

typedef struct {
  const void *q, *kv, *v;
  const float* kv_scale;
  int kv_fmt;
  const int32_t* idx;
  int B, Tq, Tk, H, Hkv, Dqk, Dv, k;
  double sm_scale;
  double *out, *lse;
} attn_ctx;

static double kv_value(const attn_ctx* c, int b, int64_t s, int g, int d) {
  int64_t r = ((int64_t)b * c->Tk + s) * c->Hkv + g;
  if (c->kv_fmt == 2)
    return oracle_mxfp4_value((const uint8_t*)c->kv + r * oracle_mxfp4_row_bytes(c->Dqk), c->Dqk, d);
  int64_t off = r * c->Dqk + d;
  if (c->kv_fmt == 1)
    return oracle_e4m3_to_double(((const uint8_t*)c->kv)[off]) *
           (double)c->kv_scale[(int64_t)b * c->Tk + s];
  return oracle_bf16_to_double(((const uint16_t*)c->kv)[off]);
}

static double v_value(const attn_ctx* c, int b, int64_t s, int g, int d) {
  if (!c->v) return kv_value(c, b, s, g, d);
  int64_t off = (((int64_t)b * c->Tk + s) * c->Hkv + g) * c->Dv + d;
  return oracle_bf16_to_double(((const uint16_t*)c->v)[off]);
}

static void attn_row(void* c_, int64_t row) {
  attn_ctx* c = (attn_ctx*)c_;
  int b = (int)(row / c->Tq);
  const int32_t* sel = c->idx + row * c->k;
  const uint16_t* qrow = (const uint16_t*)c->q + row * c->H * c->Dqk;
  double* z = (double*)malloc(sizeof(double) * (size_t)c->k);
  for (int h = 0; h < c->H; ++h) {
    int g = h * c->Hkv / c->H;
    double m = -INFINITY;
    for (int j = 0; j < c->k; ++j) {
      if (sel[j] < 0) continue;
      double dot = 0.0;
      for (int d = 0; d < c->Dqk; ++d)
        dot += oracle_bf16_to_double(qrow[h * c->Dqk + d]) * kv_value(c, b, sel[j], g, d);
      z[j] = c->sm_scale * dot;
      if (z[j] > m) m = z[j];
    }
    double* o = c->out + (row * c->H + h) * c->Dv;
    for (int d = 0; d < c->Dv; ++d) o[d] = 0.0;
    double denom = 0.0;
    for (int j = 0; j < c->k; ++j) {
      if (sel[j] < 0) continue;
      double e = exp(z[j] - m);
      denom += e;
      for (int d = 0; d < c->Dv; ++d) o[d] += e * v_value(c, b, sel[j], g, d);
    }
    if (denom == 0.0) {  /* no valid entry (a NaN logit makes denom NaN: NaN results) */
      if (c->lse) c->lse[row * c->H + h] = -INFINITY;
    } else {
      for (int d = 0; d < c->Dv; ++d) o[d] /= denom;
      if (c->lse) c->lse[row * c->H + h] = m + log(denom);
    }
  }
  free(z);
}

int oracle_sparse_attn(const void* q, const void* kv, const float* kv_scale, const void* v,
                       int kv_fmt, const int32_t* idx, int B, int Tq, int Tk, int H, int Hkv,
                       int Dqk, int Dv, int k, double sm_scale, double* out, double* lse,
                       int nthreads) {
  if (!q || !kv || !idx || !out || B < 0 || Tq < 0 || Tk < 0 || H < 1 || Hkv < 1 || H % Hkv ||
      Dqk < 1 || Dv < 1 || k < 1 || kv_fmt < 0 || kv_fmt > 2)
    return 1;
  if (kv_fmt == 1 && (!kv_scale || v)) return 1;
  if (kv_fmt == 2 && (kv_scale || v || Dqk % 32 || Dqk > 1024)) return 1;
  if (!v && Dv > Dqk) return 1;
  for (int64_t r = 0; r < (int64_t)B * Tq * k; ++r)
    if (idx[r] >= Tk) return 2;
  attn_ctx c = {q, kv, v, kv_scale, kv_fmt, idx, B, Tq, Tk, H, Hkv, Dqk, Dv, k, sm_scale, out, lse};
  for_rows((int64_t)B * Tq, nthreads, attn_row, &c);
  return 0;
}

/* ---------- whole row, streamed: scores -> top-k -> attention ---------- */
/* The three steps above for a set of query rows of one sequence, one row at a time with
 * O(Tk) memory per thread, used to time the oracle on a sample of a long workload. */

typedef struct {
  const uint16_t *q_idx, *k_idx, *w_idx, *q, *kv;
  const float* kv_scale;
  int kv_fmt;
  const int32_t* rows;
  int Tk, H_I, d_I, H, Dqk, Dv, k;
  double sm_scale;
  int32_t* idx_out;
  double* out;
} stream_ctx;

static void stream_row(void* c_, int64_t r) {
  stream_ctx* c = (stream_ctx*)c_;
  int32_t t = c->rows[r];
  int32_t kv_len = t + 1;
  float* sc = (float*)malloc(sizeof(float) * (size_t)c->Tk);
  idx_ctx ic = {c->q_idx + (int64_t)t * c->H_I * c->d_I, c->k_idx, c->w_idx + (int64_t)t * c->H_I,
                &kv_len, 1, 1, c->Tk, c->H_I, c->d_I, sc, c->Tk};
  idx_row(&ic, 0);
  topk_ctx tc = {sc, c->Tk, &kv_len, 1, 1, c->Tk, c->k, c->idx_out + r * c->k};
  topk_row(&tc, 0);
  attn_ctx ac = {c->q + (int64_t)t * c->H * c->Dqk, c->kv, NULL, c->kv_scale, c->kv_fmt,
                 c->idx_out + r * c->k, 1, 1, c->Tk, c->H, 1, c->Dqk, c->Dv, c->k,
                 c->sm_scale, c->out + r * c->H * c->Dv, NULL};
  attn_row(&ac, 0);
  free(sc);
}

int oracle_dsa_rows(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w_idx,
                    const uint16_t* q, const void* kv, const float* kv_scale, int kv_fmt,
                    const int32_t* rows, int nrows, int Tk, int H_I, int d_I, int H, int Dqk,
                    int Dv, int k, double sm_scale, int32_t* idx_out, double* out, int nthreads) {
  if (!q_idx || !k_idx || !w_idx || !q || !kv || !rows || !idx_out || !out || nrows < 0 || k < 1 ||
      kv_fmt < 0 || kv_fmt > 2)
    return 1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= Tk) return 2;
  stream_ctx c = {q_idx, k_idx, w_idx, q, (const uint16_t*)kv, kv_scale, kv_fmt, rows, Tk, H_I,
                  d_I, H, Dqk, Dv, k, sm_scale, idx_out, out};
  for_rows(nrows, nthreads, stream_row, &c);
  return 0;
}

/* ---------- indexer training objective ---------- */
/* "DSA ablation model card", model list: the indexer is trained with a KL loss against the
 * main attention distribution, which is detached; the first tenth of the steps run dense
 * attention (indexer warm-up).  The pages give no formula.  Reading: for query row t with
 * key set S_t (its valid index entries; in the dense warm-up every causal key 0..p),
 *   P_s = (1/H) sum_h softmax_{s in S_t}(sm_scale * q_h . K_{s,g(h)})      target, held fixed
 *   Q_s = softmax_{s in S_t}(I_s),   I_s = sum_j w_j max(0, q_j . k_s)     indexer (as in 1.)
 *   L_t = KL(P || Q) = sum_s P_s (log P_s - log Q_s)        (a term with P_s = 0 is 0)
 * and the gradients of sum_t L_t with respect to the indexer inputs, with G_s = dL_t/dI_s =
 * Q_s - P_s and d_js = q_j . k_s (the ReLU's derivative taken as 0 at 0):
 *   dw_j = sum_s G_s max(0, d_js),  dq_j = sum_s G_s w_j [d_js > 0] k_s,
 *   dk_s = sum over rows t and heads j of G_ts w_tj [d_tjs > 0] q_tj.
 * An index entry < 0 is skipped (a duplicate counts twice, as in attention); a row with no
 * key has L_t = 0 and no gradient.  Inputs here are doubles (the bf16 entry decodes first). */

typedef struct {
  const double *qi, *ki, *wi, *q, *k;
  const int32_t *kv_len, *idx;
  int B, Tq, Tk, H_I, d_I, H, Hkv, Dqk, kk, width;
  double sm_scale;
  double *loss, *dq, *dw;
  int32_t* keys; /* [rows][width]: the row's key list, -1 past its end */
  double* G;     /* [rows][width]: dL_t/dI for each listed key */
} kl_ctx;

static void kl_row(void* c_, int64_t row) {
  kl_ctx* c = (kl_ctx*)c_;
  int b = (int)(row / c->Tq), i = (int)(row % c->Tq);
  int32_t* keys = c->keys + row * c->width;
  double* G = c->G + row * c->width;
  int n = 0;
  if (c->idx) {
    for (int e = 0; e < c->kk; ++e)
      if (c->idx[row * c->kk + e] >= 0) keys[n++] = c->idx[row * c->kk + e];
  } else {
    int64_t p = query_pos(c->kv_len, b, c->Tq, c->Tk, i);
    for (int64_t s = 0; s <= p && s < c->Tk; ++s) keys[n++] = (int32_t)s;
  }
  for (int e = n; e < c->width; ++e) keys[e] = -1;
  const double* qi = c->qi + row * c->H_I * c->d_I;
  const double* wi = c->wi + row * c->H_I;
  double* dq = c->dq + row * c->H_I * c->d_I;
  double* dw = c->dw + row * c->H_I;
  for (int x = 0; x < c->H_I * c->d_I; ++x) dq[x] = 0.0;
  for (int j = 0; j < c->H_I; ++j) dw[j] = 0.0;
  c->loss[row] = 0.0;
  if (n == 0) return;
  double* P = (double*)calloc((size_t)n, sizeof(double));
  double* z = (double*)malloc(sizeof(double) * (size_t)n);
  double* I = (double*)malloc(sizeof(double) * (size_t)n);
  /* target: the mean over heads of each head's softmax over the key set */
  for (int h = 0; h < c->H; ++h) {
    int g = h * c->Hkv / c->H;
    const double* qh = c->q + (row * c->H + h) * c->Dqk;
    double m = -INFINITY, sum = 0.0;
    for (int e = 0; e < n; ++e) {
      const double* kr = c->k + (((int64_t)b * c->Tk + keys[e]) * c->Hkv + g) * c->Dqk;
      double dot = 0.0;
      for (int d = 0; d < c->Dqk; ++d) dot += qh[d] * kr[d];
      z[e] = c->sm_scale * dot;
      if (z[e] > m) m = z[e];
    }
    for (int e = 0; e < n; ++e) sum += exp(z[e] - m);
    for (int e = 0; e < n; ++e) P[e] += exp(z[e] - m) / sum / c->H;
  }
  /* indexer distribution over the same keys */
  double mI = -INFINITY, sumI = 0.0;
  for (int e = 0; e < n; ++e) {
    const double* kr = c->ki + ((int64_t)b * c->Tk + keys[e]) * c->d_I;
    double total = 0.0;
    for (int j = 0; j < c->H_I; ++j) {
      double dot = 0.0;
      for (int d = 0; d < c->d_I; ++d) dot += qi[j * c->d_I + d] * kr[d];
      total += wi[j] * (dot > 0.0 ? dot : 0.0);
    }
    I[e] = total;
    if (I[e] > mI) mI = I[e];
  }
  for (int e = 0; e < n; ++e) sumI += exp(I[e] - mI);
  double lse_I = mI + log(sumI);
  double L = 0.0;
  for (int e = 0; e < n; ++e) {
    double logQ = I[e] - lse_I;
    if (P[e] > 0.0) L += P[e] * (log(P[e]) - logQ);
    G[e] = exp(logQ) - P[e];
  }
  c->loss[row] = L;
  /* the row's own indexer inputs */
  for (int e = 0; e < n; ++e) {
    const double* kr = c->ki + ((int64_t)b * c->Tk + keys[e]) * c->d_I;
    for (int j = 0; j < c->H_I; ++j) {
      double dot = 0.0;
      for (int d = 0; d < c->d_I; ++d) dot += qi[j * c->d_I + d] * kr[d];
      if (dot > 0.0) {
        dw[j] += G[e] * dot;
        for (int d = 0; d < c->d_I; ++d) dq[j * c->d_I + d] += G[e] * wi[j] * kr[d];
      }
    }
  }
  free(P);
  free(z);
  free(I);
}

int oracle_indexer_kl_f64(const double* q_idx, const double* k_idx, const double* w_idx,
                          const double* q, const double* k, const int32_t* kv_len,
                          const int32_t* idx, int B, int Tq, int Tk, int H_I, int d_I, int H,
                          int Hkv, int Dqk, int kk, double sm_scale, double* loss,
                          double* dq_idx, double* dw_idx, double* dk_idx, int nthreads) {
  if (!q_idx || !k_idx || !w_idx || !q || !k || !loss || !dq_idx || !dw_idx || !dk_idx || B < 0 ||
      Tq < 0 || Tk < 0 || H_I < 1 || d_I < 1 || H < 1 || Hkv < 1 || H % Hkv || Dqk < 1 ||
      (idx && kk < 1))
    return 1;
  int64_t rows = (int64_t)B * Tq;
  if (idx)
    for (int64_t r = 0; r < rows * kk; ++r)
      if (idx[r] >= Tk) return 2;
  int width = idx ? kk : (Tk > 0 ? Tk : 1);
  kl_ctx c = {q_idx, k_idx, w_idx, q, k, kv_len, idx, B, Tq, Tk, H_I, d_I, H, Hkv, Dqk, kk, width,
              sm_scale, loss, dq_idx, dw_idx, NULL, NULL};
  c.keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows > 0 ? rows : 1) * width);
  c.G = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * width);
  for_rows(rows, nthreads, kl_row, &c);
  /* key gradients: every row's contributions, rows in order */
  for (int64_t x = 0; x < (int64_t)B * Tk * d_I; ++x) dk_idx[x] = 0.0;
  for (int64_t row = 0; row < rows; ++row) {
    int b = (int)(row / Tq);
    const double* qi = q_idx + row * H_I * d_I;
    const double* wi = w_idx + row * H_I;
    for (int e = 0; e < width && c.keys[row * width + e] >= 0; ++e) {
      int64_t s = c.keys[row * width + e];
      const double* kr = k_idx + ((int64_t)b * Tk + s) * d_I;
      double* dk = dk_idx + ((int64_t)b * Tk + s) * d_I;
      for (int j = 0; j < H_I; ++j) {
        double dot = 0.0;
        for (int d = 0; d < d_I; ++d) dot += qi[j * d_I + d] * kr[d];
        if (dot > 0.0)
          for (int d = 0; d < d_I; ++d) dk[d] += c.G[row * width + e] * wi[j] * qi[j * d_I + d];
      }
    }
  }
  free(c.keys);
  free(c.G);
  return 0;
}

static double* decode_bf16_array(const uint16_t* x, int64_t n) {
  double* y = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_bf16_to_double(x[i]);
  return y;
}

int oracle_indexer_kl(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w_idx,
                      const uint16_t* q, const uint16_t* k, const int32_t* kv_len,
                      const int32_t* idx, int B, int Tq, int Tk, int H_I, int d_I, int H, int Hkv,
                      int Dqk, int kk, double sm_scale, double* loss, double* dq_idx,
                      double* dw_idx, double* dk_idx, int nthreads) {
  if (!q_idx || !k_idx || !w_idx || !q || !k || B < 0 || Tq < 0 || Tk < 0 || H_I < 1 || d_I < 1 ||
      H < 1 || Hkv < 1 || Dqk < 1)
    return 1;
  int64_t rows = (int64_t)B * Tq;
  double* a = decode_bf16_array(q_idx, rows * H_I * d_I);
  double* bk = decode_bf16_array(k_idx, (int64_t)B * Tk * d_I);
  double* w = decode_bf16_array(w_idx, rows * H_I);
  double* qq = decode_bf16_array(q, rows * H * Dqk);
  double* kk2 = decode_bf16_array(k, (int64_t)B * Tk * Hkv * Dqk);
  int rc = oracle_indexer_kl_f64(a, bk, w, qq, kk2, kv_len, idx, B, Tq, Tk, H_I, d_I, H, Hkv, Dqk,
                                 kk, sm_scale, loss, dq_idx, dw_idx, dk_idx, nthreads);
  free(a);
  free(bk);
  free(w);
  free(qq);
  free(kk2);
  return rc;
}
