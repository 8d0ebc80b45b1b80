/*
 * moe_oracle.c -- plain, slow CPU oracle for the DeepSeekMoE layer forward.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, links it or
 * shares a line of code, a header or a table with it.
 *
 * Every function states the passage it follows.  Pages cited:
 *   [ZH]  "190行JAX复刻DeepSeek V3" (openai-hub.com news)
 *   [VI]  "DeepSeek V3 viết lại bằng 190 dòng JAX thuần" (lehuy.net)
 *   [ES]  "DeepSeek V3 JAX: arquitectura recreada en 190 líneas y entrenada
 *          en un MacBook Air" (geekiki.com)
 * What the pages leave open is fixed by a stated reading (marked READING);
 * every reading is listed in the design notes of the repository.
 *
 * Arithmetic policy.  IEEE binary32/binary64, round to nearest even, no
 * fast-math, no FP contraction except the explicit fmaf() calls of the
 * router.  bf16 -> fp32 is exact widening; rounding to bf16 is round to
 * nearest even (NaN stays NaN).  Floating point is evaluated in fp64 except
 * where the precision is part of the definition:
 *   - router logits: an fp32 fused multiply-add chain over d in ascending
 *     order (READING: the layer computes in bf16 over f32 master weights,
 *     [VI] section "Những gì có trong 190 dòng code"; the router is kept in
 *     fp32 with one fixed summation order so that expert choice -- an
 *     integer decision -- is reproducible bit for bit);
 *   - scores, keys and gates are fp32 values, because selection compares
 *     them and the gates are an fp32 output.
 * The oracle is not blocked, fused or reordered: each loop is the plain
 * definition.  Threads only split independent tokens.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even. */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp64 -> bf16 with a single rounding (nearest, ties to even).  The value is
 * first rounded to fp32 *to odd* (truncate, then set the last bit when the
 * conversion was inexact); fp32 carries 16 more bits than bf16, so the second
 * rounding cannot create a double-rounding error (Boldo & Melquiond, "When
 * double rounding is odd", 2005). */
static uint16_t f64_to_bf16(double v) {
  if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
  float f = (float)v;
  if (!isinf(f) && (double)f != v) {
    if (fabs((double)f) > fabs(v)) f = nextafterf(f, 0.0f);
    uint32_t u;
    memcpy(&u, &f, 4);
    u |= 1u;
    memcpy(&f, &u, 4);
  }
  return f32_to_bf16(f);
}

uint16_t oracle_f32_to_bf16(float f) { return f32_to_bf16(f); }
uint16_t oracle_f64_to_bf16(double v) { return f64_to_bf16(v); }

/* ------------------------------------------------------------------ */
/* Tiny parallel-for over independent items                            */
/* ------------------------------------------------------------------ */

typedef void (*item_fn)(void* ctx, int64_t i);
typedef struct {
  item_fn fn;
  void* ctx;
  int64_t lo, hi;
} span_t;

static void* run_span(void* p) {
  span_t* s = (span_t*)p;
  for (int64_t i = s->lo; i < s->hi; ++i) s->fn(s->ctx, i);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, item_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n < nthreads) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    for (int64_t i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  pthread_t th[256];
  span_t sp[256];
  for (int t = 0; t < nthreads; ++t) {
    sp[t].fn = fn;
    sp[t].ctx = ctx;
    sp[t].lo = n * t / nthreads;
    sp[t].hi = n * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, run_span, &sp[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* Routing: logits, scores, biased top-k, gates                        */
/* ------------------------------------------------------------------ */

/* Router logit of token row x for expert e:
 *   acc = 0; for i = 0..d-1: acc = fmaf(x[i], W_r[i][e], acc)
 * Each token is sent to some of the experts by a learned router
 * ([ZH] section 190行代码到底装进了什么).  The fp32 fmaf chain in ascending i
 * is the fixed reduction order (READING, see the header). */
static float router_logit(int d, int E, const uint16_t* xrow, const float* w_router, int e) {
  float acc = 0.0f;
  for (int i = 0; i < d; ++i) acc = fmaf(bf16_to_f32(xrow[i]), w_router[(size_t)i * E + e], acc);
  return acc;
}

/* Affinity score: the logistic function of the logit, evaluated in fp64 and
 * rounded once to fp32.  READING: the pages do not name the affinity
 * function; sigmoid is the stated choice (the generic softmax illustration on
 * the n1n.ai page contradicts the project's own top-4 description and is not
 * followed). */
static float sigmoid_score(float logit) {
  return (float)(1.0 / (1.0 + exp(-(double)logit)));
}

/* Selection order over (key, expert) pairs: larger key first; NaN keys below
 * every other key; equal keys (+0 == -0) go to the lower expert index.
 * Returns nonzero when (ka, ea) is selected before (kb, eb).
 * READING: tie-break and NaN placement are not on the pages. */
static int ranks_before(float ka, int ea, float kb, int eb) {
  int na = isnan(ka), nb = isnan(kb);
  if (na || nb) {
    if (na && nb) return ea < eb;
    return nb; /* a is a number, b is NaN */
  }
  if (ka > kb) return 1;
  if (ka < kb) return 0;
  return ea < eb;
}

typedef struct {
  int64_t T;
  int d, E, k;
  const uint16_t* x;
  const float* w_router;
  const float* bias;
  int32_t* idx;
  float* gate;
  float* margin;
  float* scores; /* [T,E] or NULL */
} route_ctx;

/* One token of the routing step.
 *   key_e = s_e + b_e (one fp32 add): the per-expert bias shifts which
 *   experts win, and only that ([ZH] section 最有价值的实验:无辅助损失均衡真的
 *   有效; [VI] section Những gì có trong 190 dòng code).
 *   The k winners are the k largest keys; slot j holds the j-th largest.
 *   16 routed experts with 4 chosen per token in the mini model, 256 with 8
 *   in the official shape ([ZH] 190行代码到底装进了什么 and the comparison table
 *   in 先说结论).
 *   Gates use the unbiased scores of the winners, normalised over the k
 *   winners: g_j = s_{idx_j} / sum_j' s_{idx_j'} with the sum taken in fp32 in
 *   slot order (READING: the normalisation is not on the pages; the bias never
 *   enters it, as [ZH] 最有价值的实验 requires).  A zero sum (every winner's
 *   sigmoid underflowed) gives g_j = 1/k.
 *   margin = key_(k) - key_(k+1) in fp32; +inf when k == E. */
static void route_token(void* p, int64_t t) {
  route_ctx* c = (route_ctx*)p;
  const int d = c->d, E = c->E, k = c->k;
  float* s = (float*)malloc(sizeof(float) * (size_t)E);
  float* key = (float*)malloc(sizeof(float) * (size_t)E);
  char* taken = (char*)calloc((size_t)E, 1);
  const uint16_t* xrow = c->x + (size_t)t * d;
  for (int e = 0; e < E; ++e) {
    s[e] = sigmoid_score(router_logit(d, E, xrow, c->w_router, e));
    key[e] = s[e] + c->bias[e];
    if (c->scores) c->scores[(size_t)t * E + e] = s[e];
  }
  float kth = 0.0f;
  for (int j = 0; j <= k && j < E; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(key[e], e, key[best], best)) best = e;
    }
    if (j < k) {
      taken[best] = 1;
      c->idx[t * k + j] = best;
      kth = key[best];
    } else if (c->margin) {
      c->margin[t] = kth - key[best];
    }
  }
  if (c->margin && k == E) c->margin[t] = INFINITY;
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += s[c->idx[t * k + j]];
  for (int j = 0; j < k; ++j)
    c->gate[t * k + j] = (sum == 0.0f) ? 1.0f / (float)k : s[c->idx[t * k + j]] / sum;
  free(s);
  free(key);
  free(taken);
}

/* Routing of T tokens (steps a1-a4).  x [T,d] bf16 bits, w_router [d,E] fp32,
 * bias [E] fp32 -> idx [T,k] int32, gate [T,k] fp32, margin [T] (or NULL),
 * scores [T,E] (or NULL). */
void oracle_route(int64_t T, int d, int E, int k, const uint16_t* x, const float* w_router,
                  const float* bias, int32_t* idx, float* gate, float* margin, float* scores,
                  int nthreads) {
  route_ctx c = {T, d, E, k, x, w_router, bias, idx, gate, margin, scores};
  parallel_for(T, nthreads, route_token, &c);
}

/* Logits alone, for the pins: logits [T,E]. */
void oracle_logits(int64_t T, int d, int E, const uint16_t* x, const float* w_router,
                   float* logits) {
  for (int64_t t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e)
      logits[t * E + e] = router_logit(d, E, x + (size_t)t * d, w_router, e);
}

float oracle_sigmoid(float logit) { return sigmoid_score(logit); }

/* Selection alone (keys given), for the pins. */
void oracle_select(int64_t T, int E, int k, const float* keys, int32_t* idx) {
  char* taken = (char*)malloc((size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float* key = keys + t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(key[e], e, key[best], best)) best = e;
      }
      taken[best] = 1;
      idx[t * k + j] = best;
    }
  }
  free(taken);
}

/* ------------------------------------------------------------------ */
/* Sequence-wise balance statistic (step a5)                           */
/* ------------------------------------------------------------------ */

/* The mini model keeps a small sequence-wise balance loss from the original
 * report, weight alpha = 1e-4 ([ZH] 最有价值的实验; [VI] Những gì có trong 190
 * dòng code).  READING of its formula (the pages do not print it), per
 * sequence b of S consecutive tokens:
 *   f_i = E / (k S) * #{t in b : i is among t's selected experts}
 *   P_i = 1/S * sum_{t in b} s_{t,i} / sum_{j<E} s_{t,j}
 *   L_b = alpha * sum_i f_i P_i
 * "Selected" is the routing actually used (with the bias).  A token whose
 * scores sum to zero contributes 1/E to every P_i.  fp64 throughout. */
void oracle_seq_balance(int64_t T, int E, int k, int S, const float* scores, const int32_t* idx,
                        double alpha, double* L) {
  int64_t B = T / S;
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  double* P = (double*)malloc(sizeof(double) * (size_t)E);
  for (int64_t b = 0; b < B; ++b) {
    for (int i = 0; i < E; ++i) {
      cnt[i] = 0;
      P[i] = 0.0;
    }
    for (int64_t t = b * S; t < (b + 1) * S; ++t) {
      double tot = 0.0;
      for (int j = 0; j < E; ++j) tot += (double)scores[t * E + j];
      for (int i = 0; i < E; ++i)
        P[i] += (tot == 0.0) ? 1.0 / E : (double)scores[t * E + i] / tot;
      for (int j = 0; j < k; ++j) cnt[idx[t * k + j]] += 1;
    }
    double acc = 0.0;
    for (int i = 0; i < E; ++i) {
      double f = (double)E / ((double)k * (double)S) * (double)cnt[i];
      acc += f * (P[i] / (double)S);
    }
    L[b] = alpha * acc;
  }
  free(cnt);
  free(P);
}

/* ------------------------------------------------------------------ */
/* Loads and grouping by expert (steps a6-a7)                          */
/* ------------------------------------------------------------------ */

/* counts[e] = number of (token, slot) pairs routed to e -- the per-expert
 * load that the bias rule reads ([ZH] 最有价值的实验, ablation table).
 * offsets = exclusive prefix sum of counts, offsets[E] = T*k.
 * Rows of expert e are the tokens that chose e in ascending token order
 * (READING: the pages have no sparse dispatch at all -- [VI] section Những gì
 * đã được đơn giản hóa -- so the order inside a group is fixed here to make
 * the layout deterministic).  perm_src[row] = token; pos[t*k+j] = row of the
 * pair (t, idx[t*k+j]). */
void oracle_permute(int64_t T, int E, int k, const int32_t* idx, int32_t* counts,
                    int32_t* offsets, int32_t* perm_src, int32_t* pos) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < T * k; ++i) counts[idx[i]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      int32_t row = fill[e]++;
      perm_src[row] = (int32_t)t;
      pos[t * k + j] = row;
    }
  free(fill);
}

/* ------------------------------------------------------------------ */
/* Expert feed-forward network (steps a8-a9)                           */
/* ------------------------------------------------------------------ */

/* One expert on one token row: y = W2 (silu(W1 x) * (W3 x)).
 * The experts are feed-forward networks ([ZH] 190行代码到底装进了什么).
 * READING: the gated SiLU form (SwiGLU) and its storage points are not on the
 * pages.  W1, W3 are [H, d] and W2 is [d, H], row-major bf16.  The gate and
 * up projections are accumulated in fp64; the hidden activation is stored
 * in bf16 (activations are bf16 under the pages' bf16 compute, [VI] Những gì
 * có trong 190 dòng code); the output is accumulated in fp64 and rounded
 * once to bf16. */
void oracle_expert_ffn(int d, int H, const uint16_t* xrow, const uint16_t* w1,
                       const uint16_t* w3, const uint16_t* w2, uint16_t* y) {
  double* h = (double*)malloc(sizeof(double) * (size_t)H);
  for (int r = 0; r < H; ++r) {
    double a = 0.0, b = 0.0;
    for (int i = 0; i < d; ++i) {
      double xv = (double)bf16_to_f32(xrow[i]);
      a += xv * (double)bf16_to_f32(w1[(size_t)r * d + i]);
      b += xv * (double)bf16_to_f32(w3[(size_t)r * d + i]);
    }
    double silu = a / (1.0 + exp(-a));
    h[r] = (double)bf16_to_f32(f64_to_bf16(silu * b));
  }
  for (int o = 0; o < d; ++o) {
    double acc = 0.0;
    for (int r = 0; r < H; ++r) acc += h[r] * (double)bf16_to_f32(w2[(size_t)o * H + r]);
    y[o] = f64_to_bf16(acc);
  }
  free(h);
}

typedef struct {
  int64_t T;
  int d, E, H, Hs;
  const uint16_t* x;
  const int32_t* perm_src;
  const int32_t* offsets;
  const uint16_t *w1, *w3, *w2, *ws1, *ws3, *ws2;
  uint16_t* y_perm;
  uint16_t* y_shared;
  int64_t routed_rows;
} ffn_ctx;

static void ffn_item(void* p, int64_t i) {
  ffn_ctx* c = (ffn_ctx*)p;
  const int d = c->d, H = c->H;
  if (i < c->routed_rows) {
    int e = 0;
    while (!(c->offsets[e] <= i && i < c->offsets[e + 1])) ++e;
    size_t eo = (size_t)e * H * d;
    oracle_expert_ffn(d, H, c->x + (size_t)c->perm_src[i] * d, c->w1 + eo, c->w3 + eo, c->w2 + eo,
                      c->y_perm + (size_t)i * d);
  } else {
    int64_t t = i - c->routed_rows;
    oracle_expert_ffn(d, c->Hs, c->x + (size_t)t * d, c->ws1, c->ws3, c->ws2,
                      c->y_shared + (size_t)t * d);
  }
}

/* Grouped FFN over the expert groups: row r of group e (rows offsets[e] ..
 * offsets[e+1]-1) is expert e applied to token perm_src[r]; only chosen
 * experts run (the sparse dispatch the pages' dense reference lacks, [VI]
 * Những gì đã được đơn giản hóa).  The shared expert runs on every token
 * ([ZH] 190行代码到底装进了什么).  ws1 == NULL: no shared expert. */
void oracle_grouped_ffn(int64_t T, int d, int E, int k, int H, int Hs, const uint16_t* x,
                        const int32_t* perm_src, const int32_t* offsets, const uint16_t* w1,
                        const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                        const uint16_t* ws3, const uint16_t* ws2, uint16_t* y_perm,
                        uint16_t* y_shared, int nthreads) {
  ffn_ctx c = {T, d, E, H, Hs, x, perm_src, offsets, w1, w3, w2, ws1, ws3, ws2, y_perm, y_shared,
               T * k};
  int64_t n = T * k + (ws1 ? T : 0);
  parallel_for(n, nthreads, ffn_item, &c);
}

/* ------------------------------------------------------------------ */
/* Combine (step a10)                                                   */
/* ------------------------------------------------------------------ */

/* out[t] = bf16( residual[t] + y_shared[t] + sum over t's chosen experts, in
 * ascending expert index, of g * y_perm[row] ), accumulated in fp64 in that
 * order.  The always-on shared expert is added to the routed mixture ([ZH]
 * 190行代码到底装进了什么).  residual / y_shared may be NULL (READING: the
 * optional residual is the Transformer block's residual stream, which the
 * stacked-layer workload adds here). */
void oracle_combine(int64_t T, int d, int E, int k, const uint16_t* y_perm,
                    const uint16_t* y_shared, const float* gate, const int32_t* idx,
                    const int32_t* pos, const uint16_t* residual, uint16_t* out) {
  int* order = (int*)malloc(sizeof(int) * (size_t)k);
  for (int64_t t = 0; t < T; ++t) {
    /* slots sorted by ascending expert index */
    for (int j = 0; j < k; ++j) order[j] = j;
    for (int a = 1; a < k; ++a)
      for (int b = a; b > 0 && idx[t * k + order[b]] < idx[t * k + order[b - 1]]; --b) {
        int tmp = order[b];
        order[b] = order[b - 1];
        order[b - 1] = tmp;
      }
    for (int o = 0; o < d; ++o) {
      double acc = 0.0;
      if (residual) acc += (double)bf16_to_f32(residual[(size_t)t * d + o]);
      if (y_shared) acc += (double)bf16_to_f32(y_shared[(size_t)t * d + o]);
      for (int a = 0; a < k; ++a) {
        int j = order[a];
        acc += (double)gate[t * k + j] *
               (double)bf16_to_f32(y_perm[(size_t)pos[t * k + j] * d + o]);
      }
      out[(size_t)t * d + o] = f64_to_bf16(acc);
    }
  }
  free(order);
}

/* ------------------------------------------------------------------ */
/* Dense, masked evaluation: the pages' own formulation (pin)          */
/* ------------------------------------------------------------------ */

typedef struct {
  int64_t T;
  int d, E, k, H, Hs;
  const uint16_t* x;
  const float* gate;
  const int32_t* idx;
  const uint16_t *w1, *w3, *w2, *ws1, *ws3, *ws2;
  const uint16_t* residual;
  uint16_t* out;
} dense_ctx;

static void dense_token(void* p, int64_t t) {
  dense_ctx* c = (dense_ctx*)p;
  const int d = c->d, E = c->E, k = c->k, H = c->H;
  uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)E * d);
  uint16_t* ys = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
  float* g = (float*)calloc((size_t)E, sizeof(float));
  const uint16_t* xrow = c->x + (size_t)t * d;
  for (int e = 0; e < E; ++e) {
    size_t eo = (size_t)e * H * d;
    oracle_expert_ffn(d, H, xrow, c->w1 + eo, c->w3 + eo, c->w2 + eo, y + (size_t)e * d);
  }
  if (c->ws1) oracle_expert_ffn(d, c->Hs, xrow, c->ws1, c->ws3, c->ws2, ys);
  for (int j = 0; j < k; ++j) g[c->idx[t * k + j]] = c->gate[t * k + j];
  for (int o = 0; o < d; ++o) {
    double acc = 0.0;
    if (c->residual) acc += (double)bf16_to_f32(c->residual[(size_t)t * d + o]);
    if (c->ws1) acc += (double)bf16_to_f32(ys[o]);
    for (int e = 0; e < E; ++e) acc += (double)g[e] * (double)bf16_to_f32(y[(size_t)e * d + o]);
    c->out[(size_t)t * d + o] = f64_to_bf16(acc);
  }
  free(y);
  free(ys);
  free(g);
}

/* Every routed expert runs on every token and the experts a token did not
 * choose get weight zero -- how the pages' reference evaluates the layer
 * ([ZH] 190行代码到底装进了什么; [VI] Những gì đã được đơn giản hóa).  Used
 * only as a brute-force cross-check of the sparse path. */
void oracle_dense_masked(int64_t T, int d, int E, int k, int H, int Hs, const uint16_t* x,
                         const float* gate, const int32_t* idx, const uint16_t* w1,
                         const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                         const uint16_t* ws3, const uint16_t* ws2, const uint16_t* residual,
                         uint16_t* out, int nthreads) {
  dense_ctx c = {T, d, E, k, H, Hs, x, gate, idx, w1, w3, w2, ws1, ws3, ws2, residual, out};
  parallel_for(T, nthreads, dense_token, &c);
}

/* ------------------------------------------------------------------ */
/* RMSNorm before the MoE in a pre-norm residual block                 */
/* ------------------------------------------------------------------ */

/* The model's layers are pure functions over arrays, RMSNorm among them
 * ([ZH] section "纯JAX"也需要打一个小星号), and the MoE sits in a residual
 * Transformer block ([ZH] section 先说结论).  READING (the pages give
 * neither the formula's constants nor the placement): a pre-norm block
 * x_next = x + MoE(RMSNorm(x)), with
 *   out[t,i] = bf16( x[t,i] / sqrt(mean_j x[t,j]^2 + eps) * g[i] )
 * evaluated in fp64 and rounded once to bf16; g is the norm's learned fp32
 * gain, eps is passed in (1e-6 in the workloads). */
void oracle_rmsnorm(int64_t T, int d, const uint16_t* x, const float* g, double eps,
                    uint16_t* out) {
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* xr = x + (size_t)t * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) {
      double v = (double)bf16_to_f32(xr[i]);
      ss += v * v;
    }
    double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int i = 0; i < d; ++i)
      out[(size_t)t * d + i] = f64_to_bf16((double)bf16_to_f32(xr[i]) * r * (double)g[i]);
  }
}

/* ------------------------------------------------------------------ */
/* Bias update (step a11)                                              */
/* ------------------------------------------------------------------ */

/* After each training step the bias of an overloaded expert goes down and
 * that of an idle expert goes up, at speed gamma = 1e-3 ([ZH] 最有价值的实验).
 *   b_i <- b_i + gamma * sgn(mean_load - load_i),  mean_load = T*k/E,
 * with sgn computed exactly as sgn(T*k - E*load_i) on integers and sgn(0) = 0
 * (READING: the sign form is the stated choice; the zero case is not on the
 * pages).  Both operations are fp32. */
void oracle_update_bias(int64_t T, int E, int k, const int32_t* counts, float* bias, float gamma) {
  for (int i = 0; i < E; ++i) {
    long long diff = (long long)T * k - (long long)E * counts[i];
    float sg = diff > 0 ? 1.0f : (diff < 0 ? -1.0f : 0.0f);
    bias[i] = bias[i] + gamma * sg;
  }
}
