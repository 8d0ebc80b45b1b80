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
/* Backward of the layer (training)                                    */
/* ------------------------------------------------------------------ */

/* The pages' workload is training: the model is trained for 12000 steps with
 * AdamW ([ZH] section 如何在Mac上复现), on a loss that adds the small
 * sequence-wise balance loss to the language-model loss ([ZH] section
 * 多Token预测也被保留了), while the per-expert bias stays outside the loss and
 * only moves the choice of experts ([ZH] section 最有价值的实验).
 *
 * With the choice of experts held fixed (it is piecewise constant), the
 * layer's output out[t] = r[t] + ys[t] + sum_j g[t,j] y[t,j] and the balance
 * statistic sum_b L_b are smooth functions of x and the weights.  For an
 * upstream gradient dout this computes the gradient of
 *   L = sum_t <dout[t], out[t]> + sum_b L_b
 * with respect to x, W_r and every expert weight, by the chain rule written
 * out step by step (the residual r passes dout through and is left to the
 * caller; the bias has no gradient).
 *
 * round_storage = 0: everything in fp64, no rounding -- the exact gradient of
 * the fp64 layer (oracle_moe_forward_f64), which finite differences pin.
 * round_storage = 1: the values the GPU path stores in bf16 or fp32 are
 * rounded at the same points (scores, keys and gates as in the forward;
 * h, y, dy = g * dout, dh, da, dc and each row's input gradient in bf16),
 * so that a comparison measures accumulation order only. */

static double sigm64(double v) { return 1.0 / (1.0 + exp(-v)); }
static double keep_bf16(double v, int round) {
  return round ? (double)bf16_to_f32(f64_to_bf16(v)) : v;
}

/* Scores and gates of every token, at the precision round_storage asks for. */
static void bwd_scores(int64_t T, int d, int E, int k, const double* x, const double* wr,
                       const int32_t* idx, int round, double* s, double* g, double* gsum) {
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      if (round) {
        float acc = 0.0f;
        for (int i = 0; i < d; ++i)
          acc = fmaf((float)x[(size_t)t * d + i], (float)wr[(size_t)i * E + e], acc);
        s[(size_t)t * E + e] = (double)sigmoid_score(acc);
      } else {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += x[(size_t)t * d + i] * wr[(size_t)i * E + e];
        s[(size_t)t * E + e] = sigm64(acc);
      }
    }
    double sum;
    if (round) {
      float fs = 0.0f;
      for (int j = 0; j < k; ++j) fs += (float)s[(size_t)t * E + idx[t * k + j]];
      sum = fs;
    } else {
      sum = 0.0;
      for (int j = 0; j < k; ++j) sum += s[(size_t)t * E + idx[t * k + j]];
    }
    gsum[t] = sum;
    for (int j = 0; j < k; ++j) {
      double sj = s[(size_t)t * E + idx[t * k + j]];
      double gj = sum == 0.0 ? 1.0 / k : sj / sum;
      g[t * k + j] = round ? (double)(float)gj : gj;
    }
  }
}

typedef struct {
  int64_t T;
  int d, E, k, H, Hs, round;
  const double *x, *w1, *w3, *w2, *ws1, *ws3, *ws2, *dout, *g;
  const int32_t* idx;
  double *dw1, *dw3, *dw2, *dws1, *dws3, *dws2;
  double* dxrow; /* [T, k+1, d]: input gradient of each routed row, then the shared row */
  double* dg;    /* [T, k]: <dout, y> of each routed row */
} bwd_ctx;

/* One expert (group < E) or the shared expert (group == E) over all of its
 * rows: recompute a = x W1^T, c = x W3^T, h = silu(a) c and y = h W2^T, then
 *   dy = gate * dout,  dg = <dout, y>,  dh = dy W2,
 *   da = dh * c * silu'(a),  dc = dh * silu(a),  silu'(a) = s(a) (1 + a (1 - s(a))),
 *   dW2 += dy^T h,  dW1 += da^T x,  dW3 += dc^T x,  dx_row = da W1 + dc W3.
 * Only this group writes its weight gradients, so groups run in parallel. */
static void bwd_group(void* p, int64_t grp) {
  bwd_ctx* c = (bwd_ctx*)p;
  const int d = c->d, k = c->k, rd = c->round;
  const int shared = grp == c->E;
  const int H = shared ? c->Hs : c->H;
  if (shared && H == 0) return;
  const size_t wo = shared ? 0 : (size_t)grp * H * d;
  const double* W1 = (shared ? c->ws1 : c->w1) + wo;
  const double* W3 = (shared ? c->ws3 : c->w3) + wo;
  const double* W2 = (shared ? c->ws2 : c->w2) + wo;
  double* dW1 = (shared ? c->dws1 : c->dw1) + wo;
  double* dW3 = (shared ? c->dws3 : c->dw3) + wo;
  double* dW2 = (shared ? c->dws2 : c->dw2) + wo;
  double* a = (double*)malloc(sizeof(double) * H);
  double* cc = (double*)malloc(sizeof(double) * H);
  double* hv = (double*)malloc(sizeof(double) * H);
  double* dh = (double*)malloc(sizeof(double) * H);
  double* da = (double*)malloc(sizeof(double) * H);
  double* dc = (double*)malloc(sizeof(double) * H);
  double* dy = (double*)malloc(sizeof(double) * d);
  for (int64_t t = 0; t < c->T; ++t) {
    int slot = -1;
    if (shared) {
      slot = k;
    } else {
      for (int j = 0; j < k; ++j)
        if (c->idx[t * k + j] == (int)grp) slot = j;
      if (slot < 0) continue;
    }
    const double* xr = c->x + (size_t)t * d;
    const double* dor = c->dout + (size_t)t * d;
    const double gate = shared ? 1.0 : c->g[t * k + slot];
    for (int h = 0; h < H; ++h) {
      double s1 = 0.0, s3 = 0.0;
      for (int i = 0; i < d; ++i) {
        s1 += xr[i] * W1[(size_t)h * d + i];
        s3 += xr[i] * W3[(size_t)h * d + i];
      }
      a[h] = s1;
      cc[h] = s3;
      hv[h] = keep_bf16(s1 * sigm64(s1) * s3, rd);
    }
    if (!shared) {
      double dot = 0.0;
      for (int o = 0; o < d; ++o) {
        double y = 0.0;
        for (int h = 0; h < H; ++h) y += hv[h] * W2[(size_t)o * H + h];
        dot += dor[o] * keep_bf16(y, rd);
      }
      c->dg[t * k + slot] = dot;
    }
    for (int o = 0; o < d; ++o) dy[o] = keep_bf16(gate * dor[o], rd);
    for (int h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int o = 0; o < d; ++o) acc += dy[o] * W2[(size_t)o * H + h];
      dh[h] = keep_bf16(acc, rd);
    }
    for (int o = 0; o < d; ++o)
      for (int h = 0; h < H; ++h) dW2[(size_t)o * H + h] += dy[o] * hv[h];
    for (int h = 0; h < H; ++h) {
      double sg = sigm64(a[h]);
      da[h] = keep_bf16(dh[h] * cc[h] * sg * (1.0 + a[h] * (1.0 - sg)), rd);
      dc[h] = keep_bf16(dh[h] * a[h] * sg, rd);
      for (int i = 0; i < d; ++i) {
        dW1[(size_t)h * d + i] += da[h] * xr[i];
        dW3[(size_t)h * d + i] += dc[h] * xr[i];
      }
    }
    double* dxo = c->dxrow + ((size_t)t * (k + 1) + slot) * d;
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h) acc += da[h] * W1[(size_t)h * d + i] + dc[h] * W3[(size_t)h * d + i];
      dxo[i] = keep_bf16(acc, rd);
    }
  }
  free(a); free(cc); free(hv); free(dh); free(da); free(dc); free(dy);
}

/* Gradient of L with respect to x [T,d], W_r [d,E] and the expert weights
 * (layouts as in the forward), all fp64 and overwritten.  x and the weights
 * are fp64 values (bf16 or fp32 numbers widened, or arbitrary reals for the
 * finite-difference pins); idx is the choice of experts to hold fixed.  The
 * balance term: per sequence b of S tokens, with p[t,i] = s[t,i] / Z_t and
 * Z_t = sum_e s[t,e], L_b = alpha sum_i f_i P_i, P_i = mean_t p[t,i] and
 * f_i = E/(kS) #{t in b choosing i}; so dL_b/ds[t,m] = alpha/S (f_m -
 * sum_i f_i p[t,i]) / Z_t.  The gates g_j = s_j / sum_j' s_j' give
 * dL/ds_m = (dg_m - sum_j dg_j g_j) / sum for a chosen m.  Then dlogit =
 * ds s (1 - s), dx += dlogit W_r^T and dW_r = x^T dlogit. */
void oracle_moe_backward(int64_t T, int d, int E, int k, int H, int Hs, int S, double alpha,
                         const double* x, const double* wr, const int32_t* idx, const double* w1,
                         const double* w3, const double* w2, const double* ws1, const double* ws3,
                         const double* ws2, const double* dout, int round_storage, double* dx,
                         double* dwr, double* dw1, double* dw3, double* dw2, double* dws1,
                         double* dws3, double* dws2, int nthreads) {
  double* s = (double*)calloc((size_t)T * E, sizeof(double));
  double* g = (double*)calloc((size_t)T * k, sizeof(double));
  double* gsum = (double*)calloc((size_t)T, sizeof(double));
  double* ds = (double*)calloc((size_t)T * E, sizeof(double));
  double* dg = (double*)calloc((size_t)T * k, sizeof(double));
  double* dxrow = (double*)calloc((size_t)T * (k + 1) * d, sizeof(double));
  memset(dw1, 0, sizeof(double) * (size_t)E * H * d);
  memset(dw3, 0, sizeof(double) * (size_t)E * H * d);
  memset(dw2, 0, sizeof(double) * (size_t)E * H * d);
  if (Hs) {
    memset(dws1, 0, sizeof(double) * (size_t)Hs * d);
    memset(dws3, 0, sizeof(double) * (size_t)Hs * d);
    memset(dws2, 0, sizeof(double) * (size_t)Hs * d);
  }
  bwd_scores(T, d, E, k, x, wr, idx, round_storage, s, g, gsum);
  bwd_ctx c = {T, d, E, k, H, Hs, round_storage, x, w1, w3, w2, ws1, ws3, ws2, dout, g, idx,
               dw1, dw3, dw2, dws1, dws3, dws2, dxrow, dg};
  parallel_for(E + 1, nthreads, bwd_group, &c);
  /* gates */
  for (int64_t t = 0; t < T; ++t) {
    if (gsum[t] == 0.0) continue; /* g = 1/k: constant */
    double gs = 0.0;
    for (int j = 0; j < k; ++j) gs += dg[t * k + j] * g[t * k + j];
    for (int j = 0; j < k; ++j) ds[(size_t)t * E + idx[t * k + j]] += (dg[t * k + j] - gs) / gsum[t];
  }
  /* sequence balance term */
  if (S > 0) {
    double* f = (double*)malloc(sizeof(double) * E);
    for (int64_t b0 = 0; b0 + S <= T; b0 += S) {
      for (int i = 0; i < E; ++i) f[i] = 0.0;
      for (int64_t t = b0; t < b0 + S; ++t)
        for (int j = 0; j < k; ++j) f[idx[t * k + j]] += (double)E / ((double)k * S);
      for (int64_t t = b0; t < b0 + S; ++t) {
        double Z = 0.0;
        for (int i = 0; i < E; ++i) Z += s[(size_t)t * E + i];
        if (Z == 0.0) continue;
        double q = 0.0;
        for (int i = 0; i < E; ++i) q += f[i] * s[(size_t)t * E + i] / Z;
        for (int m = 0; m < E; ++m) ds[(size_t)t * E + m] += alpha / S * (f[m] - q) / Z;
      }
    }
    free(f);
  }
  /* sigmoid, router, and the input gradient */
  memset(dwr, 0, sizeof(double) * (size_t)d * E);
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int j = 0; j <= k; ++j) acc += dxrow[((size_t)t * (k + 1) + j) * d + i];
      dx[(size_t)t * d + i] = acc;
    }
    for (int e = 0; e < E; ++e) {
      double se = s[(size_t)t * E + e];
      double dl = ds[(size_t)t * E + e] * se * (1.0 - se);
      if (dl == 0.0) continue;
      for (int i = 0; i < d; ++i) {
        dx[(size_t)t * d + i] += dl * wr[(size_t)i * E + e];
        dwr[(size_t)i * E + e] += x[(size_t)t * d + i] * dl;
      }
    }
  }
  free(s); free(g); free(gsum); free(ds); free(dg); free(dxrow);
}

/* The fp64 layer with the choice of experts held fixed and nothing rounded:
 * out[t] = sum_j g[t,j] y[t,j] + ys[t] (no residual), and *loss_bal =
 * sum_b L_b -- the function whose gradient oracle_moe_backward with
 * round_storage = 0 computes (checked against finite differences). */
void oracle_moe_forward_f64(int64_t T, int d, int E, int k, int H, int Hs, int S, double alpha,
                            const double* x, const double* wr, const int32_t* idx,
                            const double* w1, const double* w3, const double* w2,
                            const double* ws1, const double* ws3, const double* ws2, double* out,
                            double* loss_bal) {
  double* s = (double*)calloc((size_t)T * E, sizeof(double));
  double* g = (double*)calloc((size_t)T * k, sizeof(double));
  double* gsum = (double*)calloc((size_t)T, sizeof(double));
  int hmax = H > Hs ? H : Hs;
  double* hv = (double*)malloc(sizeof(double) * (hmax > 0 ? hmax : 1));
  bwd_scores(T, d, E, k, x, wr, idx, 0, s, g, gsum);
  for (int64_t t = 0; t < T; ++t) {
    const double* xr = x + (size_t)t * d;
    for (int o = 0; o < d; ++o) out[(size_t)t * d + o] = 0.0;
    for (int j = 0; j <= k; ++j) {
      const int shared = j == k;
      if (shared && !Hs) continue;
      const int Hg = shared ? Hs : H;
      const size_t wo = shared ? 0 : (size_t)idx[t * k + j] * H * d;
      const double* W1 = (shared ? ws1 : w1) + wo;
      const double* W3 = (shared ? ws3 : w3) + wo;
      const double* W2 = (shared ? ws2 : w2) + wo;
      const double gate = shared ? 1.0 : g[t * k + j];
      for (int h = 0; h < Hg; ++h) {
        double s1 = 0.0, s3 = 0.0;
        for (int i = 0; i < d; ++i) {
          s1 += xr[i] * W1[(size_t)h * d + i];
          s3 += xr[i] * W3[(size_t)h * d + i];
        }
        hv[h] = s1 * sigm64(s1) * s3;
      }
      for (int o = 0; o < d; ++o) {
        double y = 0.0;
        for (int h = 0; h < Hg; ++h) y += hv[h] * W2[(size_t)o * Hg + h];
        out[(size_t)t * d + o] += gate * y;
      }
    }
  }
  double lb = 0.0;
  if (S > 0) {
    for (int64_t b0 = 0; b0 + S <= T; b0 += S) {
      for (int i = 0; i < E; ++i) {
        double f = 0.0, P = 0.0;
        for (int64_t t = b0; t < b0 + S; ++t) {
          for (int j = 0; j < k; ++j)
            if (idx[t * k + j] == i) f += (double)E / ((double)k * S);
          double Z = 0.0;
          for (int e = 0; e < E; ++e) Z += s[(size_t)t * E + e];
          P += (Z == 0.0 ? 1.0 / E : s[(size_t)t * E + i] / Z) / S;
        }
        lb += alpha * f * P;
      }
    }
  }
  *loss_bal = lb;
  free(s); free(g); free(gsum); free(hv);
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

/* ------------------------------------------------------------------ */
/* MLA attention (the other half of the block)                         */
/* ------------------------------------------------------------------ */

/* Multi-head latent attention as the pages describe it ([ZH] sections
 * 190行代码到底装进了什么 and 先说结论; [VI] section Những gì có trong 190
 * dòng code, and section Những gì đã được đơn giản hóa for the explicit
 * decompression).  Per token, two things are cached: a latent of dc numbers
 * (128 in the mini model) from which the heads' keys and values are
 * decompressed, and one rotary key of dr numbers (16) shared by all heads --
 * 144 numbers per token and layer instead of the 480 of plain multi-head
 * attention with 6 heads.  The content part of keys and queries ("nope")
 * carries no position; the rotary part is rotated with the position.
 * READINGS (the pages give none of these formulas):
 *   q_h      = W_q[h] x,  split into q_nope (dn) and q_rope (dr), q_rope rotated
 *   c        = W_dkv x                      (the cached latent, dc)
 *   k_r      = rope(W_kr x)                 (the cached rotary key, dr)
 *   k_nope_h = W_uk[h] c,  v_h = W_uv[h] c  (decompressed explicitly)
 *   score_h(i, s) = (q_nope_h(i).k_nope_h(s) + q_rope_h(i).k_r(s)) / sqrt(dn + dr),
 *            causal (s <= i), softmax over s,
 *   o_h(i)   = sum_s p_h(i, s) v_h(s),   out(i) = r(i) + W_o concat_h o_h(i).
 * rope(u, p): pairs (u[2m], u[2m+1]) turn by the angle p * base^(-2m/dr),
 * base 10000; p = the token's position in its sequence.  The weights are
 * stored like the experts' ([N, K], K contiguous): W_q [nh (dn+dr), d],
 * W_dkv [dc, d], W_kr [dr, d], W_uk [nh dn, dc], W_uv [nh dv, dc],
 * W_o [d, nh dv].  round_storage = 1 rounds to bf16 where the GPU stores
 * bf16 (q, c, k_r, k_nope, v, o and out); 0 keeps everything in fp64.
 * Arguments are fp64 arrays (bf16 values widened). */

static void mla_rope(double* u, int dr, double pos, double base) {
  for (int m = 0; m < dr / 2; ++m) {
    double ang = pos * pow(base, -2.0 * m / dr);
    double c = cos(ang), s = sin(ang);
    double a = u[2 * m], b = u[2 * m + 1];
    u[2 * m] = a * c - b * s;
    u[2 * m + 1] = a * s + b * c;
  }
}

/* y[j] = sum_i W[j][i] x[i], i ascending, for j < n (W row-major [n, k]) */
static void mla_matvec(int n, int k, const double* W, const double* x, double* y, int round) {
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int i = 0; i < k; ++i) acc += W[(size_t)j * k + i] * x[i];
    y[j] = keep_bf16(acc, round);
  }
}

typedef struct {
  int d, nh, dc, dn, dr, dv, Lmax, round;
  double base;
  const double *wq, *wdkv, *wkr, *wuk, *wuv, *wo;
} mla_cfg;

/* token x at position p: q [nh (dn+dr)], latent c [dc], rotary key kr [dr] */
static void mla_project(const mla_cfg* m, const double* x, int p, double* q, double* c, double* kr) {
  const int qw = m->dn + m->dr;
  for (int h = 0; h < m->nh; ++h) {
    double* qh = q + (size_t)h * qw;
    mla_matvec(qw, m->d, m->wq + (size_t)h * qw * m->d, x, qh, 0);
    mla_rope(qh + m->dn, m->dr, p, m->base);
    for (int j = 0; j < qw; ++j) qh[j] = keep_bf16(qh[j], m->round);
  }
  mla_matvec(m->dc, m->d, m->wdkv, x, c, m->round);
  mla_matvec(m->dr, m->d, m->wkr, x, kr, 0);
  mla_rope(kr, m->dr, p, m->base);
  for (int j = 0; j < m->dr; ++j) kr[j] = keep_bf16(kr[j], m->round);
}

/* One query (q at position i) against cached positions 0..i of one sequence
 * (latents ckv [Lmax, dc], rotary keys ckr [Lmax, dr]); the keys and values
 * of every head are decompressed from the latents first: kn [(i+1), nh, dn],
 * vv [(i+1), nh, dv] (scratch).  Writes out [d] given the residual r [d]. */
static void mla_attend(const mla_cfg* m, const double* q, int i, const double* ckv,
                       const double* ckr, const double* r, double* kn, double* vv, double* sc,
                       double* o, double* out) {
  const int qw = m->dn + m->dr, n = i + 1;
  for (int s = 0; s < n; ++s) {
    mla_matvec(m->nh * m->dn, m->dc, m->wuk, ckv + (size_t)s * m->dc, kn + (size_t)s * m->nh * m->dn,
               m->round);
    mla_matvec(m->nh * m->dv, m->dc, m->wuv, ckv + (size_t)s * m->dc, vv + (size_t)s * m->nh * m->dv,
               m->round);
  }
  const double scale = 1.0 / sqrt((double)qw);
  for (int h = 0; h < m->nh; ++h) {
    const double* qh = q + (size_t)h * qw;
    double mx = -INFINITY;
    for (int s = 0; s < n; ++s) {
      double a = 0.0;
      for (int j = 0; j < m->dn; ++j) a += qh[j] * kn[((size_t)s * m->nh + h) * m->dn + j];
      for (int j = 0; j < m->dr; ++j) a += qh[m->dn + j] * ckr[(size_t)s * m->dr + j];
      sc[s] = a * scale;
      if (sc[s] > mx) mx = sc[s];
    }
    double z = 0.0;
    for (int s = 0; s < n; ++s) {
      sc[s] = exp(sc[s] - mx);
      z += sc[s];
    }
    for (int j = 0; j < m->dv; ++j) {
      double a = 0.0;
      for (int s = 0; s < n; ++s) a += sc[s] / z * vv[((size_t)s * m->nh + h) * m->dv + j];
      o[(size_t)h * m->dv + j] = keep_bf16(a, m->round);
    }
  }
  for (int t = 0; t < m->d; ++t) {
    double a = r ? r[t] : 0.0;
    for (int j = 0; j < m->nh * m->dv; ++j) a += m->wo[(size_t)t * m->nh * m->dv + j] * o[j];
    out[t] = keep_bf16(a, m->round);
  }
}

typedef struct {
  const mla_cfg* m;
  int S;
  const double *x, *res;
  const int32_t* pos;  /* decode: position of each sequence's new token */
  double *ckv, *ckr, *out;
} mla_ctx;

static void mla_prefill_seq(void* vctx, int64_t b) {
  const mla_ctx* c = (const mla_ctx*)vctx;
  const mla_cfg* m = c->m;
  const int qw = m->dn + m->dr, S = c->S;
  double* q = (double*)malloc(sizeof(double) * (size_t)S * m->nh * qw);
  double* kn = (double*)malloc(sizeof(double) * (size_t)S * m->nh * m->dn);
  double* vv = (double*)malloc(sizeof(double) * (size_t)S * m->nh * m->dv);
  double* sc = (double*)malloc(sizeof(double) * S);
  double* o = (double*)malloc(sizeof(double) * m->nh * m->dv);
  double* ckv = c->ckv + (size_t)b * m->Lmax * m->dc;
  double* ckr = c->ckr + (size_t)b * m->Lmax * m->dr;
  for (int i = 0; i < S; ++i)
    mla_project(m, c->x + ((size_t)b * S + i) * m->d, i, q + (size_t)i * m->nh * qw,
                ckv + (size_t)i * m->dc, ckr + (size_t)i * m->dr);
  for (int i = 0; i < S; ++i) {
    const size_t row = (size_t)b * S + i;
    mla_attend(m, q + (size_t)i * m->nh * qw, i, ckv, ckr, c->res ? c->res + row * m->d : NULL, kn,
               vv, sc, o, c->out + row * m->d);
  }
  free(q); free(kn); free(vv); free(sc); free(o);
}

static void mla_decode_seq(void* vctx, int64_t b) {
  const mla_ctx* c = (const mla_ctx*)vctx;
  const mla_cfg* m = c->m;
  const int qw = m->dn + m->dr, p = c->pos[b], n = p + 1;
  double* q = (double*)malloc(sizeof(double) * m->nh * qw);
  double* kn = (double*)malloc(sizeof(double) * (size_t)n * m->nh * m->dn);
  double* vv = (double*)malloc(sizeof(double) * (size_t)n * m->nh * m->dv);
  double* sc = (double*)malloc(sizeof(double) * n);
  double* o = (double*)malloc(sizeof(double) * m->nh * m->dv);
  double* ckv = c->ckv + (size_t)b * m->Lmax * m->dc;
  double* ckr = c->ckr + (size_t)b * m->Lmax * m->dr;
  mla_project(m, c->x + (size_t)b * m->d, p, q, ckv + (size_t)p * m->dc, ckr + (size_t)p * m->dr);
  mla_attend(m, q, p, ckv, ckr, c->res ? c->res + (size_t)b * m->d : NULL, kn, vv, sc, o,
             c->out + (size_t)b * m->d);
  free(q); free(kn); free(vv); free(sc); free(o);
}

/* Prefill of B sequences of S tokens (positions 0..S-1): x [B S, d];
 * writes the caches ckv [B, Lmax, dc], ckr [B, Lmax, dr] at positions
 * 0..S-1 and out [B S, d] = res + attention (res may be NULL). */
void oracle_mla_prefill(int B, int S, int Lmax, int d, int nh, int dc, int dn, int dr, int dv,
                        double base, const double* x, const double* wq, const double* wdkv,
                        const double* wkr, const double* wuk, const double* wuv, const double* wo,
                        const double* res, int round_storage, double* ckv, double* ckr,
                        double* out, int nthreads) {
  mla_cfg m = {d, nh, dc, dn, dr, dv, Lmax, round_storage, base, wq, wdkv, wkr, wuk, wuv, wo};
  mla_ctx c = {&m, S, x, res, NULL, ckv, ckr, out};
  parallel_for(B, nthreads, mla_prefill_seq, &c);
}

/* One decoding step: sequence b's new token x [b] sits at position pos[b]
 * (its cache holds positions 0..pos[b]-1); its latent and rotary key are
 * written at pos[b] and it attends to positions 0..pos[b]. */
void oracle_mla_decode(int B, int Lmax, int d, int nh, int dc, int dn, int dr, int dv, double base,
                       const int32_t* pos, const double* x, const double* wq, const double* wdkv,
                       const double* wkr, const double* wuk, const double* wuv, const double* wo,
                       const double* res, int round_storage, double* ckv, double* ckr, double* out,
                       int nthreads) {
  mla_cfg m = {d, nh, dc, dn, dr, dv, Lmax, round_storage, base, wq, wdkv, wkr, wuk, wuv, wo};
  mla_ctx c = {&m, 0, x, res, pos, ckv, ckr, out};
  parallel_for(B, nthreads, mla_decode_seq, &c);
}

/* The rotation of the rotary part, exported for its pins. */
void oracle_mla_rope(double* u, int dr, double pos, double base) { mla_rope(u, dr, pos, base); }
