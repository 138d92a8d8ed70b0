/*
 * oracle.c -- plain CPU definition of the decode-step MoE block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library.
 *
 * Sources (web pages on the Kimi K3 specialised decode path):
 *   [WRITEUP] "vLLM 如何用智能体辅助优化 Kimi K3 解码性能" -- Chinese
 *             translation of the vLLM write-up.  Part 1 §1 (tuning shapes to
 *             the workload), Part 1 §2 (overlapping computation and
 *             communication: the attention output projection fused with its
 *             all-reduce and the residual), Part 1 §3 (MoE scheduling: router scores, routed
 *             experts, shared expert), Part 2 §3 (correctness).
 *   [AREX]    "vLLM 宣布 Kimi K3 在 GB300 NVL72 上实现 batch 1 解码 842
 *             tokens/s" -- section "每层从 23 个内核减到 13 个" (MoE schedule).
 *   [AICODER] "2.8 万亿参数 Kimi K3 单请求飙至 842 tok/s！..." -- section
 *             "架构亮点与底层机制" (MoE gating and expert GEMM).
 * The pages name the stages (router scoring, top-k routed experts, a shared
 * expert that runs for every token, expert GEMMs) but print no formula; the
 * arithmetic below is the standard definition of each stage, with the
 * readings taken where the pages are silent:
 *   - router: logits = x . Wr^T + bias; select the k largest logits (ties:
 *     lower expert index first); weights = softmax over the selected logits
 *     (equal to a softmax over all E renormalised over the top-k); no scale.
 *   - the selection decision is taken on logits rounded to fp32, the
 *     precision the GPU kernel accumulates them in; everything else is fp64.
 *   - expert: h = silu(x . Wg^T) * (x . Wu^T), y = h . W2^T, with the gate
 *     rows first and the up rows second in the fused [2I][d] matrix, and
 *     silu(z) = z / (1 + exp(-z)).
 *   - shared expert: the same FFN with its own weights, weight 1, every token.
 *   - combine: out[t] = sum_j w[t][j] * y[t][j] (ascending expert id)
 *     + y_shared[t].
 *   - dense skinny GEMM: Y[b][n] = sum_c X[b][c] * W[n][c].
 *   - attention output projection with residual (Part 1 §2, without its
 *     all-reduce): Y[b][n] = sum_c X[b][c] * W[n][c] + R[b][n].
 *
 * Everything is computed token by token and slot by slot -- never grouped by
 * expert -- in fp64, with bf16 inputs widened exactly.  Inputs must be finite.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DT_F32 0
#define ORACLE_DT_BF16 1

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double widen_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Element i of an array of dtype dt, widened to double. */
static double elem(const void *p, int dt, size_t i) {
  if (dt == ORACLE_DT_F32) return (double)((const float *)p)[i];
  return widen_bf16(((const uint16_t *)p)[i]);
}

/* sum_{c<n} a[a0+c] * b[b0+c], ascending c, in fp64. */
static double dot(const void *a, size_t a0, const void *b, size_t b0,
                  int dt, int n) {
  double s = 0.0;
  for (int c = 0; c < n; ++c) s += elem(a, dt, a0 + c) * elem(b, dt, b0 + c);
  return s;
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Dense skinny GEMM: Y[b][n] = sum_c X[b][c] W[n][c]; X [B][K], W [N][K]. */
void oracle_skinny_gemm(int dt, int B, int N, int K, const void *X,
                        const void *W, double *Y) {
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n)
      Y[(size_t)b * N + n] =
          dot(X, (size_t)b * K, W, (size_t)n * K, dt, K);
}

/* Attention output projection with the residual added ([WRITEUP] part 1
 * §2: the output projection fused with its all-reduce and the following
 * residual; on one GPU the all-reduce is absent):
 * Y[b][n] = sum_c X[b][c] W[n][c] + R[b][n]; X [B][K], W [N][K], R [B][N]. */
void oracle_skinny_gemm_residual(int dt, int B, int N, int K, const void *X,
                                 const void *W, const void *R, double *Y) {
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n)
      Y[(size_t)b * N + n] =
          dot(X, (size_t)b * K, W, (size_t)n * K, dt, K) +
          elem(R, dt, (size_t)b * N + n);
}

/* Router logits: l[t][e] = sum_c x[t][c] Wr[e][c] + bias(t, e).
 * bias may be NULL; bias_ld = 0 broadcasts one row [E] to every token,
 * bias_ld = E gives one row per token. */
void oracle_router_logits(int dt, int B, int d, int E, const void *X,
                          const void *Wr, const float *bias, int bias_ld,
                          double *logits) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < B; ++t)
    for (int e = 0; e < E; ++e) {
      double l = dot(X, (size_t)t * d, Wr, (size_t)e * d, dt, d);
      if (bias) l += (double)bias[(size_t)t * bias_ld + e];
      logits[(size_t)t * E + e] = l;
    }
}

/* Latent input projection ([WRITEUP] part 1 §3: the router scores and the
 * latent input projection both take the token's hidden state x, and the
 * specialised path computes them as one matrix product):
 * latent[t][j] = sum_c X[t][c] Wl[j][c]; X [B][d], Wl [L][d]. */
void oracle_latent_projection(int dt, int B, int d, int L, const void *X,
                              const void *Wl, double *latent) {
  for (int t = 0; t < B; ++t)
    for (int j = 0; j < L; ++j)
      latent[(size_t)t * L + j] = dot(X, (size_t)t * d, Wl, (size_t)j * d, dt, d);
}

/* Top-k of one token's logits.  The k winners are taken one at a time: each
 * round picks the largest remaining fp32-rounded logit, and on an exact tie
 * the lower expert index.  They are returned in ascending expert id, with
 * weights w_j = exp(l_j - m) / sum_i exp(l_i - m), m the largest selected
 * logit, computed from the same fp32-rounded logits. */
void oracle_topk(int E, int k, const double *logits, int32_t *ids,
                 double *w) {
  unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
  for (int r = 0; r < k; ++r) {
    int best = -1;
    float bv = 0.0f;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      float v = (float)logits[e];
      if (best < 0 || v > bv) { best = e; bv = v; }
    }
    taken[best] = 1;
  }
  int n = 0;
  for (int e = 0; e < E; ++e)
    if (taken[e]) ids[n++] = e;
  free(taken);

  double m = -INFINITY;
  for (int j = 0; j < k; ++j) {
    double v = (double)(float)logits[ids[j]];
    if (v > m) m = v;
  }
  double z = 0.0;
  for (int j = 0; j < k; ++j) z += exp((double)(float)logits[ids[j]] - m);
  for (int j = 0; j < k; ++j)
    w[j] = exp((double)(float)logits[ids[j]] - m) / z;
}

/* Words in a routing plan for B tokens, top-k of E experts. */
int oracle_plan_words(int B, int k, int E) {
  int maxa = B * k < E ? B * k : E;
  return 2 + 2 * maxa + B * k;
}

/* Routing plan from ids [B][k]:
 *   plan[0]                      number of distinct experts chosen, n
 *   plan[1 .. 1+maxa)            those experts, ascending (unused: -1)
 *   plan[1+maxa .. 2+2*maxa)     offsets into the slot list, n+1 used
 *                                (unused: B*k)
 *   plan[2+2*maxa .. +B*k)       slots s = t*k + j ordered by expert, then
 *                                by token
 * with maxa = min(E, B*k).  Built by a plain scan over experts and slots. */
void oracle_plan(int B, int k, int E, const int32_t *ids, int32_t *plan) {
  int maxa = B * k < E ? B * k : E;
  int32_t *active = plan + 1;
  int32_t *offs = plan + 1 + maxa;
  int32_t *slots = plan + 2 + 2 * maxa;
  for (int a = 0; a < maxa; ++a) active[a] = -1;
  for (int a = 0; a <= maxa; ++a) offs[a] = B * k;
  int n = 0, pos = 0;
  for (int e = 0; e < E; ++e) {
    int first = 1;
    for (int s = 0; s < B * k; ++s) {
      if (ids[s] != e) continue;
      if (first) { active[n] = e; offs[n] = pos; ++n; first = 0; }
      slots[pos++] = s;
    }
  }
  offs[n] = pos;
  plan[0] = n;
}

/* Router stage: logits, ids, weights and plan for all B tokens. */
void oracle_route(int dt, int B, int d, int E, int k, const void *X,
                  const void *Wr, const float *bias, int bias_ld,
                  double *logits, int32_t *ids, double *w, int32_t *plan) {
  oracle_router_logits(dt, B, d, E, X, Wr, bias, bias_ld, logits);
  for (int t = 0; t < B; ++t)
    oracle_topk(E, k, logits + (size_t)t * E, ids + (size_t)t * k,
                w + (size_t)t * k);
  if (plan) oracle_plan(B, k, E, ids, plan);
}

/* One expert FFN on one token.  x_row [d]; W13 [2I][d] (gate rows 0..I-1,
 * up rows I..2I-1); W2 [d][I].  Writes y [d] and, if h is not NULL, the
 * intermediate h [I]. */
void oracle_expert(int dt, int d, int I, const void *X, size_t x_off,
                   const void *W13, const void *W2, double *y, double *h) {
  double *hh = (double *)malloc(sizeof(double) * (size_t)I);
  for (int i = 0; i < I; ++i) {
    double g = dot(X, x_off, W13, (size_t)i * d, dt, d);
    double u = dot(X, x_off, W13, (size_t)(I + i) * d, dt, d);
    hh[i] = oracle_silu(g) * u;
  }
  for (int r = 0; r < d; ++r) {
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += hh[i] * elem(W2, dt, (size_t)r * I + i);
    y[r] = s;
  }
  if (h) memcpy(h, hh, sizeof(double) * (size_t)I);
  free(hh);
}

/* Token t of the block: its k routed experts, each weighted, then the shared
 * expert with weight 1, summed in that order into out[t]; the per-slot
 * outputs to yslot[t] if not NULL.  Returns -1 if a selected expert has no
 * weights. */
static int block_token(int dt, int t, int d, int k, int I, int Is,
                       const void *X, const int32_t *id, const double *ww,
                       const void *const *W13e, const void *const *W2e,
                       const void *Ws13, const void *Ws2, double *yslot,
                       double *out) {
  double *y = (double *)malloc(sizeof(double) * (size_t)d);
  double *o = out + (size_t)t * d;
  int rc = 0;
  for (int r = 0; r < d; ++r) o[r] = 0.0;
  for (int j = 0; j < k && rc == 0; ++j) {
    int e = id[(size_t)t * k + j];
    if (!W13e[e] || !W2e[e]) { rc = -1; break; }
    oracle_expert(dt, d, I, X, (size_t)t * d, W13e[e], W2e[e], y, NULL);
    for (int r = 0; r < d; ++r) o[r] += ww[(size_t)t * k + j] * y[r];
    if (yslot)
      memcpy(yslot + ((size_t)t * (k + 1) + j) * d, y, sizeof(double) * d);
  }
  if (rc == 0) {
    if (Ws13) {
      oracle_expert(dt, d, Is, X, (size_t)t * d, Ws13, Ws2, y, NULL);
      for (int r = 0; r < d; ++r) o[r] += y[r];
    } else {
      for (int r = 0; r < d; ++r) y[r] = 0.0;
    }
    if (yslot)
      memcpy(yslot + ((size_t)t * (k + 1) + k) * d, y, sizeof(double) * d);
  }
  free(y);
  return rc;
}

/* Whole block.  W13e / W2e are arrays of E pointers, one per expert
 * ([2I][d] and [d][I]); an expert no token selects may be NULL.  Ws13
 * [2Is][d] and Ws2 [d][Is] are the shared expert (Ws13 NULL: none).
 * Outputs (any may be NULL except out): logits [B][E], ids [B][k],
 * w [B][k], plan, yslot [B][k+1][d] (slot k is the shared expert, zero if
 * none), out [B][d].  Returns 0, or -1 if a selected expert has no weights.
 * Tokens are independent; built with OpenMP (the all-cores timing build)
 * they run in parallel, each with the same arithmetic. */
int oracle_moe_block(int dt, int B, int d, int E, int k, int I, int Is,
                     const void *X, const void *Wr, const float *bias,
                     int bias_ld, const void *const *W13e,
                     const void *const *W2e, const void *Ws13,
                     const void *Ws2, double *logits, int32_t *ids,
                     double *w, int32_t *plan, double *yslot, double *out) {
  double *lg = logits ? logits : (double *)malloc(sizeof(double) * (size_t)B * E);
  int32_t *id = ids ? ids : (int32_t *)malloc(sizeof(int32_t) * (size_t)B * k);
  double *ww = w ? w : (double *)malloc(sizeof(double) * (size_t)B * k);
  int rc = 0;
  oracle_route(dt, B, d, E, k, X, Wr, bias, bias_ld, lg, id, ww, plan);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
  for (int t = 0; t < B; ++t)
    rc |= block_token(dt, t, d, k, I, Is, X, id, ww, W13e, W2e, Ws13, Ws2,
                      yslot, out);
  if (!logits) free(lg);
  if (!ids) free(id);
  if (!w) free(ww);
  return rc ? -1 : 0;
}

/* Threads the block runs its tokens on: 1 in the plain build. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Weighted combine on given per-slot outputs (for checking the combine stage
 * alone): out[t] = sum_j w[t][j] yslot[t][j] + (has_shared ? yslot[t][k] : 0).
 * yslot [B][k+1][d] and w [B][k] are fp32 as the GPU stage consumes them. */
void oracle_combine(int B, int d, int k, const float *yslot, const float *w,
                    int has_shared, double *out) {
  for (int t = 0; t < B; ++t)
    for (int r = 0; r < d; ++r) {
      double s = 0.0;
      for (int j = 0; j < k; ++j)
        s += (double)w[(size_t)t * k + j] *
             (double)yslot[((size_t)t * (k + 1) + j) * d + r];
      if (has_shared) s += (double)yslot[((size_t)t * (k + 1) + k) * d + r];
      out[(size_t)t * d + r] = s;
    }
}
