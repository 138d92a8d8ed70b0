/* Harness of the CPU oracle for the sanitizer build (ASan + UBSan): every
 * oracle function on small seeded inputs, including the degenerate cases
 * (k = E, top-1, no shared expert, an unselected expert missing, fp32 and
 * bf16 storage).  Test infrastructure: links oracle.c directly.  Exits 0
 * when the weights of every token sum to 1 and the calls returned what
 * their contracts state. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_skinny_gemm(int, int, int, int, const void *, const void *, double *);
void oracle_skinny_gemm_residual(int, int, int, int, const void *, const void *, const void *, double *);
void oracle_router_logits(int, int, int, int, const void *, const void *, const float *, int, double *);
void oracle_topk(int, int, const double *, int32_t *, double *);
int oracle_plan_words(int, int, int);
void oracle_plan(int, int, int, const int32_t *, int32_t *);
int oracle_moe_block(int, int, int, int, int, int, int, const void *, const void *, const float *, int,
                     const void *const *, const void *const *, const void *, const void *, double *, int32_t *,
                     double *, int32_t *, double *, double *);
void oracle_combine(int, int, int, const float *, const float *, int, double *);

static uint32_t g_state = 12345u;
static float rnd(void) { /* xorshift, uniform in [-1, 1) */
  g_state ^= g_state << 13; g_state ^= g_state >> 17; g_state ^= g_state << 5;
  return (float)((double)g_state / 2147483648.0 - 1.0);
}
static void *arr(int bf16, size_t n) {
  if (!bf16) { float *p = malloc(n * 4); for (size_t i = 0; i < n; ++i) p[i] = rnd(); return p; }
  uint16_t *p = malloc(n * 2);
  for (size_t i = 0; i < n; ++i) { float f = rnd(); uint32_t u; memcpy(&u, &f, 4); p[i] = (uint16_t)(u >> 16); }
  return p;
}

static int run(int bf16, int B, int d, int E, int k, int I, int Is, int bias_ld, int drop_unselected) {
  int bad = 0;
  void *X = arr(bf16, (size_t)B * d), *Wr = arr(bf16, (size_t)E * d);
  float *bias = bias_ld >= 0 ? arr(0, (size_t)(bias_ld ? B : 1) * E) : NULL;
  void **W13 = calloc(E, sizeof(void *)), **W2 = calloc(E, sizeof(void *));
  for (int e = 0; e < E; ++e) { W13[e] = arr(bf16, (size_t)2 * I * d); W2[e] = arr(bf16, (size_t)d * I); }
  void *Ws13 = Is ? arr(bf16, (size_t)2 * Is * d) : NULL, *Ws2 = Is ? arr(bf16, (size_t)d * Is) : NULL;
  double *lg = malloc(sizeof(double) * B * E), *w = malloc(sizeof(double) * B * k);
  int32_t *ids = malloc(4 * B * k), *plan = malloc(4 * oracle_plan_words(B, k, E));
  double *ys = malloc(sizeof(double) * B * (k + 1) * d), *out = malloc(sizeof(double) * B * d);
  int rc = oracle_moe_block(bf16, B, d, E, k, I, Is, X, Wr, bias, bias_ld < 0 ? 0 : bias_ld,
                            (const void *const *)W13, (const void *const *)W2, Ws13, Ws2, lg, ids, w, plan, ys, out);
  if (rc != 0) bad++;
  for (int t = 0; t < B; ++t) {
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += w[t * k + j];
    if (fabs(s - 1.0) > 1e-12) bad++;
  }
  if (plan[0] < 1 || plan[0] > (B * k < E ? B * k : E)) bad++;
  if (drop_unselected) {   /* drop a selected expert: the block must report it */
    int e = ids[0];
    free(W13[e]); W13[e] = NULL;
    rc = oracle_moe_block(bf16, B, d, E, k, I, Is, X, Wr, bias, bias_ld < 0 ? 0 : bias_ld,
                          (const void *const *)W13, (const void *const *)W2, Ws13, Ws2, NULL, NULL, NULL, NULL, NULL,
                          out);
    if (rc != -1) bad++;
  }
  double *Y = malloc(sizeof(double) * B * E);
  oracle_skinny_gemm(bf16, B, E, d, X, Wr, Y);
  void *R = arr(bf16, (size_t)B * E);
  oracle_skinny_gemm_residual(bf16, B, E, d, X, Wr, R, Y);
  float *ysf = arr(0, (size_t)B * (k + 1) * d), *wf = arr(0, (size_t)B * k);
  oracle_combine(B, d, k, ysf, wf, Is > 0, out);
  free(Y); free(R); free(ysf); free(wf);
  for (int e = 0; e < E; ++e) { free(W13[e]); free(W2[e]); }
  free(W13); free(W2); free(Ws13); free(Ws2); free(X); free(Wr); free(bias);
  free(lg); free(w); free(ids); free(plan); free(ys); free(out);
  return bad;
}

int main(void) {
  int bad = 0;
  bad += run(0, 1, 64, 16, 2, 32, 0, -1, 1);     /* fp32, no shared expert, no bias */
  bad += run(1, 5, 96, 8, 8, 16, 16, 0, 0);      /* k = E, broadcast bias */
  bad += run(1, 9, 128, 40, 1, 32, 48, 40, 1);   /* top-1, per-token bias, wider shared */
  bad += run(1, 17, 64, 64, 16, 8, 8, -1, 0);    /* top-16, more slots than experts */
  printf("oracle harness: %d failures\n", bad);
  return bad ? 1 : 0;
}
