/* Host-only driver of the fp64 oracle (oracle/k3oracle.c), built by
 * tests/test_host_sanitize.py with AddressSanitizer and UndefinedBehaviorSanitizer: small
 * layers of several shapes (ragged widths, k = E, one expert, block mode, an E8M0 255 scale)
 * through every exported routine, checking the invariants of the results as it goes. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "k3oracle.h"

static uint32_t rng_state = 2463534242u;
static uint32_t rnd(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return rng_state;
}
static uint16_t bf16_of(float v) { /* truncation is enough for test inputs */
  uint32_t u;
  memcpy(&u, &v, 4);
  return (uint16_t)(u >> 16);
}
static float unif(void) { return (float)(rnd() & 0xFFFFFF) / 16777216.0f - 0.5f; }

static int fails = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static uint8_t* bytes(size_t n) {
  uint8_t* p = (uint8_t*)malloc(n ? n : 1);
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd();
  return p;
}
static uint8_t* scales(size_t n) {
  uint8_t* p = (uint8_t*)malloc(n ? n : 1);
  for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)(120 + rnd() % 9);
  return p;
}
static uint16_t* bf16s(size_t n, float sd) {
  uint16_t* p = (uint16_t*)malloc((n ? n : 1) * 2);
  for (size_t i = 0; i < n; ++i) p[i] = bf16_of(sd * unif());
  return p;
}

static void run_shape(int T, int d, int f, int E, int k, int block, int nan_scale) {
  k3o_expert* ex = (k3o_expert*)calloc((size_t)E, sizeof(k3o_expert));
  uint8_t** owned = (uint8_t**)calloc((size_t)E * 6, sizeof(uint8_t*));
  for (int e = 0; e < E; ++e) {
    owned[6 * e + 0] = bytes((size_t)f * d / 2);
    owned[6 * e + 1] = scales((size_t)f * d / 32);
    owned[6 * e + 2] = bytes((size_t)f * d / 2);
    owned[6 * e + 3] = scales((size_t)f * d / 32);
    owned[6 * e + 4] = bytes((size_t)d * f / 2);
    owned[6 * e + 5] = scales((size_t)d * f / 32);
    ex[e].gate_q = owned[6 * e + 0];
    ex[e].gate_s = owned[6 * e + 1];
    ex[e].up_q = owned[6 * e + 2];
    ex[e].up_s = owned[6 * e + 3];
    ex[e].down_q = owned[6 * e + 4];
    ex[e].down_s = owned[6 * e + 5];
  }
  if (nan_scale) owned[5][0] = 255; /* expert 0, down row 0, block 0 */
  uint16_t* wr = bf16s((size_t)d * E, 0.1f);
  float* bias = (float*)malloc((size_t)E * 4);
  for (int e = 0; e < E; ++e) bias[e] = unif();
  uint16_t* gamma = bf16s((size_t)d, 2.0f);
  uint16_t* sg = bf16s((size_t)f * d, 1.0f);
  uint16_t* su = bf16s((size_t)f * d, 1.0f);
  uint16_t* sd = bf16s((size_t)d * f, 1.0f);
  k3o_block blk = {gamma, 1e-6, sg, su, sd};
  float* xf = (float*)malloc((size_t)T * d * 4 + 4);
  for (int i = 0; i < T * d; ++i) xf[i] = 4.0f * unif();
  uint16_t* xb = bf16s((size_t)T * d, 4.0f);
  const void* x = block ? (const void*)xf : (const void*)xb;
  const int dt = block ? K3O_F32 : K3O_BF16;

  int32_t* ids = (int32_t*)malloc((size_t)T * k * 4 + 4);
  double* gates = (double*)malloc((size_t)T * k * 8 + 8);
  double* logits = (double*)malloc((size_t)T * E * 8 + 8);
  double* xin = (double*)malloc((size_t)T * d * 8 + 8);
  double* y = (double*)malloc((size_t)T * d * 8 + 8);
  int32_t* ids2 = (int32_t*)malloc((size_t)T * k * 4 + 4);
  double* gates2 = (double*)malloc((size_t)T * k * 8 + 8);

  CHECK(k3o_layer_route(T, d, E, k, x, dt, wr, bias, block ? &blk : NULL, ids, gates, logits,
                        xin) == 0);
  for (int t = 0; t < T; ++t) {
    double gs = 0.0;
    for (int s = 0; s < k; ++s) {
      const int e = ids[t * k + s];
      CHECK(e >= 0 && e < E);
      for (int s2 = 0; s2 < s; ++s2) CHECK(ids[t * k + s2] != e);
      if (s > 0) CHECK(logits[t * E + ids[t * k + s - 1]] >= logits[t * E + e]);
      CHECK(gates[t * k + s] > 0.0 && gates[t * k + s] <= 1.0);
      gs += gates[t * k + s];
    }
    CHECK(gs <= 1.0 + 1e-12);
  }
  int32_t* offs = (int32_t*)malloc((size_t)(E + 1) * 4);
  int32_t* rows = (int32_t*)malloc((size_t)T * k * 4 + 4);
  CHECK(k3o_bucket(T, E, k, ids, offs, rows) == 0);
  CHECK(offs[0] == 0 && offs[E] == T * k);
  for (int e = 0; e < E; ++e) CHECK(offs[e] <= offs[e + 1]);
  for (int e = 0; e < E; ++e)
    for (int p = offs[e]; p < offs[e + 1]; ++p) {
      CHECK(rows[p] >= 0 && rows[p] < T * k);
      CHECK(ids[rows[p]] == e);
      if (p > offs[e]) CHECK(rows[p - 1] < rows[p]);
    }
  CHECK(k3o_layer_forward(T, d, f, E, k, x, dt, wr, bias, ex, block ? &blk : NULL, y, ids2,
                          gates2) == 0);
  CHECK(memcmp(ids, ids2, (size_t)T * k * 4) == 0);
  for (int t = 0; t < T; ++t) {
    int picked0 = 0;
    for (int s = 0; s < k; ++s) picked0 |= ids[t * k + s] == 0;
    for (int i = 0; i < d; ++i) {
      const double v = y[(size_t)t * d + i];
      if (nan_scale && picked0 && i == 0) CHECK(isnan(v));
      else CHECK(isfinite(v));
    }
  }
  /* the single-expert routines on one decoded token */
  double* h = (double*)malloc((size_t)f * 8);
  double* out = (double*)malloc((size_t)d * 8);
  double* w = (double*)malloc((size_t)d * 8);
  k3o_expert_ffn(d, f, xin, &ex[E - 1], h, out);
  k3o_mx_row(ex[0].gate_q, ex[0].gate_s, d, w);
  const double a = k3o_mx_dot(ex[0].gate_q, ex[0].gate_s, d, xin);
  const double b = k3o_mx_dot_blockscaled(ex[0].gate_q, ex[0].gate_s, d, xin);
  CHECK(isfinite(a) && isfinite(b));
  k3o_rmsnorm(d, xin, gamma, 1e-6, out);
  k3o_dense_swiglu(d, f, xin, sg, su, sd, out);
  for (int i = 0; i < d; ++i) CHECK(isfinite(out[i]));
  double* p = (double*)malloc((size_t)E * 8);
  k3o_softmax(E, logits, p);
  double ps = 0.0;
  for (int e = 0; e < E; ++e) ps += p[e];
  CHECK(fabs(ps - 1.0) < 1e-12);

  free(h); free(out); free(w); free(p);
  free(offs); free(rows);
  free(ids); free(gates); free(logits); free(xin); free(y); free(ids2); free(gates2);
  free(xf); free(xb); free(wr); free(bias); free(gamma); free(sg); free(su); free(sd);
  for (int i = 0; i < E * 6; ++i) free(owned[i]);
  free(owned);
  free(ex);
}

int main(void) {
  for (uint32_t c = 0; c < 16; ++c) CHECK(k3o_e2m1(c) == -k3o_e2m1(c ^ 8u) || c == 0 || c == 8);
  CHECK(isnan(k3o_e8m0(255)));
  run_shape(3, 64, 32, 8, 2, 0, 0);    /* the tiny layer */
  run_shape(5, 96, 64, 13, 3, 0, 0);   /* three blocks per row, ragged E */
  run_shape(2, 160, 96, 5, 5, 0, 0);   /* k = E */
  run_shape(4, 64, 32, 1, 1, 0, 0);    /* one expert */
  run_shape(2, 64, 32, 8, 2, 1, 0);    /* block mode, fp32 residual */
  run_shape(3, 64, 32, 4, 4, 0, 1);    /* E8M0 255 in one down row of expert 0 */
  run_shape(1, 512, 256, 32, 4, 0, 0); /* the toy layer's shape */
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
