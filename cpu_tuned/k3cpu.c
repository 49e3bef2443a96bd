/*
 * k3cpu.c — tuned CPU implementation of the routed-expert MoE layer for bf16 tokens
 * (router GEMV, softmax, top-k, SwiGLU experts on MXFP4 weights, slot-ordered combine),
 * the realistic CPU comparator of the GPU path.
 *
 * It computes what the layer is defined to compute, in fp64, with every sum in the
 * order of the plain definition: each router logit sums x_k W[k][e] for k in order and
 * then adds the bias; each expert row sums (e2m1(code_k) 2^(s_b - 127)) x_k for k in
 * order; the combine adds gate * E(x) slot by slot. Products are formed, rounded and
 * then added (no fused multiply-add), so its results equal the plain fp64 definition
 * bit for bit. What makes it fast is how the same operations are scheduled, not a
 * different order:
 *  - vectors run across independent outputs (four router logits, four expert rows per
 *    AVX2 register), never along a sum;
 *  - MXFP4 codes are decoded through a 16-entry table times the block's power of two
 *    (exact), a block of 32 codes of four rows at a time;
 *  - OpenMP spreads independent outputs over the cores.
 * The pages' own engine keeps a scalar path and an AVX2 path that reproduce each other
 * bit for bit ("kimi-k3-in-c 路线图深读", yfxerp.com, roadmap item 4: the MXFP4 expert
 * matmul's AVX2 path mirrors the scalar reduction order with double accumulators); this
 * file follows that rule against the plain definition. Without AVX2 and FMA on the host,
 * the same loops run scalar.
 */
#include "k3cpu.h"

#include <immintrin.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static double g_e2m1[16];
static double g_e8m0[256];
static int g_ready = 0;

static void tables(void) {
  if (g_ready) return;
  /* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa */
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  for (int c = 0; c < 16; ++c) g_e2m1[c] = (c & 8) ? -mag[c & 7] : mag[c & 7];
  for (int s = 0; s < 256; ++s) g_e8m0[s] = (s == 255) ? NAN : ldexp(1.0, s - 127);
  g_ready = 1;
}

static inline double bf16d(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---- one MXFP4 row against x, k in order (scalar) --------------------------------- */
static double mx_dot1(const uint8_t* q, const uint8_t* s, int32_t K, const double* x) {
  double acc = 0.0;
  for (int32_t b = 0; b < K / 32; ++b) {
    const double sc = g_e8m0[s[b]];
    for (int j = 0; j < 16; ++j) {
      const uint8_t by = q[16 * b + j];
      const double w0 = g_e2m1[by & 15u] * sc, w1 = g_e2m1[by >> 4] * sc;
      const double p0 = w0 * x[32 * b + 2 * j];
      acc = acc + p0;
      const double p1 = w1 * x[32 * b + 2 * j + 1];
      acc = acc + p1;
    }
  }
  return acc;
}

/* ---- four rows (stride rq bytes, rs scale bytes) against x, one AVX2 lane each ---- */
__attribute__((target("avx2"))) static void mx_dot4(const uint8_t* q, const uint8_t* s,
                                                    int64_t rq, int64_t rs, int32_t K,
                                                    const double* x, double* out) {
  double wt[32][4] __attribute__((aligned(32)));
  __m256d acc = _mm256_setzero_pd();
  for (int32_t b = 0; b < K / 32; ++b) {
    for (int r = 0; r < 4; ++r) {
      const uint8_t* qr = q + r * rq + 16 * b;
      const double sc = g_e8m0[s[r * rs + b]];
      for (int j = 0; j < 16; ++j) {
        const uint8_t by = qr[j];
        wt[2 * j][r] = g_e2m1[by & 15u] * sc;
        wt[2 * j + 1][r] = g_e2m1[by >> 4] * sc;
      }
    }
    const double* xb = x + 32 * b;
    for (int kk = 0; kk < 32; ++kk) {
      const __m256d p = _mm256_mul_pd(_mm256_load_pd(wt[kk]), _mm256_set1_pd(xb[kk]));
      acc = _mm256_add_pd(acc, p);
    }
  }
  _mm256_storeu_pd(out, acc);
}

static int have_avx2(void) {
  static int v = -1;
  if (v < 0) v = __builtin_cpu_supports("avx2") ? 1 : 0;
  return v;
}

/* rows [0, n) of a stacked MXFP4 matrix against x into out */
static void mx_rows(const uint8_t* q, const uint8_t* s, int32_t n, int32_t K, const double* x,
                    double* out) {
  const int64_t rq = K / 2, rs = K / 32;
  const int avx = have_avx2();
  const int32_t ng = avx ? n / 4 : 0;
#pragma omp parallel for schedule(static)
  for (int32_t g = 0; g < ng; ++g) mx_dot4(q + 4 * g * rq, s + 4 * g * rs, rq, rs, K, x, out + 4 * g);
#pragma omp parallel for schedule(static)
  for (int32_t r = 4 * ng; r < n; ++r) out[r] = mx_dot1(q + r * rq, s + r * rs, K, x);
}

/* ---- router logits: l[e] = sum_k x_k W[k][e] (k in order), then + bias -------------- */
__attribute__((target("avx2"))) static void router4(const double* x, const uint16_t* w,
                                                    int32_t d, int32_t E, int32_t e0,
                                                    double* l) {
  __m256d acc = _mm256_setzero_pd();
  for (int32_t k = 0; k < d; ++k) {
    const __m128i h = _mm_loadl_epi64((const __m128i*)(w + (int64_t)k * E + e0));
    const __m128 wf = _mm_castsi128_ps(_mm_slli_epi32(_mm_cvtepu16_epi32(h), 16));
    const __m256d p = _mm256_mul_pd(_mm256_set1_pd(x[k]), _mm256_cvtps_pd(wf));
    acc = _mm256_add_pd(acc, p);
  }
  _mm256_storeu_pd(l + e0, acc);
}

static void router_logits(const double* x, const uint16_t* w, const float* bias, int32_t d,
                          int32_t E, double* l) {
  const int avx = have_avx2();
  const int32_t ng = avx ? E / 4 : 0;
#pragma omp parallel for schedule(static)
  for (int32_t g = 0; g < ng; ++g) router4(x, w, d, E, 4 * g, l);
#pragma omp parallel for schedule(static)
  for (int32_t e = 4 * ng; e < E; ++e) {
    double acc = 0.0;
    for (int32_t k = 0; k < d; ++k) {
      const double p = x[k] * bf16d(w[(int64_t)k * E + e]);
      acc = acc + p;
    }
    l[e] = acc;
  }
  if (bias)
    for (int32_t e = 0; e < E; ++e) l[e] = l[e] + (double)bias[e];
}

/* softmax over all experts (max-subtracted) and top-k: larger logit first, equal logits
 * -> lower id, NaN last; gates are the full-softmax probabilities of the chosen ids */
static int ranks_before(double la, int32_t a, double lb, int32_t b) {
  const int na = isnan(la), nb = isnan(lb);
  if (na != nb) return nb;
  if (!na && la != lb) return la > lb;
  return a < b;
}

static void route(const double* l, int32_t E, int32_t k, int32_t* ids, double* gates,
                  double* p, unsigned char* taken) {
  double m = l[0];
  for (int32_t e = 1; e < E; ++e)
    if (l[e] > m) m = l[e];
  double s = 0.0;
  for (int32_t e = 0; e < E; ++e) {
    p[e] = exp(l[e] - m);
    s += p[e];
  }
  for (int32_t e = 0; e < E; ++e) p[e] = p[e] / s;
  memset(taken, 0, (size_t)E);
  for (int32_t r = 0; r < k; ++r) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
    }
    ids[r] = best;
    taken[best] = 1;
    gates[r] = p[best];
  }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

int k3cpu_layer_forward(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                        const uint16_t* x, const uint16_t* w_router, const float* bias,
                        const k3cpu_expert* experts, double* y, int32_t* ids, double* gates) {
  if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k < 1 || k > E || d % 32 || f % 32) return -1;
  tables();
  double* xd = (double*)malloc((size_t)d * sizeof(double));
  double* l = (double*)malloc((size_t)E * sizeof(double));
  double* p = (double*)malloc((size_t)E * sizeof(double));
  double* u = (double*)malloc((size_t)f * sizeof(double));
  double* v = (double*)malloc((size_t)f * sizeof(double));
  double* z = (double*)malloc((size_t)d * sizeof(double));
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  int rc = (xd && l && p && u && v && z && taken) ? 0 : -2;
  for (int32_t t = 0; t < T && rc == 0; ++t) {
    for (int32_t i = 0; i < d; ++i) xd[i] = bf16d(x[(int64_t)t * d + i]);
    router_logits(xd, w_router, bias, d, E, l);
    int32_t* it = ids + (int64_t)t * k;
    double* gt = gates + (int64_t)t * k;
    route(l, E, k, it, gt, p, taken);
    double* yt = y + (int64_t)t * d;
    for (int32_t i = 0; i < d; ++i) yt[i] = 0.0;
    for (int32_t r = 0; r < k; ++r) {
      const k3cpu_expert* ex = experts + it[r];
      if (!ex->gate_q || !ex->gate_s || !ex->up_q || !ex->up_s || !ex->down_q || !ex->down_s) {
        rc = -1;
        break;
      }
      mx_rows(ex->gate_q, ex->gate_s, f, d, xd, u);
      mx_rows(ex->up_q, ex->up_s, f, d, xd, v);
      for (int32_t j = 0; j < f; ++j) u[j] = silu(u[j]) * v[j];
      mx_rows(ex->down_q, ex->down_s, d, f, u, z);
      const double g = gt[r];
      for (int32_t i = 0; i < d; ++i) {
        const double q = g * z[i];
        yt[i] = yt[i] + q;
      }
    }
  }
  free(xd); free(l); free(p); free(u); free(v); free(z); free(taken);
  return rc;
}

int k3cpu_layer_route(int32_t T, int32_t d, int32_t E, int32_t k, const uint16_t* x,
                      const uint16_t* w_router, const float* bias, int32_t* ids,
                      double* gates) {
  if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E) return -1;
  tables();
  double* xd = (double*)malloc((size_t)d * sizeof(double));
  double* l = (double*)malloc((size_t)E * sizeof(double));
  double* p = (double*)malloc((size_t)E * sizeof(double));
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  const int rc = (xd && l && p && taken) ? 0 : -2;
  for (int32_t t = 0; t < T && rc == 0; ++t) {
    for (int32_t i = 0; i < d; ++i) xd[i] = bf16d(x[(int64_t)t * d + i]);
    router_logits(xd, w_router, bias, d, E, l);
    route(l, E, k, ids + (int64_t)t * k, gates + (int64_t)t * k, p, taken);
  }
  free(xd); free(l); free(p); free(taken);
  return rc;
}

int k3cpu_simd(void) { return have_avx2(); }
