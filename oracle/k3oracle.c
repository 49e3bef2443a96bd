/*
 * k3oracle.c — plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY; see
 * k3oracle.h for who may load it and for the source key [A]/[B]/[C]).
 *
 * Readings taken where the pages leave a step open:
 *  - E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; no inf/NaN.
 *  - E8M0: value 2^(s-127); s = 255 encodes NaN.
 *  - One E8M0 scale per 32 consecutive K-elements of one output row.
 *  - Element 2j sits in the low nibble (bits 3..0) of byte j, 2j+1 in the high nibble.
 *  - Top-k order: larger logit first; an exact tie goes to the lower expert id;
 *    NaN logits rank after every number. Gates are the full-softmax probabilities
 *    of the chosen ids (no renormalisation over the k).
 *  - Expert: SwiGLU without biases, E(x) = D (silu(G x) * (U x)), silu(z) = z/(1+e^-z).
 *  - Combine: y = sum over slots 0..k-1, in slot order, of gate * E(x).
 *  - Block: xhat = h / sqrt(mean(h^2) + eps) * gamma; h_out = (h + S(xhat)) + y(xhat).
 */
#include "k3oracle.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- element decoding ---------------------------------------------------- */

/* OCP MX v1.0 E2M1: normal (e>0) = (-1)^s 2^(e-1) (1 + m/2); subnormal (e=0) = (-1)^s m/2. */
double k3o_e2m1(uint32_t code) {
  uint32_t sgn = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return sgn ? -mag : mag;
}

/* E8M0 shared scale: a bare biased exponent (bias 127); 0xFF is NaN. */
double k3o_e8m0(uint32_t s) {
  s &= 0xFFu;
  if (s == 255u) return NAN;
  return ldexp(1.0, (int)s - 127);
}

double k3o_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static inline double bf16d(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint32_t k3o_nibble(const uint8_t* q, int64_t k) {
  uint8_t b = q[k >> 1];
  return (k & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 15u);
}

/* Decode one packed row of K elements: w[k] = e2m1(code_k) * e8m0(scale of block k/32). */
void k3o_mx_row(const uint8_t* q, const uint8_t* s, int32_t K, double* w) {
  for (int32_t k = 0; k < K; ++k) w[k] = k3o_e2m1(k3o_nibble(q, k)) * k3o_e8m0(s[k >> 5]);
}

/* sum_k w_k x_k, k = 0..K-1 in order, per-element scaling. */
double k3o_mx_dot(const uint8_t* q, const uint8_t* s, int32_t K, const double* x) {
  double acc = 0.0;
  for (int32_t k = 0; k < K; ++k)
    acc += (k3o_e2m1(k3o_nibble(q, k)) * k3o_e8m0(s[k >> 5])) * x[k];
  return acc;
}

/* Same contraction, scale applied once per 32-block after the block's own sum
 * ([C]: accumulate on the unscaled codes, multiply by the scale once). With
 * power-of-two scales this equals k3o_mx_dot exactly, barring over/underflow. */
double k3o_mx_dot_blockscaled(const uint8_t* q, const uint8_t* s, int32_t K,
                              const double* x) {
  double acc = 0.0;
  for (int32_t b = 0; b < K / 32; ++b) {
    double bs = 0.0;
    for (int32_t k = 32 * b; k < 32 * b + 32; ++k) bs += k3o_e2m1(k3o_nibble(q, k)) * x[k];
    acc += k3o_e8m0(s[b]) * bs;
  }
  return acc;
}

void k3o_load_x(int64_t n, const void* x, int32_t dtype, double* out) {
  if (dtype == K3O_BF16) {
    const uint16_t* p = (const uint16_t*)x;
    for (int64_t i = 0; i < n; ++i) out[i] = bf16d(p[i]);
  } else if (dtype == K3O_F32) {
    const float* p = (const float*)x;
    for (int64_t i = 0; i < n; ++i) out[i] = (double)p[i];
  } else {
    memcpy(out, x, (size_t)n * sizeof(double));
  }
}

/* ---- routing ------------------------------------------------------------- */

/* [A] §2.4 router GEMV: logit_e = sum_k x_k W[k][e] over the [hidden][experts]
 * gate matrix, k in order; then + bias_e when a bias is given. */
void k3o_router_logits(int32_t T, int32_t d, int32_t E, const double* x,
                       const uint16_t* w, const float* bias, double* logits) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t t = 0; t < T; ++t) {
    double* l = logits + (int64_t)t * E;
    for (int32_t e = 0; e < E; ++e) l[e] = 0.0;
    const double* xt = x + (int64_t)t * d;
    for (int32_t k = 0; k < d; ++k) {
      const double xk = xt[k];
      const uint16_t* wr = w + (int64_t)k * E;
      for (int32_t e = 0; e < E; ++e) l[e] += xk * bf16d(wr[e]);
    }
    if (bias)
      for (int32_t e = 0; e < E; ++e) l[e] += (double)bias[e];
  }
}

/* [A] §2.4 stable softmax over ALL experts: subtract the max, exponentiate, normalise. */
void k3o_softmax(int32_t E, const double* l, double* p) {
  double m = l[0];
  for (int32_t e = 1; e < E; ++e)
    if (l[e] > m) m = l[e];
  double s = 0.0;
  for (int32_t e = 0; e < E; ++e) {
    p[e] = exp(l[e] - m);
    s += p[e];
  }
  for (int32_t e = 0; e < E; ++e) p[e] = p[e] / s;
}

/* a ranks before b? larger logit first; equal logits -> lower id; NaN last. */
static int ranks_before(double la, int32_t a, double lb, int32_t b) {
  int na = isnan(la), nb = isnan(lb);
  if (na != nb) return nb;
  if (!na && la != lb) return la > lb;
  return a < b;
}

/* [A] §2.4 top-k by repeated selection of the best remaining expert (strict
 * comparison, so the first index wins a tie); returns ids in rank order. */
void k3o_topk(int32_t E, int32_t k, const double* l, int32_t* ids) {
  unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
  for (int32_t r = 0; r < k; ++r) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
    }
    ids[r] = best;
    taken[best] = 1;
  }
  free(taken);
}

/* [A] §1.2 / §2.4: gates are softmax probabilities of the chosen experts. */
void k3o_route(int32_t T, int32_t E, int32_t k, const double* logits, int32_t* ids,
               double* gates) {
#pragma omp parallel
  {
    double* p = (double*)malloc((size_t)E * sizeof(double));
#pragma omp for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
      const double* l = logits + (int64_t)t * E;
      k3o_softmax(E, l, p);
      k3o_topk(E, k, l, ids + (int64_t)t * k);
      for (int32_t r = 0; r < k; ++r) gates[(int64_t)t * k + r] = p[ids[(int64_t)t * k + r]];
    }
    free(p);
  }
}

/* Stable counting sort of the T*k (token, slot) pairs by expert: offsets[e] is
 * the first position of expert e, rows[] holds pair ids t*k+slot, ascending
 * within each expert. Returns -1 on an id outside [0, E). */
int k3o_bucket(int32_t T, int32_t E, int32_t k, const int32_t* ids, int32_t* offsets,
               int32_t* rows) {
  const int64_t n = (int64_t)T * k;
  for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
  for (int64_t p = 0; p < n; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return -1;
    offsets[ids[p] + 1] += 1;
  }
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  int32_t* next = (int32_t*)malloc((size_t)(E > 0 ? E : 1) * sizeof(int32_t));
  for (int32_t e = 0; e < E; ++e) next[e] = offsets[e];
  for (int64_t p = 0; p < n; ++p) rows[next[ids[p]]++] = (int32_t)p;
  free(next);
  return 0;
}

/* ---- experts --------------------------------------------------------------- */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert on one token: u = G x, v = U x, h = silu(u) * v, out = D h. */
void k3o_expert_ffn(int32_t d, int32_t f, const double* x, const k3o_expert* w,
                    double* h_out, double* out) {
  double* h = h_out ? h_out : (double*)malloc((size_t)f * sizeof(double));
  const int64_t rq = d / 2, rs = d / 32;
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < f; ++j) {
    double u = k3o_mx_dot(w->gate_q + j * rq, w->gate_s + j * rs, d, x);
    double v = k3o_mx_dot(w->up_q + j * rq, w->up_s + j * rs, d, x);
    h[j] = silu(u) * v;
  }
  const int64_t dq = f / 2, ds = f / 32;
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < d; ++i) out[i] = k3o_mx_dot(w->down_q + i * dq, w->down_s + i * ds, f, h);
  if (!h_out) free(h);
}

/* [A] §1.2 y = sum_i g_i E_i(x) over the token's k experts, in slot order. */
int k3o_moe_combine(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                    const double* x, const int32_t* ids, const double* gates,
                    const k3o_expert* experts, double* y) {
  double* z = (double*)malloc((size_t)d * sizeof(double));
  for (int32_t t = 0; t < T; ++t) {
    double* yt = y + (int64_t)t * d;
    for (int32_t i = 0; i < d; ++i) yt[i] = 0.0;
    for (int32_t r = 0; r < k; ++r) {
      int32_t e = ids[(int64_t)t * k + r];
      if (e < 0 || e >= E || !experts[e].gate_q || !experts[e].gate_s || !experts[e].up_q ||
          !experts[e].up_s || !experts[e].down_q || !experts[e].down_s) {
        free(z);
        return -1;
      }
      k3o_expert_ffn(d, f, x + (int64_t)t * d, &experts[e], NULL, z);
      const double g = gates[(int64_t)t * k + r];
      for (int32_t i = 0; i < d; ++i) yt[i] += g * z[i];
    }
  }
  free(z);
  return 0;
}

/* ---- block extras ------------------------------------------------------------ */

void k3o_rmsnorm(int32_t d, const double* h, const uint16_t* gamma, double eps,
                 double* out) {
  double ss = 0.0;
  for (int32_t i = 0; i < d; ++i) ss += h[i] * h[i];
  const double r = sqrt(ss / (double)d + eps);
  for (int32_t i = 0; i < d; ++i) out[i] = h[i] / r * bf16d(gamma[i]);
}

/* Dense bf16 SwiGLU (the always-active shared expert). */
void k3o_dense_swiglu(int32_t d, int32_t f, const double* x, const uint16_t* wg,
                      const uint16_t* wu, const uint16_t* wd, double* out) {
  double* h = (double*)malloc((size_t)f * sizeof(double));
#pragma omp parallel for schedule(static)
  for (int32_t j = 0; j < f; ++j) {
    double u = 0.0, v = 0.0;
    for (int32_t k = 0; k < d; ++k) u += bf16d(wg[(int64_t)j * d + k]) * x[k];
    for (int32_t k = 0; k < d; ++k) v += bf16d(wu[(int64_t)j * d + k]) * x[k];
    h[j] = silu(u) * v;
  }
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < d; ++i) {
    double a = 0.0;
    for (int32_t j = 0; j < f; ++j) a += bf16d(wd[(int64_t)i * f + j]) * h[j];
    out[i] = a;
  }
  free(h);
}

/* ---- whole layer ------------------------------------------------------------ */

/* Input of the router and experts: x itself, or RMSNorm(h) in block mode. */
static double* layer_input(int32_t T, int32_t d, const void* x, int32_t x_dtype,
                           const k3o_block* blk) {
  double* xin = (double*)malloc((size_t)T * d * sizeof(double));
  k3o_load_x((int64_t)T * d, x, x_dtype, xin);
  if (blk) {
    double* tmp = (double*)malloc((size_t)d * sizeof(double));
    for (int32_t t = 0; t < T; ++t) {
      k3o_rmsnorm(d, xin + (int64_t)t * d, blk->gamma, blk->eps, tmp);
      memcpy(xin + (int64_t)t * d, tmp, (size_t)d * sizeof(double));
    }
    free(tmp);
  }
  return xin;
}

int k3o_layer_route(int32_t T, int32_t d, int32_t E, int32_t k, const void* x,
                    int32_t x_dtype, const uint16_t* w_router, const float* bias,
                    const k3o_block* blk, int32_t* ids, double* gates, double* logits,
                    double* xin_out) {
  if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E) return -1;
  double* xin = layer_input(T, d, x, x_dtype, blk);
  double* l = logits ? logits : (double*)malloc((size_t)T * E * sizeof(double) + 8);
  k3o_router_logits(T, d, E, xin, w_router, bias, l);
  k3o_route(T, E, k, l, ids, gates);
  if (xin_out) memcpy(xin_out, xin, (size_t)T * d * sizeof(double));
  if (!logits) free(l);
  free(xin);
  return 0;
}

int k3o_layer_forward(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                      const void* x, int32_t x_dtype, const uint16_t* w_router,
                      const float* bias, const k3o_expert* experts, const k3o_block* blk,
                      double* y, int32_t* ids, double* gates) {
  if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k < 1 || k > E || d % 32 || f % 32) return -1;
  double* xin = layer_input(T, d, x, x_dtype, blk);
  double* l = (double*)malloc((size_t)T * E * sizeof(double) + 8);
  k3o_router_logits(T, d, E, xin, w_router, bias, l);
  k3o_route(T, E, k, l, ids, gates);
  free(l);
  int rc = k3o_moe_combine(T, d, f, E, k, xin, ids, gates, experts, y);
  if (rc == 0 && blk) {
    /* h_out = (h + S(xhat)) + y(xhat), with h the fp32/bf16 input itself */
    double* h = (double*)malloc((size_t)T * d * sizeof(double));
    double* s = (double*)malloc((size_t)d * sizeof(double));
    k3o_load_x((int64_t)T * d, x, x_dtype, h);
    for (int32_t t = 0; t < T; ++t) {
      k3o_dense_swiglu(d, f, xin + (int64_t)t * d, blk->sh_gate, blk->sh_up, blk->sh_down, s);
      double* yt = y + (int64_t)t * d;
      const double* ht = h + (int64_t)t * d;
      for (int32_t i = 0; i < d; ++i) yt[i] = (ht[i] + s[i]) + yt[i];
    }
    free(s);
    free(h);
  }
  free(xin);
  return rc;
}
