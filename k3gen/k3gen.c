/*
 * k3gen.c — host implementation of the seeded input generator declared in
 * k3gen.h (SplitMix64 in counter form; Box-Muller normals; one-step RNE to
 * bf16). Input drawing only: nothing here decodes, multiplies or routes.
 */
#include "k3gen.h"
#include <math.h>
#include <string.h>

#define K3GEN_GAMMA 0x9E3779B97F4A7C15ULL

uint64_t k3gen_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t k3gen_at(uint64_t key, uint64_t i) {
  return k3gen_mix(key + (i + 1) * K3GEN_GAMMA);
}

uint64_t k3gen_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c) {
  return k3gen_at(k3gen_at(k3gen_at(seed, a), b), c);
}

void k3gen_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out) {
  if (n == 0) return;
  /* head up to the next 8-byte word boundary */
  uint64_t idx = 0;
  while (idx < n && ((start + idx) & 7)) {
    uint64_t j = start + idx;
    out[idx++] = (uint8_t)(k3gen_at(key, j >> 3) >> (8 * (j & 7)));
  }
  uint64_t nw = (n - idx) >> 3;
  uint64_t w0 = (start + idx) >> 3;
  uint8_t* base = out + idx;
#pragma omp parallel for schedule(static) if (nw > (1u << 16))
  for (int64_t w = 0; w < (int64_t)nw; ++w) {
    uint64_t v = k3gen_at(key, w0 + (uint64_t)w);
    for (int b = 0; b < 8; ++b) base[8 * w + b] = (uint8_t)(v >> (8 * b));
  }
  idx += nw << 3;
  while (idx < n) {
    uint64_t j = start + idx;
    out[idx++] = (uint8_t)(k3gen_at(key, j >> 3) >> (8 * (j & 7)));
  }
}

void k3gen_e8m0(uint64_t key, uint64_t start, uint64_t n, int lo, int count,
                uint8_t* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 16))
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint64_t hi = k3gen_at(key, start + (uint64_t)i) >> 32;
    out[i] = (uint8_t)(lo + (int)((hi * (uint64_t)count) >> 32));
  }
}

double k3gen_normal_f64(uint64_t key, uint64_t j) {
  uint64_t a = k3gen_at(key, 2 * j), b = k3gen_at(key, 2 * j + 1);
  double u1 = ((double)(a >> 11) + 1.0) * 0x1p-53; /* (0, 1] */
  double u2 = (double)(b >> 11) * 0x1p-53;         /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

uint16_t k3gen_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  /* 8 significant bits for normals; fixed spacing 2^-133 below 2^-126 */
  int ulp_exp = (e >= -125) ? e - 8 : -133;
  double q = nearbyint(ldexp(a, -ulp_exp)); /* exact scale, then RNE */
  double r = ldexp(q, ulp_exp);
  if (r >= 0x1p128) return sign | 0x7F80;
  float f = (float)r; /* exact: at most 8 significant bits */
  uint32_t fu;
  memcpy(&fu, &f, 4);
  return sign | (uint16_t)(fu >> 16);
}

void k3gen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double mean,
                       double sd, uint16_t* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 14))
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = k3gen_f64_to_bf16(mean + sd * k3gen_normal_f64(key, start + (uint64_t)i));
}

void k3gen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double mean,
                      double sd, float* out) {
#pragma omp parallel for schedule(static) if (n > (1u << 14))
  for (int64_t i = 0; i < (int64_t)n; ++i)
    out[i] = (float)(mean + sd * k3gen_normal_f64(key, start + (uint64_t)i));
}

void k3gen_zipf_bias(uint64_t key, int32_t E, double alpha, int32_t* rank_out,
                     float* bias_out) {
  for (int32_t i = 0; i < E; ++i) rank_out[i] = i + 1;
  for (int32_t i = E - 1; i > 0; --i) {
    uint64_t hi = k3gen_at(key, (uint64_t)i) >> 32;
    int32_t j = (int32_t)((hi * (uint64_t)(i + 1)) >> 32);
    int32_t t = rank_out[i];
    rank_out[i] = rank_out[j];
    rank_out[j] = t;
  }
  for (int32_t e = 0; e < E; ++e)
    bias_out[e] = (float)(-alpha * log((double)rank_out[e]));
}
