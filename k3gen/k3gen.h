/*
 * k3gen.h — seeded synthetic-input generator (host side).
 *
 * This module only draws inputs. It holds none of the MoE method's
 * arithmetic: no decoding, no dot products, no routing. Both the CPU oracle
 * harness and the GPU tests take their inputs from it, so it is the one piece
 * of code the two sides share.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used in counter form: output i of the
 * stream with key K is mix(K + (i+1)*0x9E3779B97F4A7C15), where mix is the
 * published SplitMix64 finaliser. Every value is therefore addressable by
 * (key, index) and can be regenerated on demand, on the host or the device,
 * without holding whole tensors in memory.
 *
 * Draws (all little-endian, index-addressed):
 *   bytes   : byte j = byte (j mod 8) of output floor(j/8)        -> packed
 *             MXFP4 nibbles, each nibble uniform over the 16 codes
 *   e8m0    : byte j = lo + ((output j >> 32) * count >> 32)      -> scale
 *             exponent bytes uniform in [lo, lo+count)
 *   normal  : value j = mean + sd * sqrt(-2 ln u1) cos(2 pi u2),
 *             u1 = ((out(2j) >> 11) + 1) * 2^-53 in (0,1],
 *             u2 = (out(2j+1) >> 11) * 2^-53 in [0,1)  (Box-Muller)
 *             then rounded ONCE, fp64 -> bf16, round-to-nearest-even.
 *   zipf    : Fisher-Yates permutation of ranks 1..E driven by the stream;
 *             bias_e = (float)(-alpha * ln(rank_e)).
 */
#ifndef K3GEN_H
#define K3GEN_H
#include <stdint.h>
#include <stddef.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Master seed of every synthetic workload ("K3MOE" in ASCII). */
#define K3GEN_MASTER_SEED 0x4B334D4F45ULL

/* Tensor tags used to derive stream keys. */
enum {
  K3GEN_T_X = 1,        /* token activations (c = token-set index)      */
  K3GEN_T_WROUTER = 2,  /* router weight [d][E] bf16                    */
  K3GEN_T_ZIPF = 3,     /* permutation behind the Zipf logit bias       */
  K3GEN_T_GATE_Q = 4, K3GEN_T_GATE_S = 5,
  K3GEN_T_UP_Q = 6,   K3GEN_T_UP_S = 7,
  K3GEN_T_DOWN_Q = 8, K3GEN_T_DOWN_S = 9,
  K3GEN_T_GAMMA = 10,   /* RMSNorm gain, bf16(1 + 0.1 N(0,1))           */
  K3GEN_T_SH_GATE = 11, K3GEN_T_SH_UP = 12, K3GEN_T_SH_DOWN = 13,
  K3GEN_T_RESID = 14    /* fp32 residual stream entering the first block */
};

uint64_t k3gen_mix(uint64_t z);
/* Output i of the SplitMix64 stream whose state starts at `key`. */
uint64_t k3gen_at(uint64_t key, uint64_t i);
/* Key of the stream for (seed, a, b, c): at(at(at(seed, a), b), c). */
uint64_t k3gen_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c);

void k3gen_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out);
void k3gen_e8m0(uint64_t key, uint64_t start, uint64_t n, int lo, int count,
                uint8_t* out);
double k3gen_normal_f64(uint64_t key, uint64_t j);
/* One-step round-to-nearest-even of a double to bfloat16 bits. */
uint16_t k3gen_f64_to_bf16(double v);
void k3gen_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double mean,
                       double sd, uint16_t* out);
/* fp32 normals: value rounded once, fp64 -> fp32 (C cast, RNE). */
void k3gen_normal_f32(uint64_t key, uint64_t start, uint64_t n, double mean,
                      double sd, float* out);
void k3gen_zipf_bias(uint64_t key, int32_t E, double alpha, int32_t* rank_out,
                     float* bias_out);

#ifdef __cplusplus
}
#endif
#endif
