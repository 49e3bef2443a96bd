/* k3cpu.h — tuned CPU implementation of the routed-expert MoE layer (bf16 tokens), equal
 * to the plain fp64 definition bit for bit; the CPU comparator of the GPU path. */
#ifndef K3CPU_H
#define K3CPU_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct { /* one expert, host pointers (layouts as in include/k3moe.h) */
  const uint8_t *gate_q, *gate_s; /* [d_ff][d_model/2], [d_ff][d_model/32] */
  const uint8_t *up_q, *up_s;
  const uint8_t *down_q, *down_s; /* [d_model][d_ff/2], [d_model][d_ff/32] */
} k3cpu_expert;

/* T tokens x (bf16 [T][d]); w_router bf16 [d][E]; bias fp32 [E] or NULL; experts[E] (only
 * the selected ones are read). Writes y fp64 [T][d], ids [T][k], gates fp64 [T][k].
 * Returns 0, -1 on bad sizes or a selected expert without weights, -2 without memory. */
int k3cpu_layer_forward(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                        const uint16_t* x, const uint16_t* w_router, const float* bias,
                        const k3cpu_expert* experts, double* y, int32_t* ids, double* gates);
/* Routing only (router GEMV, softmax, top-k) of the same layer: ids [T][k], gates [T][k]. */
int k3cpu_layer_route(int32_t T, int32_t d, int32_t E, int32_t k, const uint16_t* x,
                      const uint16_t* w_router, const float* bias, int32_t* ids,
                      double* gates);
/* 1 when the AVX2 paths run on this host, else 0 (scalar loops, same results). */
int k3cpu_simd(void);

#ifdef __cplusplus
}
#endif
#endif
