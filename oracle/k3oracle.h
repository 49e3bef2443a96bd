/*
 * k3oracle.h — plain, slow, fp64 CPU oracle of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * Everything is computed in fp64 from exactly decoded inputs; every sum runs
 * sequentially in index order, so results do not depend on the OpenMP thread
 * count (threads only split independent outputs).
 *
 * Sources (the web pages describing the CPU engine kimi-k3-in-c):
 *  [A] "Kimi K3 纯 C 语言 CPU 推理实战" (chenxutan.com/d/5901.html):
 *      §1.2 (MoE routing formula y = sum_i g_i(x) E_i(x), g = TopK(Softmax(W_gate x)), K=16),
 *      §2.3 (quantised GEMM: weight stored [N][K], one scale per 32 consecutive K),
 *      §2.4 (router GEMV over a [hidden][experts] gate matrix; max-subtracted softmax over
 *            all experts; top-k by strict-greater selection; combine weighted by the
 *            full-softmax probability).
 *  [B] "P053 FareedKhan-dev/kimi-k3-in-c" (ai-trend-radar project card), core features:
 *      MXFP4 = 4-bit E2M1 nibble + shared E8M0 scale, 0.53125 B/weight; top-16 of 896.
 *  [C] "用纯C语言把1.56TB的Kimi K3模型塞进8GB内存运行" (kongchang.com), section on experts
 *      never being resident: multiply the packed 4-bit form, accumulate, scale once.
 * Element encodings follow the OCP Microscaling Formats (MX) v1.0 specification
 * (E2M1 element, E8M0 shared scale), which is what "E2M1 + E8M0" names.
 */
#ifndef K3ORACLE_H
#define K3ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { K3O_BF16 = 0, K3O_F32 = 1, K3O_F64 = 2 };

typedef struct {
  const uint8_t *gate_q, *gate_s; /* [f][d/2] packed nibbles, [f][d/32] E8M0 */
  const uint8_t *up_q, *up_s;     /* same shapes as gate                      */
  const uint8_t *down_q, *down_s; /* [d][f/2], [d][f/32]                      */
} k3o_expert;

typedef struct {
  const uint16_t* gamma; /* bf16 [d] RMSNorm gain                          */
  double eps;            /* added to mean(h^2) inside the square root      */
  const uint16_t *sh_gate, *sh_up; /* bf16 [f][d]                          */
  const uint16_t* sh_down;         /* bf16 [d][f]                          */
} k3o_block;

/* ---- element decoding (exact) ------------------------------------------ */
double k3o_e2m1(uint32_t code);         /* 4-bit code -> value              */
double k3o_e8m0(uint32_t s);            /* 2^(s-127); s = 255 -> NaN        */
double k3o_bf16(uint16_t bits);
uint32_t k3o_nibble(const uint8_t* q, int64_t k); /* code of element k      */
void k3o_mx_row(const uint8_t* q, const uint8_t* s, int32_t K, double* w);
double k3o_mx_dot(const uint8_t* q, const uint8_t* s, int32_t K, const double* x);
double k3o_mx_dot_blockscaled(const uint8_t* q, const uint8_t* s, int32_t K,
                              const double* x);
void k3o_load_x(int64_t n, const void* x, int32_t dtype, double* out);

/* ---- routing ------------------------------------------------------------ */
void k3o_router_logits(int32_t T, int32_t d, int32_t E, const double* x,
                       const uint16_t* w, const float* bias, double* logits);
void k3o_softmax(int32_t E, const double* l, double* p);
void k3o_topk(int32_t E, int32_t k, const double* l, int32_t* ids);
void k3o_route(int32_t T, int32_t E, int32_t k, const double* logits, int32_t* ids,
               double* gates);
int k3o_bucket(int32_t T, int32_t E, int32_t k, const int32_t* ids, int32_t* offsets,
               int32_t* rows);

/* ---- experts -------------------------------------------------------------- */
void k3o_expert_ffn(int32_t d, int32_t f, const double* x, const k3o_expert* w,
                    double* h_out, double* out);
int k3o_moe_combine(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                    const double* x, const int32_t* ids, const double* gates,
                    const k3o_expert* experts, double* y);

/* ---- block extras ------------------------------------------------------- */
void k3o_rmsnorm(int32_t d, const double* h, const uint16_t* gamma, double eps,
                 double* out);
void k3o_dense_swiglu(int32_t d, int32_t f, const double* x, const uint16_t* wg,
                      const uint16_t* wu, const uint16_t* wd, double* out);

/* ---- whole layer -------------------------------------------------------- */
int k3o_layer_route(int32_t T, int32_t d, int32_t E, int32_t k, const void* x,
                    int32_t x_dtype, const uint16_t* w_router, const float* bias,
                    const k3o_block* blk, int32_t* ids, double* gates, double* logits,
                    double* xin_out);
int k3o_layer_forward(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                      const void* x, int32_t x_dtype, const uint16_t* w_router,
                      const float* bias, const k3o_expert* experts, const k3o_block* blk,
                      double* y, int32_t* ids, double* gates);

#ifdef __cplusplus
}
#endif
#endif
