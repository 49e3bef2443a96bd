/*
 * k3moe.h — C ABI of the MI355X (gfx950) routed-expert MoE FFN on MXFP4 weights.
 *
 * What it computes. For each token t with activation x_t (d_model wide):
 *     logits_t = W_router^T x_t (+ bias)           router GEMV over all E experts
 *     p_t      = softmax(logits_t) over all E       max-subtracted
 *     ids_t    = the top_k experts by logit, largest first, equal logits -> lower id
 *     gates_t  = p_t[ids_t]                         full-softmax probabilities, no renorm
 *     y_t      = sum_{slot} gates_t[slot] * E_{ids_t[slot]}(x_t)
 *     E_e(x)   = D_e (silu(G_e x) * (U_e x))        SwiGLU expert, silu(z) = z/(1+e^-z)
 * with G_e, U_e, D_e stored as MXFP4 and multiplied from the packed form.
 * Sources: "Kimi K3 纯 C 语言 CPU 推理实战" (chenxutan.com/d/5901.html) §1.2 (the routing
 * formula y = sum_i g_i(x) E_i(x), g = TopK(Softmax(W_gate x)), K = 16) and §2.4 (router
 * GEMV over a [hidden][experts] gate matrix, stable softmax over all experts,
 * strict-greater top-k selection, combine weighted by the full probability);
 * project card "P053 FareedKhan-dev/kimi-k3-in-c", core features (MXFP4 = E2M1 nibble +
 * shared E8M0 scale, 0.53125 B/weight; packed nibbles are multiplied, never dequantised).
 *
 * Data formats (all row-major, little-endian):
 *   MXFP4 matrix [R][K]: nibbles uint8 [R][K/2], element 2j in bits 3..0 of byte j,
 *     element 2j+1 in bits 7..4; scales uint8 [R][K/32], one E8M0 byte per 32
 *     consecutive K-elements of a row. E2M1 code: bit 3 sign, bits 2..1 exponent
 *     (bias 1), bit 0 mantissa (values 0, .5, 1, 1.5, 2, 3, 4, 6 and negatives).
 *     E8M0 byte s: 2^(s-127); s = 255 is NaN and propagates as NaN.
 *   Expert tensors of one layer: gate, up [E][d_ff][d_model] and down [E][d_model][d_ff]
 *     as MXFP4 matrices stacked over experts (so gate_q is [E][d_ff][d_model/2]).
 *   Router weight: bf16 [d_model][E]. Optional logit bias: fp32 [E], added before softmax.
 *   Activations: bf16 (K3MOE_BF16) or fp32 (K3MOE_F32), [T][d_model].
 *   Routing: topk_ids int32 [T][top_k], topk_gates fp32 [T][top_k].
 *   Bucketing: expert_offsets int32 [E+1] (prefix sums of per-expert token counts),
 *     bucket_rows int32 [T*top_k] holding pair ids t*top_k+slot, grouped by expert in
 *     ascending expert id and ascending t within each expert.
 *   Output y: fp32 [T][d_model], overwritten. y_bf16, when given, holds the
 *     round-to-nearest-even bf16 of y.
 *
 * Conventions of every entry point:
 *   - Every pointer argument except `stream` and the structs' host copies is DEVICE
 *     memory owned by the caller. The library never allocates device memory; its only
 *     state is cached device properties and, once block mode has run on a device, one
 *     non-blocking side stream of default priority for that device and, per host thread
 *     that ran block mode there, one pair of fork/join events (kept until k3moe_release()
 *     or the process end; the slot cache below keeps copy streams the same way). Calls
 *     with distinct workspaces may run concurrently on distinct streams.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = default
 *     stream). The caller synchronises. In block mode the shared expert runs on the
 *     side stream, forked from `stream` after the RMSNorm and joined back into it (by
 *     the calling thread's events) before the launch that adds it into y, so all of a
 *     call's work is complete once `stream` is; the same calls can be captured into a
 *     HIP graph on `stream` (the side stream joins the capture through the fork event).
 *     Results are bit-identical from run to run.
 *   - Arguments are validated on the host before anything is enqueued; nothing is
 *     defaulted. Errors: K3MOE_EINVAL (null required pointer, negative T, d_model or
 *     d_ff not a positive multiple of 32, n_experts < 1, top_k outside
 *     [1, min(n_experts, 32)], unknown dtype), K3MOE_EUNSUPPORTED (valid but outside
 *     what the kernels implement, e.g. T or E above the limits below),
 *     K3MOE_EWORKSPACE (ws_bytes below k3moe_workspace_bytes(dims, T)), K3MOE_EHIP (a
 *     HIP launch failed). T = 0 returns K3MOE_OK and enqueues nothing.
 *     k3moe_last_error() gives a message for the calling thread's last failure.
 *   - Input values are not scanned: NaN inputs and E8M0 255 propagate as NaN.
 *   - Alignment: x, y and the MXFP4 nibble arrays must be 16-byte aligned (EINVAL).
 *     With 16 or more tokens, bf16 activations, d_model and d_ff multiples of 128 and
 *     4-byte aligned scale arrays, the expert matmuls run as grouped GEMMs on the
 *     block-scaled FP4 x FP8 MFMA: the token enters as two FP8 (E4M3) terms with one
 *     E8M0 scale per term row, which carry every bf16 element to about 2^-22 of the row's
 *     largest magnitude (smaller elements lose low bits); h enters as three FP8 terms
 *     with one scale per term and 32-element block (to about 2^-13 of the block's
 *     largest magnitude). Otherwise the matmuls run as per-expert GEMVs on fp32
 *     conversions of the packed weights. All accumulate in fp32.
 *   - Limits (EUNSUPPORTED beyond): n_experts <= 4096, T <= 1048576, d_model <= 16384,
 *     d_ff <= 16384; the expert kernels also need (d_ff/32)/p <= 4, with p the largest
 *     power of two <= 64 dividing d_ff/32 (true for d_ff = 1536, 256, 32, any multiple
 *     of 2048, ...). The workspace grows about as T * top_k * 4 * (d_model + d_ff) bytes
 *     (1.27 GB at T = 2048 on the K3 layer), so in practice HBM bounds T well below the
 *     nominal limit: split longer prefills into chunks.
 */
#ifndef K3MOE_H
#define K3MOE_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define K3MOE_VERSION 1

#if defined(__GNUC__)
#define K3MOE_API __attribute__((visibility("default")))
#else
#define K3MOE_API
#endif

typedef struct {
  int32_t d_model;   /* hidden width d (7168 for the K3 layer)   */
  int32_t d_ff;      /* expert inner width f (1536)              */
  int32_t n_experts; /* routed experts E (896)                   */
  int32_t top_k;     /* experts per token k (16)                 */
} k3moe_dims;

typedef struct { /* one layer of routed experts, device pointers, caller-owned */
  const uint8_t *gate_q, *gate_s; /* [E][d_ff][d_model/2], [E][d_ff][d_model/32] */
  const uint8_t *up_q, *up_s;     /* same shapes as gate                        */
  const uint8_t *down_q, *down_s; /* [E][d_model][d_ff/2], [E][d_model][d_ff/32] */
} k3moe_mx_experts;

typedef struct { /* extras of a full block; device pointers except rms_eps */
  const uint16_t* rms_gamma; /* bf16 [d_model]                          */
  float rms_eps;             /* added to mean(h^2) inside the sqrt      */
  const uint16_t* sh_gate;   /* bf16 [d_ff][d_model] shared expert      */
  const uint16_t* sh_up;     /* bf16 [d_ff][d_model]                    */
  const uint16_t* sh_down;   /* bf16 [d_model][d_ff]                    */
} k3moe_block;

enum {
  K3MOE_OK = 0,
  K3MOE_EINVAL = -1,
  K3MOE_EUNSUPPORTED = -2,
  K3MOE_EWORKSPACE = -3,
  K3MOE_EHIP = -4
};
enum { K3MOE_BF16 = 0, K3MOE_F32 = 1 };

/* Library version (K3MOE_VERSION). */
K3MOE_API int k3moe_version(void);

/* Device workspace, in bytes, that any entry point needs for up to max_tokens
 * tokens with these dims; 0 when dims are invalid. Pure host function. */
K3MOE_API size_t k3moe_workspace_bytes(const k3moe_dims* dims, int32_t max_tokens);

/* Router GEMV + softmax + top-k ("Kimi K3 纯 C 语言 CPU 推理实战" §2.4, compute_gate_scores
 * followed by the softmax and top-k steps of moe_forward).
 * x: [T][d_model] of x_dtype. w_router: bf16 [d_model][E]. logit_bias: fp32 [E] or NULL.
 * Logits are accumulated in fp64 (bf16*bf16 and bf16*fp32 products are exact there), so
 * the selected ids and their order are those of the exact-arithmetic definition.
 * Writes topk_ids [T][k] and topk_gates [T][k]. */
K3MOE_API int k3moe_router(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                 const uint16_t* w_router, const float* logit_bias, int32_t* topk_ids,
                 float* topk_gates, void* ws, size_t ws_bytes, void* stream);

/* Stable counting sort of the T*k (token, slot) pairs by expert: the per-expert token lists
 * that let each selected expert's weights be read once for all tokens routed to it, and
 * experts routed no token be skipped ("用纯C语言把1.56TB的Kimi K3模型塞进8GB内存运行",
 * kongchang.com, section 专家权重永不常驻内存: the router decides which experts are read;
 * "Kimi K3 纯 C 语言 CPU 推理实战" §2.4, moe_forward's loop over the selected experts of each
 * token). topk_ids: [T][k], each in [0, E) and distinct within a token (ids outside [0, E)
 * are a caller error; the kernels ignore such pairs).
 * Writes expert_offsets [E+1] and bucket_rows [T*k]. */
K3MOE_API int k3moe_route_bucket(const k3moe_dims* dims, int32_t T, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* bucket_rows, void* ws,
                       size_t ws_bytes, void* stream);

/* Routed experts + gate-weighted combine for already-routed tokens ("Kimi K3 纯 C 语言 CPU
 * 推理实战" §1.2, y = sum_i g_i(x) E_i(x); §2.4, moe_forward's expert evaluation and
 * gate-weighted accumulation; §2.3, the [N][K] weight layout with 32-element scale groups;
 * project card "P053 FareedKhan-dev/kimi-k3-in-c", core features: the MXFP4 weights are
 * multiplied in packed form):
 * y_t = sum_slot topk_gates[t][slot] * E_e(x_t), e the expert whose bucket holds pair
 * t*k+slot. Each expert's MXFP4 weights are read once per call for all of its tokens and
 * either converted in registers (GEMV kernels) or fed as stored to the block-scaled FP4 x
 * FP8 MFMA (one token's down projection with d_ff a multiple of 128 up to 1536 and top_k
 * <= 16; grouped GEMMs from 16 tokens); nothing dequantised is written to memory. In the
 * MFMA paths h enters as three FP8 (E4M3) terms with E8M0 scales. Slots are summed in slot
 * order. x: [T][d_model] of x_dtype. y: fp32 [T][d_model], overwritten. */
K3MOE_API int k3moe_expert_ffn(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                     const k3moe_mx_experts* experts, const int32_t* expert_offsets,
                     const int32_t* bucket_rows, const float* topk_gates, float* y,
                     void* ws, size_t ws_bytes, void* stream);

/* One whole layer: router -> top-k -> bucket -> experts -> combine ("Kimi K3 纯 C 语言 CPU
 * 推理实战" §1.2 and §2.4, moe_forward). Block mode adds the parts of a decoder block
 * around it: RMSNorm ("用纯C语言把1.56TB的Kimi K3模型塞进8GB内存运行", kongchang.com, the
 * model's layer structure) and the always-active shared expert kept at high precision
 * ("Kimi K3 纯 C 语言 CPU 推理实战" §1.2, 16 routed experts plus one shared expert).
 * blk == NULL: y = MoE(x).
 * blk != NULL (block mode): x must be fp32 (x_dtype K3MOE_F32), the residual h;
 *   xhat = h / sqrt(mean(h^2) + rms_eps) * rms_gamma feeds the router, the routed experts
 *   and the shared bf16 SwiGLU expert S; y = h + S(xhat) + MoE(xhat) (fp32).
 * y_bf16 [T][d_model] (nullable) receives RNE(y). topk_ids / topk_gates (nullable)
 * receive the routing. */
K3MOE_API int k3moe_layer_forward(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                        const uint16_t* w_router, const float* logit_bias,
                        const k3moe_mx_experts* experts, const k3moe_block* blk, float* y,
                        uint16_t* y_bf16, int32_t* topk_ids, float* topk_gates, void* ws,
                        size_t ws_bytes, void* stream);

/* ---- Packed tile layout of the expert weights ------------------------------------------
 * The row-major layout above lets one load of a block-scaled MFMA operand (16 rows x 128
 * elements) read only 64 contiguous bytes per row. The packed layout stores each such tile
 * contiguously, in the order the MFMA's 64 lanes hold it, so one 16-byte-per-lane load reads
 * 1 KB in one piece; it holds the same E2M1 codes and E8M0 scales, permuted (nothing is
 * decoded). For an MXFP4 matrix [R][K] of one expert (R % 16 == 0, K % 128 == 0), with
 * nk = K/128 steps, nch = ceil(nk/8) chunks of 8 steps, tile t = rows 16t .. 16t+15 and lane
 * L = i + 16 g (i < 16, g < 4):
 *   codes  [R/16][nk][64][16 B]: entry (t, s, L) = bytes [64 s + 16 g, 64 s + 16 g + 16) of
 *          row 16 t + i (elements 128 s + 32 g .. 128 s + 32 g + 31), R K / 2 bytes in all;
 *   scales [R/16][nch][64][8 B]: byte j of entry (t, c, L) = the E8M0 scale of block
 *          4 (8 c + j) + g of row 16 t + i; 0 where 8 c + j >= nk.
 * Experts are stacked as in k3moe_mx_experts. The layout follows the MFMA's operand order on
 * gfx950; the formats themselves are those of "Kimi K3 纯 C 语言 CPU 推理实战" §2.3 ([N][K]
 * weights, one scale per 32 consecutive K elements) and the project card "P053
 * FareedKhan-dev/kimi-k3-in-c", core features (MXFP4, multiplied in packed form). Packed
 * experts need d_model % 1024 == 0 and d_ff % 512 == 0 (K3: 7168, 1536). */
typedef struct {
  size_t gate_q, gate_s, up_q, up_s, down_q, down_s; /* bytes per expert of each tensor */
} k3moe_packed_bytes;

/* Per-expert sizes of the packed tensors (codes keep their size; scales are padded to whole
 * chunks of 8 steps). Pure host function; K3MOE_EUNSUPPORTED for shapes the layout excludes. */
K3MOE_API int k3moe_packed_expert_bytes(const k3moe_dims* dims, k3moe_packed_bytes* per_expert);

/* Writes the packed copy of all dims->n_experts experts of `src` (row-major, device) into
 * `dst` (device buffers of k3moe_packed_expert_bytes per expert, scales 8-byte aligned;
 * must not overlap src). Asynchronous on `stream`. Meant to run once when weights are
 * loaded. */
K3MOE_API int k3moe_pack_experts(const k3moe_dims* dims, const k3moe_mx_experts* src,
                                 const k3moe_mx_experts* dst, void* stream);

/* k3moe_layer_forward with the experts in the packed layout (same arguments and results to
 * rounding). Every weight tile step is read as 1 KB contiguous. Activations are bf16; for one
 * token (T == 1, d_ff <= 1536, top_k <= 16) also fp32, and block mode (whose experts take the
 * fp32 RMSNorm output). One token: gate/up as a GEMV in fp32, one block per (slot, 16-row
 * tile) and one wave per 8 K steps, then the one-token down kernel on the block-scaled MFMA
 * (h as three FP8 terms) with the gate-weighted sum in slot order. More tokens: grouped GEMMs
 * on the block-scaled FP4 x FP8 MFMA (token as two FP8 terms, h as three).
 * K3MOE_EUNSUPPORTED for shapes or activations outside the above. */
K3MOE_API int k3moe_layer_forward_packed(const k3moe_dims* dims, int32_t T, const void* x,
                                         int x_dtype, const uint16_t* w_router,
                                         const float* logit_bias,
                                         const k3moe_mx_experts* experts,
                                         const k3moe_block* blk, float* y, uint16_t* y_bf16,
                                         int32_t* topk_ids, float* topk_gates, void* ws,
                                         size_t ws_bytes, void* stream);

/* Bytes of the static device scratch behind k3moe_layer_forward_noalloc (one copy per GPU
 * the library runs on). 64 MiB: T <= 64 tokens on the K3 layer (d_model 7168, d_ff 1536,
 * 896 experts, top-16) need at most 45 MiB. */
#define K3MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* k3moe_layer_forward for callers that cannot allocate device memory or pass a workspace
 * (code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments without ws / ws_bytes, same kernels and the same results bit
 * for bit. Its scratch is a static device array of K3MOE_NOALLOC_SCRATCH_BYTES per GPU, whose
 * address is looked up (hipGetSymbolAddress) by the first call on each device; the call
 * itself allocates nothing (no hipMalloc / hipFree, and in block mode the shared expert runs
 * in order on `stream` rather than on the library's side stream). K3MOE_EUNSUPPORTED if
 * k3moe_workspace_bytes(dims, T) exceeds the scratch; K3MOE_EHIP if the lookup fails. Every
 * call on a GPU shares that GPU's scratch and nothing in it needs to start zeroed: calls that
 * overlap on one GPU (on different streams or host threads) race, so serialise them, e.g. on
 * one stream. */
K3MOE_API int k3moe_layer_forward_noalloc(const k3moe_dims* dims, int32_t T, const void* x,
                                          int x_dtype, const uint16_t* w_router,
                                          const float* logit_bias,
                                          const k3moe_mx_experts* experts,
                                          const k3moe_block* blk, float* y, uint16_t* y_bf16,
                                          int32_t* topk_ids, float* topk_gates, void* stream);

/* ---- Routed experts beyond HBM: an HBM slot cache over host-resident experts ----------
 * The routed experts are never all kept in fast memory: those a token selects are read on
 * demand from slower storage and multiplied in their packed form, and recently used ones
 * stay cached, least recently used evicted first ("用纯C语言把1.56TB的Kimi K3模型塞进8GB内存
 * 运行", kongchang.com, section 专家权重永不常驻内存; project card "P053
 * FareedKhan-dev/kimi-k3-in-c", core features, expert streaming; "Kimi K3 纯 C 语言 CPU 推理
 * 实战" §3.3, the LRU expert cache). Here a layer's E experts stay in HOST memory and
 * n_slots of them at a time in HBM:
 *   host_experts: the k3moe_mx_experts layout with HOST pointers, all E experts (pinned
 *     memory, e.g. hipHostMalloc, lets the copies run asynchronously; pageable memory works
 *     but each copy then blocks the host);
 *   slot_experts: the same layout with DEVICE pointers and n_slots in place of E;
 *   state: a caller-owned HOST buffer of k3moe_cache_state_bytes() bytes, 8-byte aligned,
 *     set up by k3moe_cache_init(); it maps experts to slots and keeps the host copies of
 *     the routed ids. One state belongs to one (host_experts, slot_experts) pair; calls
 *     that share a state must not overlap.
 * Policy (k3moe_cache_plan): an expert already in a slot keeps it (hit); each missing expert,
 * in order of first appearance among the ids, takes the least recently used slot that the
 * same call does not use (lowest slot index among equals; empty slots first) (miss). */
typedef struct {
  int64_t hits;          /* distinct routed experts found in a slot       */
  int64_t misses;        /* distinct routed experts copied into a slot    */
  int64_t bytes_copied;  /* host -> HBM bytes enqueued for the misses     */
  int32_t distinct;      /* distinct experts of the last call (0 if none) */
} k3moe_cache_stats;

/* Bytes of a state for n_experts experts, n_slots slots (1 <= n_slots <= n_experts) and up
 * to max_ids routed ids (T * top_k) per call; 0 if the arguments are invalid. */
K3MOE_API size_t k3moe_cache_state_bytes(int32_t n_experts, int32_t n_slots, int32_t max_ids);
/* Empty cache (no expert resident). EINVAL: invalid arguments or state not 8-byte aligned;
 * EWORKSPACE: state_bytes too small. */
K3MOE_API int k3moe_cache_init(void* state, size_t state_bytes, int32_t n_experts,
                               int32_t n_slots, int32_t max_ids);
/* Host-side plan for n_ids routed ids (HOST array, each in [0, E)): updates the state and
 * writes slot_ids[n_ids] (the slot of each id) and, per miss, fetch[2 i] = expert and
 * fetch[2 i + 1] = slot (room for 2 * n_slots ints), *n_fetch = misses. EINVAL: an id out of
 * range or a bad state; EUNSUPPORTED: more distinct experts than slots (nothing assigned).
 * No GPU work. */
K3MOE_API int k3moe_cache_plan(void* state, int32_t n_ids, const int32_t* ids,
                               int32_t* slot_ids, int32_t* fetch, int32_t* n_fetch);
/* Cumulative hits, misses and bytes of the state (distinct: that of the last call). */
K3MOE_API int k3moe_cache_stats_get(const void* state, k3moe_cache_stats* out);
/* One MoE layer (no block extras) with the experts in the slot cache: router on `stream`,
 * routed ids copied to the host (this SYNCHRONISES `stream`), plan, host -> HBM copies of
 * the missing experts enqueued on `stream`, slot ids to the device, bucketing by slot, and
 * the routed experts run from the slots. The copies of several missing experts are spread
 * over 4 copy streams per device (non-blocking, default priority, created on first use and
 * kept until the process ends), forked from `stream` and joined back into it by the calling
 * thread's events before the bucketing, so the call's work is complete once `stream` is.
 * y, y_bf16, topk_ids and topk_gates are those of
 * k3moe_layer_forward with all E experts resident, bit for bit. call_stats (nullable, host)
 * receives this call's hits, misses, bytes and distinct count. EUNSUPPORTED: T * top_k
 * above the state's max_ids, top_k above n_slots, or more distinct experts in the batch
 * than slots. ws: k3moe_workspace_bytes(dims, T). */
K3MOE_API int k3moe_layer_forward_cached(const k3moe_dims* dims, int32_t T, const void* x,
                                         int x_dtype, const uint16_t* w_router,
                                         const float* logit_bias,
                                         const k3moe_mx_experts* host_experts,
                                         const k3moe_mx_experts* slot_experts, void* state,
                                         float* y, uint16_t* y_bf16, int32_t* topk_ids,
                                         float* topk_gates, k3moe_cache_stats* call_stats,
                                         void* ws, size_t ws_bytes, void* stream);

/* Diagnostics for live per-kernel timing. Arms a one-shot probe on the calling thread:
 * the next entry-point call that launches kernel `which` records hipEvent_t ev_start on
 * its stream right before that launch and ev_stop right after it, then disarms. The
 * events are created and owned by the caller. which: K3MOE_KERNEL_*. Passing NULL events
 * disarms. Returns K3MOE_EINVAL for an unknown `which`. */
enum { K3MOE_KERNEL_ROUTER = 1, K3MOE_KERNEL_GATE_UP = 2, K3MOE_KERNEL_DOWN = 3 };
K3MOE_API int k3moe_time_next_kernel(int which, void* ev_start, void* ev_stop);

/* Message describing the calling thread's last non-OK status ("" if none). */
K3MOE_API const char* k3moe_last_error(void);

/* Cache policy of the expert weight reads in the grouped (many-token) kernels, process-wide:
 * an expert with fewer than `hot_tokens` tokens in a call reads its weights non-temporally
 * (streamed past the caches), one with more keeps the normal policy, so that the weights of
 * experts that many tokens choose can stay in the caches for their other 64-token tiles and,
 * under skewed routing, for later calls ("Kimi K3 纯 C 语言 CPU 推理实战" §1.3, obstacle 3: keep
 * loaded experts in the last-level cache; §6.2: a small hot set is chosen far more often).
 * 0 <= hot_tokens <= 16 (0: normal policy for every expert); default 16. Results do not
 * depend on it. K3MOE_EINVAL outside the range. k3moe_hot_tokens() returns the setting. */
K3MOE_API int k3moe_set_hot_tokens(int32_t hot_tokens);
K3MOE_API int32_t k3moe_hot_tokens(void);

/* Teardown of what the library keeps between calls: synchronises and destroys, on every
 * device where they exist, the block-mode side stream and the slot cache's copy streams,
 * and destroys the CALLING thread's fork/join events (other threads' events stay until the
 * process ends). Call it when no call into the library is in flight on any thread, before
 * the HIP runtime is torn down (e.g. from an exit handler; the Python binding registers
 * one). Returns K3MOE_OK, or K3MOE_EHIP if a HIP call failed (the rest is still released).
 * Touches no HIP state if the library never created any of these. A later call that needs
 * them creates them again. */
K3MOE_API int k3moe_release(void);

#ifdef __cplusplus
}
#endif
#endif
