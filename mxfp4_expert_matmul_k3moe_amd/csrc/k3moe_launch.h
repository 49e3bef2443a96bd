// k3moe_launch.h — host-side launch wrappers of the gfx950 kernels (internal).
// Every wrapper enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace k3moe {

// Event pair of k3moe_time_next_kernel, set on the calling thread while the probed launch is
// being enqueued. The launcher of a timed kernel passes the events to hipExtLaunchKernel,
// which stamps the kernel's own begin and end (events recorded around the launch would also
// take in the wait for the kernel before it), and marks them used.
struct LaunchTiming {
  hipEvent_t start, stop;
  bool used;
};
extern thread_local LaunchTiming* t_launch_timing;

// kernel<<<grid, block, lds, s>>>(args...), with the pending timing events if there are any.
template <typename... Args, typename F>
inline void launch_timed(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                         Args... args) {
  LaunchTiming* lt = t_launch_timing;
  if (lt && !lt->used) {
    lt->used = true;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, lt->start, lt->stop, 0u, args...);
  } else {
    kernel<<<grid, block, lds, s>>>(args...);
  }
}

// ---- router (router.hip) -------------------------------------------------------
// Rows of W handled per partial-sum chunk of the small-T router.
int router_chunk_rows(int d);
int router_num_chunks(int d);
constexpr int kRouterGemvMaxT = 64;   // above this the tiled fp64 GEMM is used

// part[c][t][e] over 512-row chunks c. With E % 8 == 0 and 16-byte aligned operands: one
// token on the all-loads-in-flight GEMV, 2..9 tokens in groups of 4 sharing the block's
// weights, 10..64 tokens on work items (chunk, 512 columns, 4 tokens) that sum over K inside
// each lane; otherwise the scalar kernel.
hipError_t launch_router_gemv(int T, int d, int E, const void* x, int xf32,
                              const uint16_t* w, double* part, hipStream_t s);
// K chunks of the many-token router (its partial-sum count; at most 8), and the bound
// router_mfma_splits(T) * T <= max(T, min(8 T, router_split_budget(E))).
int router_mfma_splits(int T, int d, int E);
int router_split_budget(int E);
// part[c][t][e] for c < *nsum (set on return), summed in order by route_topk.
hipError_t launch_router_gemm(int T, int d, int E, const void* x, int xf32,
                              const uint16_t* w, double* part, int* nsum, hipStream_t s);
// ---- bucketing (bucket.hip) ----------------------------------------------------
constexpr int kBucketTokens = 64;  // tokens per bucketing block
constexpr int kMfmaTileM = 64;     // tokens per full grouped-GEMM tile
// Grouped-GEMM tiles of an expert with n tokens: one 16- or 32-row tile when n <= 32,
// else ceil(n / 64) tiles of 64 rows (the MFMA work follows the real token count).
__host__ __device__ inline int mfma_tiles_of(int n) {
  return n <= 0 ? 0 : (n <= 32 ? 1 : (n + kMfmaTileM - 1) / kMfmaTileM);
}
struct BucketOut {
  int32_t* offsets;    // [E+1]
  int32_t* rows;       // [P] pair ids by bucket position
  int32_t* act;        // [E] active experts, ascending
  int32_t* n_act;      // [1]
  int32_t* pair_pos;   // [P] bucket position of pair id
  int32_t* pair_exp;   // [P] expert of pair id
  int32_t* mtile_off;  // [E+1] prefix over active experts of mfma_tiles_of(count)
};
// nsum: number of fp64 partial arrays [nsum][T][E] to add (1 = plain logits).
// bucket1 (T == 1 only, may be NULL): also write the single token's bucket.
hipError_t launch_route_topk(int T, int E, int k, const double* part, int nsum,
                             const float* bias, int32_t* ids, float* gates,
                             const BucketOut* bucket1, hipStream_t s);
// Block mode, one token: the RMSNorm of the residual h (into xhat), the router GEMV on it and
// the shared expert's gate/up GEMV (hsh = silu(G xhat) * (U xhat)) in one launch, then the
// top-k with the token's bucket and the shared expert's down GEMV (ssh = D hsh) in a second;
// every value as from the standalone kernels. Needs route_shared_supported (d % 8 == 0,
// d <= 8192, E % 8 == 0, 256 < E <= 4096, 16-byte aligned router weights); gateup_blocks > 0
// caps the shared gate/up blocks.
bool route_shared_supported(int d, int E, int k, const uint16_t* w_router);
hipError_t launch_route_shared(int d, int f, int E, int k, const float* h,
                               const uint16_t* gamma, float eps, float* xhat,
                               const uint16_t* w_router, const float* bias, double* part,
                               const uint16_t* sh_gate, const uint16_t* sh_up,
                               const uint16_t* sh_down, float* hsh, float* ssh, int32_t* ids,
                               float* gates, const BucketOut& bucket1, int gateup_blocks,
                               hipStream_t s);
// Same shapes, packed experts (whose one-token gate/up launch takes the shared down, see
// launch_gateup_decode_packed): the RMSNorm and the router GEMV in one launch, then the top-k
// with the token's bucket and the shared gate/up GEMV (on the stored xhat) in a second.
hipError_t launch_route_norm_shared_gateup(int d, int f, int E, int k, const float* h,
                                           const uint16_t* gamma, float eps, float* xhat,
                                           const uint16_t* w_router, const float* bias,
                                           double* part, const uint16_t* sh_gate,
                                           const uint16_t* sh_up, float* hsh, int32_t* ids,
                                           float* gates, const BucketOut& bucket1,
                                           hipStream_t s);
hipError_t launch_bucket(int T, int E, int k, const int32_t* ids, const BucketOut& o,
                         uint32_t* hist, uint32_t* base, uint64_t* masks, hipStream_t s);
// From caller-supplied offsets/rows (k3moe_expert_ffn): act, n_act, pair_pos, pair_exp.
hipError_t launch_pairs_from_bucket(int T, int E, int k, const int32_t* offsets,
                                    const int32_t* rows, const BucketOut& o, hipStream_t s);

// ---- expert FFN, GEMV family (ffn_gemv.hip) -----------------------------------------
struct MxPtrs {
  const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
};
bool gemv_shape_supported(int d, int f);
// The T == 1 down kernel puts one lane group per slot in one block.
bool down_fused_supported(int f, int k);
hipError_t launch_gateup_gemv(int T, int d, int f, int E, int k, const void* x, int xf32,
                              const MxPtrs& w, const int32_t* offsets, const int32_t* rows,
                              const int32_t* act, const int32_t* n_act, int max_act,
                              float* h, hipStream_t s);
// T == 1, persistent decode kernels (grid sized from the CU count); blocks_per_cu <= 0
// picks 4 resident blocks per CU. Needs gateup_decode_supported(d): at most 8 MXFP4 blocks
// of a row per lane (else hipErrorInvalidValue; the GEMV kernel above takes such rows).
bool gateup_decode_supported(int d);
hipError_t launch_gateup_decode(int d, int f, int k, const void* x, int xf32, const MxPtrs& w,
                                const int32_t* offsets, const int32_t* act, const int32_t* n_act,
                                float* h, int n_cu, hipStream_t s, int blocks_per_cu = 0);
// rows_per_block == 0: the MFMA kernel below when the shape and a 4-byte aligned down_s
// allow it, else the fp32-FMA kernel with about two blocks per CU; rows_per_block > 0
// forces the fp32-FMA kernel with that many rows per block; rows_per_step in {2, 4, 8}.
hipError_t launch_down_decode(int d, int f, int k, const MxPtrs& w, const float* h,
                              const int32_t* pair_pos, const int32_t* pair_exp,
                              const float* gates, const float* resid, const float* shared,
                              float* y, uint16_t* y_bf16, int n_cu, hipStream_t s,
                              int rows_per_block = 0, int rows_per_step = 4);
// T == 1 down projection + ordered combine on the block-scaled MFMA (ffn_mfma.hip): one
// persistent block per CU walking its equal share of output rows in 16-row tiles, one wave
// per slot; needs d % 16 == 0, f % 128 == 0, f <= 1536 and k <= 16. launch_down_decode takes
// it whenever the shape allows. packed: down in the packed tile layout.
bool down_decode_mfma_supported(int d, int f, int k);
hipError_t launch_down_decode_mfma(int d, int f, int k, const MxPtrs& w, const float* h,
                                   const int32_t* pair_pos, const int32_t* pair_exp,
                                   const float* gates, const float* resid, const float* shared,
                                   float* y, uint16_t* y_bf16, int n_cu, hipStream_t s,
                                   bool packed = false);
// One token, packed tile layout (d % 1024 == 0, d <= 16384, f % 16 == 0): h = silu(G x) * (U x)
// of every slot as fp32 into h [k][f] at the slot's bucket position, on the block-scaled MFMA
// (ffn_mfma.hip; the token split into E4M3 terms per 32-element block inside the kernel); one
// block per (slot, 16-row tile), one wave per 8-step K chunk. x is bf16 (xf32 == 0) or fp32.
// shared (nullable, block mode): the same launch also runs the shared expert's down GEMV,
// out[r] = W[r] . hsh for the d rows of the bf16 [d][f] W, in blocks after the expert ones.
struct SharedDown {
  const float* hsh;
  const uint16_t* w;
  float* out;
};
hipError_t launch_gateup_decode_packed(int d, int f, int k, const void* x, int xf32,
                                       const MxPtrs& w, const int32_t* pair_pos,
                                       const int32_t* pair_exp, float* h, hipStream_t s,
                                       const SharedDown* shared = nullptr);
// Any T: per-expert down projection into z [P][d] (pair-indexed).
hipError_t launch_down_gemv(int T, int d, int f, int E, int k, const MxPtrs& w,
                            const float* h, const int32_t* offsets, const int32_t* rows,
                            const int32_t* act, const int32_t* n_act, int max_act, float* z,
                            hipStream_t s);
// y[t] = (resid + shared) + sum_slot g * z[t*k+slot], slot order.
hipError_t launch_combine(int T, int d, int k, const float* z, const float* gates,
                          const int32_t* pair_pos, const float* resid, const float* shared,
                          float* y, uint16_t* y_bf16, hipStream_t s);

// ---- expert FFN, grouped GEMM on bf16 MFMA (ffn_mfma.hip) ---------------------------
// Upper bound on the number of M tiles over all active experts.
int mfma_mtiles_bound(int T, int E, int k);
bool mfma_shape_supported(int d, int f);
// h = silu(G x) * (U x) for every (expert, token) pair, bucket order, as three E4M3 terms
// h8 [P][3][f] with their E8M0 scales hs8 [P][3][f/32] (one per term and 32-block); x8
// [T][2][d] and xs8 [T][2] receive the tokens' own FP8 terms on the way.
// packed: G and U in the packed tile layout (pack.hip; needs d % 1024 == 0, f % 16 == 0).
hipError_t launch_gateup_mfma(int T, int d, int f, int E, int k, const uint16_t* x,
                              const MxPtrs& w, const int32_t* offsets, const int32_t* rows,
                              const int32_t* act, const int32_t* n_act,
                              const int32_t* mtile_off, uint8_t* h8, uint8_t* hs8, uint8_t* x8,
                              uint8_t* xs8, hipStream_t s, bool packed = false);
// Shapes the packed-layout grouped GEMMs take (d: whole 8-step scale chunks; f: the down
// kernel's scale groups).
bool packed_shape_supported(int d, int f);
// Grouped GEMMs: experts with fewer than n tokens in a call read their weights
// non-temporally, the others with the normal cache policy (0 <= n <= 16; default 16).
// Returns false (and changes nothing) for n outside that range.
bool set_hot_tokens(int n);
int hot_tokens();
// z (fp32 [P][d], pair-indexed) = D h from the three terms of h; packed: D in the packed tile
// layout (weights streamed per M tile, each tile step one 1-KB DMA).
hipError_t launch_down_mfma(int T, int d, int f, int E, int k, const MxPtrs& w,
                            const uint8_t* h8, const uint8_t* hs8, const int32_t* offsets,
                            const int32_t* rows, const int32_t* act, const int32_t* n_act,
                            const int32_t* mtile_off, float* z, hipStream_t s,
                            bool packed = false);

// ---- packed tile layout (pack.hip) ----------------------------------------------------
// Bytes of the packed scales of one [R][K] matrix (the packed codes take R K / 2, as before).
size_t packed_scale_bytes(int R, int K);
// n_mat stacked [R][K] matrices (codes q, scales s) -> packed codes pq and scales ps.
hipError_t launch_pack_matrix(int R, int K, int n_mat, const uint8_t* q, const uint8_t* s,
                              uint8_t* pq, uint8_t* ps, hipStream_t st);

// ---- block extras (block.hip) ---------------------------------------------------------
hipError_t launch_rmsnorm(int T, int d, const float* h, const uint16_t* gamma, float eps,
                          float* xhat, hipStream_t s);
// Dense bf16 SwiGLU: out [T][d] = Wd (silu(Wg x) * (Wu x)); hbuf [T][f] scratch. Each GEMV
// runs on at most max_blocks blocks (0: one per row group of 4 waves).
hipError_t launch_dense_swiglu(int T, int d, int f, const float* x, const uint16_t* wg,
                               const uint16_t* wu, const uint16_t* wd, float* hbuf,
                               float* out, hipStream_t s, int max_blocks = 0);

}  // namespace k3moe
