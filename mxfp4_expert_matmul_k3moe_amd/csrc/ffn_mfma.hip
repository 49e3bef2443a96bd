// ffn_mfma.hip — grouped expert GEMMs on the gfx950 block-scaled MFMA for many tokens per
// expert (prefill, batched decode).
//
// Each tile is up to 64 tokens of one expert (its bucket rows; experts with at most 16 or
// 32 tokens take a 16- or 32-row tile) times a slice of that expert's weight rows. Both
// GEMMs run on v_mfma_scale_f32_16x16x128_f8f6f4 with the MXFP4 weights as its FP4
// operand exactly as stored (a lane's 16 bytes are one 32-element block of its row, the
// block's E8M0 byte is that lane's scale) and the activations as its FP8 operand, split
// exactly enough into E4M3 terms that each carry their own E8M0 scales:
//  - gate/up: the token as two terms with one scale per term row (exact for bf16 x to
//    about 2^-22 of the row maximum); h = silu(G x) * (U x) leaves the epilogue as three
//    terms with one scale per term and 32-element block of h;
//  - down: z = D h from the three terms, fp32, one row per (token, slot) pair, combined
//    later in slot order.
// Every term is one more MFMA into the same fp32 accumulator; no instruction decodes a
// weight. K is walked in steps of 128 (4 scale blocks). Source of the form: "Kimi K3 纯
// C 语言 CPU 推理实战" (chenxutan.com/d/5901.html) §1.2, §2.3.
#include <atomic>
#include <type_traits>
#include <utility>

#include "block_dev.h"
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = kMfmaTileM;     // 64 tokens per full tile
constexpr int BK = 128;            // K per step (4 MXFP4 blocks per weight row)
constexpr int kWaves = 8;          // 512 threads: two waves per SIMD, one block per CU
constexpr int NT = 4;              // 16-wide N tiles per wave
constexpr int kLdsBytes = 160 * 1024;
constexpr int kBStage = kWaves * NT * 1024;  // weight blocks of one step: 16 B per lane per tile
constexpr int kSStage = kWaves * 256;        // per-step scale words: 4 B per lane
constexpr int kSGroup = kWaves * 1024;       // scale groups: 16 B per lane = 4 steps of scales
// register-fed gate/up tiles (mx_gateup_tile_rw)
constexpr int kWRing = 4;       // weight steps held per wave: the current one and 3 ahead
constexpr int kTokStages = 4;   // token stages in LDS
constexpr int kScaleSteps = 8;  // K steps per scale chunk (32 bytes of a row)
// Cache policy of the weight reads of one expert tile. An expert with fewer than hot_tokens
// tokens in the call reads its weights non-temporally (one pass, nothing to keep); one with
// more keeps the normal policy, so that its weights can stay cached for its other M tiles and,
// under skewed routing, for the next call that routes to it again ("Kimi K3 纯 C 语言 CPU
// 推理实战" §1.3, obstacle 3, and §6.2: a small set of hot experts is chosen far more often
// than the rest, and loaded experts are worth keeping in the last-level cache).
// The threshold is a launch argument (set_hot_tokens), at most kHotTokensMax = 16 so that only
// single-subtile experts (at most 16 tokens) can be cold; the default is 16.
constexpr int kHotTokensMax = 16;
constexpr int kCpNormal = 0, kCpStream = 2;  // load cache-policy bits: normal, non-temporal
std::atomic<int> g_hot_tokens{kHotTokensMax};
static_assert(kTokStages - 1 == 3, "the last scale chunk of the K loop peels three steps");

// Gate/up on the gfx950 block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): the MXFP4
// weights are the FP4 operand as stored (a lane's 16 bytes = one 32-element block of its
// row, with that block's E8M0 scale), the token is the FP8 operand as two E4M3 terms
// x = hi * 2^s_hi + lo * 2^s_lo (scales per token row), multiplied in two MFMAs into one
// fp32 accumulator. No weight decoding instructions at all. Per stage in LDS:
// [A: MT x 2 terms x 2 halves of 1 KB][weights: kBStage] (+ per-step scale words).
template <int MT, bool SG4>
struct MxPipe {
  static constexpr int ABLK = MT * 4;  // 1-KB token blocks: [m][term][half]
  static constexpr int ABYTES = ABLK * 1024;
  static constexpr int BYTES = ABYTES + kBStage + (SG4 ? 0 : kSStage);
  static constexpr int RING = SG4 ? 2 * kSGroup : 0;
  static constexpr int S0 = (kLdsBytes - RING) / BYTES;
  static constexpr int S = S0 < 4 ? S0 : 4;
  static_assert(S >= 2, "pipeline needs two stages");
};

// Same, with the weight scales held in registers; LDS keeps only a 2-KB staging slot per
// wave through which the next scale chunk passes.
constexpr int kScaleStage = 2048;
template <int MT>
struct MxPipeR {
  static constexpr int ABYTES = MT * 4 * 1024;
  static constexpr int BYTES = ABYTES + kBStage;
  static constexpr int S0 = (kLdsBytes - kWaves * kScaleStage) / BYTES;
  static constexpr int S = S0 < 4 ? S0 : 4;
  static_assert(S >= 2, "pipeline needs two stages");
};

// Active expert owning logical block L (blocks of expert a start at mtile_off[a] * nb).
__device__ __forceinline__ int tile_expert_blocks(const int32_t* mtile_off, int n_act, int nb,
                                                  int L) {
  int lo = 0, hi = n_act - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mtile_off[mid] * nb <= L) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Asynchronous global -> LDS copies: 16 (or 4) bytes per lane, lane l writes dst + 16 l
// (or dst + 4 l). dst must be the same for the whole wave.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
template <int CP>
__device__ __forceinline__ void dma16p(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, CP);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations are outstanding. The
// compiler does not order LDS reads after the DMA writes they depend on, so the pipeline
// places these waits itself; the memory clobber keeps LDS reads below them.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads (which would wait for
// every DMA in flight). Each wave first waits for its own DMA of the stage it is about to
// read (wait_vm); LDS reads of the previous stage have all been consumed by MFMAs before a
// wave reaches the barrier. The empty asm statements keep the compiler from moving memory
// operations across it.
// Same with a wave-uniform count n < 32 (one scalar branch to the matching immediate).
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
#define K3_W(N) \
  case N:       \
    wait_vm<N>(); \
    break;
    K3_W(0) K3_W(1) K3_W(2) K3_W(3) K3_W(4) K3_W(5) K3_W(6) K3_W(7) K3_W(8) K3_W(9) K3_W(10)
    K3_W(11) K3_W(12) K3_W(13) K3_W(14) K3_W(15) K3_W(16) K3_W(17) K3_W(18) K3_W(19) K3_W(20)
    K3_W(21) K3_W(22) K3_W(23) K3_W(24) K3_W(25) K3_W(26) K3_W(27) K3_W(28) K3_W(29) K3_W(30)
#undef K3_W
    default:
      wait_vm<0>();
      break;
  }
}

// s_waitcnt vmcnt(N) (other counters left alone) as the builtin, so the compiler's own wait
// insertion knows which vector-memory results it guarantees.
template <int N>
__device__ __forceinline__ void wait_vm_known() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct MfmaArgs {
  int T, d, f, k;
  const uint8_t* x8;      // gate/up: x as fp8 E4M3 terms [T][2][d] (hi, lo)
  const uint8_t* xs8;     // gate/up: E8M0 scale of each term row [T][2]
  const uint8_t *q0, *s0, *q1, *s1;  // gate/up: G and U; down: D (q1 unused)
  const int32_t *offsets, *rows, *act, *n_act, *mtile_off;
  int nblk_n;
  int packed;    // weights in the packed tile layout (pack.hip)
  uint8_t* h8;   // h as three E4M3 terms [P][3][f], bucket order (gate/up out, down in)
  uint8_t* hs8;  // their E8M0 scales [P][3][f/32], one per term and 32-element block
  float* z_out;  // down output
  int hot_tokens;  // experts with fewer tokens read their weights non-temporally
};


// OCP E4M3 code of v (round to nearest even) and the value of a code.
__device__ __forceinline__ int e4m3_code(float v) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFF;
}
__device__ __forceinline__ float e4m3_value(int q) { return __builtin_amdgcn_cvt_f32_fp8(q, 0); }
// Exponent e putting m in [128, 256); kExpZero for m == 0, kExpBad for a non-finite m.
constexpr int kExpZero = -0x7fffffff, kExpBad = 0x7fffffff;
__device__ __forceinline__ int top_exp(float m) {
  if (!__builtin_isfinite(m)) return kExpBad;
  if (m == 0.0f) return kExpZero;
  return ilogbf(m) - 7;
}

// Gate/up epilogue: h = silu(gate) * up of a lane's 8 values, stored as three E4M3 terms
// with one E8M0 scale per term and 32-element block of h. A wave's block of j holds the
// values of the 4 lanes ln + 16 g' (2 tiles x 4 rows each), so each block maximum is two
// lane exchanges. Term t: 2^s_t puts the block maximum of what is left in [128, 256), the
// values are rounded to E4M3 and the exact remainder goes to the next term (arithmetic in
// the domain scaled by the first term). Three terms carry h to about 2^-13 of the block
// maximum (rel. L2 error of D h about 2e-5 on SwiGLU-like h, against 2e-3 for one bf16
// rounding). A non-finite block maximum gives scale bytes 255 (NaN).
template <int MT>
__device__ __forceinline__ void store_h_terms(const MfmaArgs& a, const f32x4 (&acc)[MT][NT], int p0,
                                              int pn, int nb, int wave, int ln, int g) {
  const int F = a.f, FB = F >> 5;
  const int jb = nb * 256 + wave * 32;  // first j of this wave's block (f % 32 == 0)
  if (jb >= F) return;                 // wave-uniform
  auto bmax = [](float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
  };
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float y[8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[4 * nt + r] = silu_f32(acc[m][nt][r]) * acc[m][nt + 2][r];
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(y[i]));
    mx = bmax(mx);
    const int e0 = top_exp(mx);
    const bool bad = e0 == kExpBad;
    const int s0 = bad ? 255 : min(max(e0 + 127, 0), 254);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = ldexpf(y[i], 127 - s0);  // exact: maximum below 256
    uint32_t w[3][2];
    int sc[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      int er = 0;  // exponent of term t relative to term 0
      if (t == 0) {
        sc[0] = s0;
      } else {
        float rm = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) rm = fmaxf(rm, fabsf(y[i]));
        rm = bmax(rm);
        const int ex = top_exp(rm);
        sc[t] = bad ? 255 : min(max(s0 + max(ex, -300), 0), 254);
        er = sc[t] - s0;
      }
      w[t][0] = w[t][1] = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = e4m3_code(ldexpf(y[i], -er));
        y[i] -= ldexpf(e4m3_value(q), er);
        w[t][i >> 2] |= (uint32_t)q << (8 * (i & 3));
      }
    }
    const int row = 16 * m + ln;
    if (row < pn) {
      const size_t base = (size_t)(p0 + row) * 3;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        uint8_t* dst = a.h8 + (base + t) * F + jb + 4 * g;
        *reinterpret_cast<uint32_t*>(dst) = w[t][0];
        *reinterpret_cast<uint32_t*>(dst + 16) = w[t][1];
        if (g == 0) a.hs8[(base + t) * FB + (jb >> 5)] = (uint8_t)sc[t];
      }
    }
  }
}

// Block -> work: blocks are spread over the 8 XCDs round-robin by the hardware; logical
// work index L is laid out so that the blocks one XCD receives are consecutive in L,
// and L runs expert-major, then N slice, then M tile, so the M tiles of one weight slice
// run back to back on one XCD and find that slice in its L2.
template <int MT, bool SG4>
__device__ __forceinline__ void mx_gateup_tile(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                               int pn, int nb);
template <int MT>
__device__ __forceinline__ void mx_gateup_tile_sr(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                                  int pn, int nb);
template <int MT, bool PK, int CP = kCpNormal>
__device__ __forceinline__ void mx_gateup_tile_rw(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                                  int pn, int nb);
template <int MT, int NK, int CP>
__device__ __forceinline__ void mx_down_tile_rw(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                                int pn, int nb);
// f(integral_constant<int, I>) for I = 0, 1, ... in order (a compile-time unrolled loop)
template <int... I, class F>
__device__ __forceinline__ void for_each_const(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int MT, bool SG4, bool PK = false, int CP = kCpNormal>
__device__ __forceinline__ void mx_down_tile(const MfmaArgs& a, uint8_t* lds, int e, int p0, int pn,
                                             int nb);

template <bool GATEUP>
__global__ __launch_bounds__(512) void mfma_ffn_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  const int n_act = *a.n_act;
  if (n_act <= 0) return;
  const int N = a.mtile_off[n_act] * a.nblk_n;  // blocks with work
  const int b = blockIdx.x;
  if (b >= N) return;
  const int x = b & 7, slot = b >> 3;
  int L = slot;
  for (int x2 = 0; x2 < x; ++x2) L += (N - x2 + 7) >> 3;
  const int ai = tile_expert_blocks(a.mtile_off, n_act, a.nblk_n, L);
  const int e = a.act[ai];
  const int P = a.T * a.k;
  const int pe0 = min(max(a.offsets[e], 0), P), pe1 = min(max(a.offsets[e + 1], pe0), P);
  const int cnt = pe1 - pe0;
  const int mt_a = a.mtile_off[ai + 1] - a.mtile_off[ai];
  const int Lr = L - a.mtile_off[ai] * a.nblk_n;
  const int nb = Lr / mt_a, mloc = Lr - nb * mt_a;
  const int p0 = pe0 + mloc * BM;
  const int pn = max(0, min(BM, pe1 - p0));
  if (pn <= 0) return;
  // 16-byte scale groups need K a multiple of 512 and 16-byte aligned scale arrays
  const bool sg4 = ((GATEUP ? a.d : a.f) % (4 * BK)) == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.s0) |
                     reinterpret_cast<uintptr_t>(GATEUP ? a.s1 : a.s0)) & 15u) == 0;
  if (GATEUP) {
    // (hot_tokens <= 16: only single-subtile experts can be cold)
    if (a.packed) {
      if (cnt < a.hot_tokens) mx_gateup_tile_rw<1, true, kCpStream>(a, lds, e, p0, pn, nb);
      else if (cnt <= 16) mx_gateup_tile_rw<1, true>(a, lds, e, p0, pn, nb);
      else if (cnt <= 32) mx_gateup_tile_rw<2, true>(a, lds, e, p0, pn, nb);
      else mx_gateup_tile_rw<4, true>(a, lds, e, p0, pn, nb);
    } else if (sg4 && a.d % (kScaleSteps * BK) == 0) {
      if (cnt < a.hot_tokens) mx_gateup_tile_rw<1, false, kCpStream>(a, lds, e, p0, pn, nb);
      else if (cnt <= 16) mx_gateup_tile_rw<1, false>(a, lds, e, p0, pn, nb);
      else if (cnt <= 32) mx_gateup_tile_rw<2, false>(a, lds, e, p0, pn, nb);
      else mx_gateup_tile_rw<4, false>(a, lds, e, p0, pn, nb);
    } else if (sg4) {
      if (cnt <= 16) mx_gateup_tile_sr<1>(a, lds, e, p0, pn, nb);
      else if (cnt <= 32) mx_gateup_tile_sr<2>(a, lds, e, p0, pn, nb);
      else mx_gateup_tile_sr<4>(a, lds, e, p0, pn, nb);
    } else {
      if (cnt <= 16) mx_gateup_tile<1, false>(a, lds, e, p0, pn, nb);
      else if (cnt <= 32) mx_gateup_tile<2, false>(a, lds, e, p0, pn, nb);
      else mx_gateup_tile<4, false>(a, lds, e, p0, pn, nb);
    }
    return;
  }
  if (a.packed && a.f % 512 == 0 && a.f <= 16 * BK) {
    // register-fed weights, compile-time K steps (f = 512, 1024, 1536 or 2048)
    switch (a.f / BK) {
#define K3_DRW(NKV)                                                                     \
  case NKV:                                                                              \
    if (cnt < a.hot_tokens) mx_down_tile_rw<1, NKV, kCpStream>(a, lds, e, p0, pn, nb);   \
    else if (cnt <= 16) mx_down_tile_rw<1, NKV, kCpNormal>(a, lds, e, p0, pn, nb);       \
    else if (cnt <= 32) mx_down_tile_rw<2, NKV, kCpNormal>(a, lds, e, p0, pn, nb);       \
    else mx_down_tile_rw<4, NKV, kCpNormal>(a, lds, e, p0, pn, nb);                      \
    break;
      K3_DRW(4) K3_DRW(8) K3_DRW(12) K3_DRW(16)
#undef K3_DRW
      default:
        break;
    }
  } else if (a.packed) {
    if (cnt < a.hot_tokens) mx_down_tile<1, true, true, kCpStream>(a, lds, e, p0, pn, nb);
    else if (cnt <= 16) mx_down_tile<1, true, true>(a, lds, e, p0, pn, nb);
    else if (cnt <= 32) mx_down_tile<2, true, true>(a, lds, e, p0, pn, nb);
    else mx_down_tile<4, true, true>(a, lds, e, p0, pn, nb);
  } else if (sg4) {
    if (cnt < a.hot_tokens) mx_down_tile<1, true, false, kCpStream>(a, lds, e, p0, pn, nb);
    else if (cnt <= 16) mx_down_tile<1, true>(a, lds, e, p0, pn, nb);
    else if (cnt <= 32) mx_down_tile<2, true>(a, lds, e, p0, pn, nb);
    else mx_down_tile<4, true>(a, lds, e, p0, pn, nb);
  } else {
    if (cnt <= 16) mx_down_tile<1, false>(a, lds, e, p0, pn, nb);
    else if (cnt <= 32) mx_down_tile<2, false>(a, lds, e, p0, pn, nb);
    else mx_down_tile<4, false>(a, lds, e, p0, pn, nb);
  }
}

template <int MT, bool SG4>
__device__ __forceinline__ void mx_gateup_tile(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                               int pn, int nb) {
  using PP = MxPipe<MT, SG4>;
  constexpr int S = PP::S, SB = PP::BYTES, AB = PP::ABYTES;
  const int P = a.T * a.k;
  const int K = a.d, NR = a.f, KB = K >> 5;
  const size_t rq = (size_t)(K >> 1);
  const int nk = K / BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, g = lane >> 4;

  // token of tile row 16 m + ln (rows past the tile's end repeat its last row)
  auto tok_of = [&](int m) {
    const int r = min(16 * m + ln, pn - 1);
    const int pair = a.rows[p0 + r];
    return (pair >= 0 && pair < P) ? pair / a.k : 0;
  };
  // A loads: wave w < 2 MT stages term (w & 1) of the tokens of M subtile w >> 1, in two
  // halves; lane (ln, g) takes the 16 bytes the FP8 operand layout puts in its registers:
  // k = 32 (g >> 1) + 16 (g & 1) (+ 64 for the second half) within the step
  const bool has_a = wave < 2 * MT;
  const int am = (wave >> 1) < MT ? (wave >> 1) : 0, at = wave & 1;
  const uint8_t* asrc =
      a.x8 + ((size_t)tok_of(am) * 2 + at) * K + 32 * (g >> 1) + 16 * (g & 1);
  // per-lane E8M0 scales of the token terms of each M subtile (whole-row scales)
  int sxh[MT], sxl[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = tok_of(m);
    sxh[m] = a.xs8[2 * t];
    sxl[m] = a.xs8[2 * t + 1];
  }

  // weight rows as in the bf16 path: lane (ln, g) of tile nt reads block 4 ks + g of row rB
  const uint8_t* bsrc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int r = nb * 256 + wave * 32 + (nt & 1) * 16 + ln;
    const uint8_t* qb = (nt < 2) ? a.q0 : a.q1;
    r = min(r, NR - 1);
    bsrc[nt] = qb + ((size_t)e * NR + r) * rq + 16 * g;
  }
  const uint8_t* ssrc;
  {
    const int snt = lane >> 4, sln = lane & 15;
    int r = nb * 256 + wave * 32 + (snt & 1) * 16 + sln;
    const uint8_t* sb = (snt < 2) ? a.s0 : a.s1;
    r = min(r, NR - 1);
    ssrc = sb + ((size_t)e * NR + r) * KB;
  }
  uint8_t* const sring = lds + S * SB;
  auto issue = [&](int ks, int slotno) {
    uint8_t* st = lds + slotno * SB;
    if (has_a) {
      const int o = (am * 2 + at) * 2;
      dma16(asrc + (size_t)ks * BK, st + o * 1024);
      dma16(asrc + (size_t)ks * BK + 64, st + (o + 1) * 1024);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      dma16(bsrc[nt] + (size_t)ks * 64, st + AB + (wave * NT + nt) * 1024);
    if (SG4) {
      if ((ks & 3) == 0) dma16(ssrc + ks * 4, sring + ((ks >> 2) & 1) * kSGroup + wave * 1024);
    } else {
      dma4(ssrc + ks * 4, st + AB + kBStage + wave * 256);
    }
  };
  constexpr int OPS_A = 2 + NT + (SG4 ? 0 : 1);
  constexpr int OPS_NOA = NT + (SG4 ? 0 : 1);
  auto wait_stage = [&](int ks) {
    if (ks + S - 2 >= nk) {
      wait_vm<0>();
      return;
    }
    const int extra = SG4 ? ((ks + S - 2) >> 2) - (ks >> 2) : 0;
    if (has_a) {
      if (extra) wait_vm<(S - 2) * OPS_A + 1>();
      else wait_vm<(S - 2) * OPS_A>();
    } else {
      if (extra) wait_vm<(S - 2) * OPS_NOA + 1>();
      else wait_vm<(S - 2) * OPS_NOA>();
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);

  for (int ks = 0; ks < nk; ++ks) {
    wait_stage(ks);
    barrier_no_fence();
    if (ks + S - 1 < nk) issue(ks + S - 1, (ks + S - 1) % S);

    const uint8_t* st = lds + (ks % S) * SB;
    i32x8 wop[NT];
    int wsc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(st + AB + (wave * NT + nt) * 1024 + lane * 16);
      wop[nt] = i32x8{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
      wsc[nt] = SG4 ? sring[((ks >> 2) & 1) * kSGroup + wave * 1024 + 16 * (nt * 16 + ln) + 4 * (ks & 3) + g]
                    : st[AB + kBStage + wave * 256 + 4 * (nt * 16 + ln) + g];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint8_t* xh = st + ((m * 2 + 0) * 2) * 1024 + lane * 16;
      const uint8_t* xl = st + ((m * 2 + 1) * 2) * 1024 + lane * 16;
      const u32x4 h0 = *reinterpret_cast<const u32x4*>(xh), h1 = *reinterpret_cast<const u32x4*>(xh + 1024);
      const u32x4 l0 = *reinterpret_cast<const u32x4*>(xl), l1 = *reinterpret_cast<const u32x4*>(xl + 1024);
      const i32x8 xhi = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      const i32x8 xlo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xhi, acc[m][nt], 4, 0, 0,
                                                                       wsc[nt], 0, sxh[m]);
        acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xlo, acc[m][nt], 4, 0, 0,
                                                                       wsc[nt], 0, sxl[m]);
      }
    }
  }

  // epilogue: lane (ln, g) holds weight rows 4 g .. 4 g + 3 of each 16-row tile, token ln
  store_h_terms<MT>(a, acc, p0, pn, nb, wave, ln, g);
}

// Gate/up tile for K % 512 == 0 with the weight scales kept in registers. Fetching a
// 16-byte scale group every 4 K steps touches each 128-byte scale line eight times, far
// enough apart that the line has left L2 in between; here the scales move 32 K steps
// (128 blocks, 128 bytes per row) at a time, so each line is fetched once. Lane (ln, g) of
// tile nt holds bytes [32 g, 32 g + 32) of its row's chunk; the 4 bytes of step j are
// dword j & 7 of lane (ln, j >> 3), fetched with one ds_bpermute, and lane g keeps byte g.
// The next chunk comes in during the current one, one tile per 8 K steps: a DMA into the
// wave's staging slot, read into registers S steps later, once the pipeline's own wait has
// covered it.
template <int MT>
__device__ __forceinline__ void mx_gateup_tile_sr(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                                  int pn, int nb) {
  using PP = MxPipeR<MT>;
  constexpr int S = PP::S, SB = PP::BYTES, AB = PP::ABYTES;
  static_assert(S <= 7, "scale read-back must land in the same 8-step group");
  const int P = a.T * a.k;
  const int K = a.d, NR = a.f, KB = K >> 5;
  const size_t rq = (size_t)(K >> 1);
  const int nk = K / BK;            // multiple of 4
  const int nch = (KB + 127) >> 7;  // scale chunks of 32 K steps
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, g = lane >> 4;

  auto tok_of = [&](int m) {
    const int r = min(16 * m + ln, pn - 1);
    const int pair = a.rows[p0 + r];
    return (pair >= 0 && pair < P) ? pair / a.k : 0;
  };
  const bool has_a = wave < 2 * MT;
  const int am = (wave >> 1) < MT ? (wave >> 1) : 0, at = wave & 1;
  const uint8_t* asrc =
      a.x8 + ((size_t)tok_of(am) * 2 + at) * K + 32 * (g >> 1) + 16 * (g & 1);
  int sxh[MT], sxl[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = tok_of(m);
    sxh[m] = a.xs8[2 * t];
    sxl[m] = a.xs8[2 * t + 1];
  }
  auto row_of = [&](int nt) { return min(nb * 256 + wave * 32 + (nt & 1) * 16 + ln, NR - 1); };
  const uint8_t* bsrc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    bsrc[nt] = ((nt < 2) ? a.q0 : a.q1) + ((size_t)e * NR + row_of(nt)) * rq + 16 * g;
  // this lane's 16-byte piece h of tile nt's scale chunk c (pieces past the row: offset 0)
  auto spiece = [&](int nt, int c, int h) {
    const int off = 128 * c + 32 * g + 16 * h;
    return ((nt < 2) ? a.s0 : a.s1) + ((size_t)e * NR + row_of(nt)) * KB + (off < KB ? off : 0);
  };
  uint8_t* const stg = lds + S * SB + wave * kScaleStage;
  auto issue = [&](int ks, int slotno) {
    uint8_t* st = lds + slotno * SB;
    if (has_a) {
      const int o = (am * 2 + at) * 2;
      dma16(asrc + (size_t)ks * BK, st + o * 1024);
      dma16(asrc + (size_t)ks * BK + 64, st + (o + 1) * 1024);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      dma16(bsrc[nt] + (size_t)ks * 64, st + AB + (wave * NT + nt) * 1024);
  };
  constexpr int OPS_A = 2 + NT, OPS_NOA = NT, OPS_SC = 2;
  // stage ks complete; `late`: a scale DMA was issued after stage ks (it is newer)
  auto wait_stage = [&](int ks, bool late) {
    if (ks + S - 2 >= nk) {
      wait_vm<0>();
      return;
    }
    if (has_a) {
      if (late) wait_vm<(S - 2) * OPS_A + OPS_SC>();
      else wait_vm<(S - 2) * OPS_A>();
    } else {
      if (late) wait_vm<(S - 2) * OPS_NOA + OPS_SC>();
      else wait_vm<(S - 2) * OPS_NOA>();
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // chunk 0 straight into registers, issued ahead of the prologue; the asm below makes the
  // compiler wait for it there (exact count) rather than inside the loop
  u32x4 scur[NT][2], snxt[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int h = 0; h < 2; ++h) scur[nt][h] = *reinterpret_cast<const u32x4*>(spiece(nt, 0, h));
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(scur[nt][h]));

  for (int ks0 = 0; ks0 < nk; ks0 += 8) {
    const int q = (ks0 & 31) >> 3;  // group within the chunk = tile whose next chunk moves
    const int c = ks0 >> 5;
    if (q == 0 && c > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        scur[nt][0] = snxt[nt][0];
        scur[nt][1] = snxt[nt][1];
      }
    }
    const bool pf = c + 1 < nch;  // whole chunk ahead of us: all 8 steps of the group exist
    const int baddr = (ln + 16 * q) * 4;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ks = ks0 + u;
      if (ks < nk) {
        wait_stage(ks, pf && u >= 1 && u <= S - 1);
        barrier_no_fence();
        if (ks + S - 1 < nk) issue(ks + S - 1, (ks + S - 1) % S);
        if (pf && u == 0) {
          // the previous tile's read-back (u == S of the last group) has returned
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          dma16(spiece(q, c + 1, 0), stg);
          dma16(spiece(q, c + 1, 1), stg + 1024);
        }
        if (pf && u == S) {
          const u32x4 v0 = *reinterpret_cast<const u32x4*>(stg + lane * 16);
          const u32x4 v1 = *reinterpret_cast<const u32x4*>(stg + 1024 + lane * 16);
          switch (q) {
            case 0: snxt[0][0] = v0; snxt[0][1] = v1; break;
            case 1: snxt[1][0] = v0; snxt[1][1] = v1; break;
            case 2: snxt[2][0] = v0; snxt[2][1] = v1; break;
            default: snxt[3][0] = v0; snxt[3][1] = v1; break;
          }
        }

        const uint8_t* st = lds + (ks % S) * SB;
        i32x8 wop[NT];
        int wsc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(st + AB + (wave * NT + nt) * 1024 + lane * 16);
          wop[nt] = i32x8{(int)qv[0], (int)qv[1], (int)qv[2], (int)qv[3], 0, 0, 0, 0};
          wsc[nt] = (int)((uint32_t)__builtin_amdgcn_ds_bpermute(baddr, (int)scur[nt][u >> 2][u & 3]) >> (8 * g));
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint8_t* xh = st + ((m * 2 + 0) * 2) * 1024 + lane * 16;
          const uint8_t* xl = st + ((m * 2 + 1) * 2) * 1024 + lane * 16;
          const u32x4 h0 = *reinterpret_cast<const u32x4*>(xh), h1 = *reinterpret_cast<const u32x4*>(xh + 1024);
          const u32x4 l0 = *reinterpret_cast<const u32x4*>(xl), l1 = *reinterpret_cast<const u32x4*>(xl + 1024);
          const i32x8 xhi = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
          const i32x8 xlo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xhi, acc[m][nt], 4, 0, 0,
                                                                           wsc[nt], 0, sxh[m]);
            acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xlo, acc[m][nt], 4, 0, 0,
                                                                           wsc[nt], 0, sxl[m]);
          }
        }
      }
    }
  }

  store_h_terms<MT>(a, acc, p0, pn, nb, wave, ln, g);
}

// Gate/up tile for K % 512 == 0 with the weights loaded straight into the MFMA's FP4
// operand registers: lane (ln, g) of tile nt loads the 16 bytes of MXFP4 block 4 ks + g of
// its row (the four lanes of a row read 64 contiguous bytes per step), kWRing - 1 steps ahead
// of the step that uses them, into a register ring. Only the tokens' FP8 terms pass through
// LDS (a kTokStages-stage DMA pipeline shared by the block's waves), so the weights cost no
// LDS bandwidth. The weight scales come into registers 8 steps (32 bytes of a row) at a
// time, one chunk ahead: lane (ln, g) holds bytes [8 g, 8 g + 8) of its row's chunk, and
// the byte of block g of step j is byte g of dword j & 1 of lane (ln, j >> 1), fetched with
// one ds_bpermute. Every byte of weights and scales leaves HBM once per tile.

// Buffer resource over `bytes` bytes at `base` (raw loads; out-of-range lanes read 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int MT, bool PK, int CP>
__device__ __forceinline__ void mx_gateup_tile_rw(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                                  int pn, int nb) {
  constexpr int S = kTokStages, AB = MT * 4 * 1024;
  static_assert(S * AB <= kLdsBytes, "token stages exceed LDS");
  static_assert(kWRing == S, "the wait counts below assume as many weight steps as stages");
  const int P = a.T * a.k;
  const int K = a.d, NR = a.f, KB = K >> 5;
  const uint32_t rq = (uint32_t)(K >> 1);
  const int nk = K / BK;  // multiple of kScaleSteps (K % 1024 == 0)
  const int nch = nk / kScaleSteps;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int ln = lane & 15, g = lane >> 4;

  auto tok_of = [&](int m) {
    const int r = min(16 * m + ln, pn - 1);
    const int pair = a.rows[p0 + r];
    return (pair >= 0 && pair < P) ? pair / a.k : 0;
  };
  // token DMA: waves w < 2 MT stage term (w & 1) of M subtile w >> 1 (as in the LDS-fed tiles)
  const int am = (wave >> 1) < MT ? (wave >> 1) : 0, at = wave & 1;
  const uint8_t* asrc =
      a.x8 + ((size_t)tok_of(am) * 2 + at) * K + 32 * (g >> 1) + 16 * (g & 1);
  int sxh[MT], sxl[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = tok_of(m);
    sxh[m] = a.xs8[2 * t];
    sxl[m] = a.xs8[2 * t + 1];
  }
  // expert e's G and U (weights, scales) as buffer resources; tiles 0, 1: rows +0..15,
  // +16..31 of G; tiles 2, 3: the same rows of U (rows past the end read the last row again;
  // their results are never stored)
  // packed layout: tile t's step s is 1 KB at (t nk + s) KB, its scale chunk c 512 B at
  // (t nch + c) 512 B, both in lane order; row-major: lane (ln, g) reads 16 bytes of its row
  const uint32_t sbytes = PK ? (uint32_t)(NR / 16) * nch * 512u : (uint32_t)(NR * KB);
  const size_t eoff = (size_t)e * NR;
  const __amdgpu_buffer_rsrc_t rq_g = buf_rsrc(a.q0 + eoff * rq, (uint32_t)NR * rq);
  const __amdgpu_buffer_rsrc_t rq_u = buf_rsrc(a.q1 + eoff * rq, (uint32_t)NR * rq);
  const __amdgpu_buffer_rsrc_t rs_g = buf_rsrc(a.s0 + (size_t)e * sbytes, sbytes);
  const __amdgpu_buffer_rsrc_t rs_u = buf_rsrc(a.s1 + (size_t)e * sbytes, sbytes);
  constexpr int QSTEP = PK ? 1024 : 64, SCHUNK = PK ? 512 : 32;
  uint32_t vq[NT], vs[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr (PK) {
      const uint32_t t = (uint32_t)min(nb * 16 + wave * 2 + (nt & 1), NR / 16 - 1);
      vq[nt] = (t * (uint32_t)nk * 64u + (uint32_t)lane) * 16u;
      vs[nt] = (t * (uint32_t)nch * 64u + (uint32_t)lane) * 8u;
    } else {
      const uint32_t r = (uint32_t)min(nb * 256 + wave * 32 + (nt & 1) * 16 + ln, NR - 1);
      vq[nt] = r * rq + 16u * g;
      vs[nt] = r * (uint32_t)KB + 8u * g;
    }
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  auto sload = [&](int nt, int c) {  // this lane's 8 bytes of scale chunk c
    return __builtin_amdgcn_raw_buffer_load_b64(nt < 2 ? rs_g : rs_u, vs[nt], SCHUNK * c, CP);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The K loop, compiled once for the waves that stage tokens (HA) and once for the others,
  // so that each copy issues a fixed number of loads per step and every wait is exact.
  auto kloop = [&](auto ha_c) {
    constexpr bool HA = decltype(ha_c)::value;
    constexpr int OPS = NT + (HA ? 2 : 0);  // loads per step: weights, then the token stage
    u32x4 wr[kWRing][NT];
    u32x2 scur[NT], snxt[NT];
    auto issue = [&](int ks, u32x4 (&dst)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        dst[nt] = __builtin_amdgcn_raw_buffer_load_b128(nt < 2 ? rq_g : rq_u, vq[nt], ks * QSTEP, CP);
      asm volatile("" ::: "memory");
      if constexpr (HA) {
        uint8_t* st = lds + (ks % S) * AB;
        const int o = (am * 2 + at) * 2;
        dma16(asrc + (size_t)ks * BK, st + o * 1024);
        dma16(asrc + (size_t)ks * BK + 64, st + (o + 1) * 1024);
      }
      asm volatile("" ::: "memory");
    };
    // Step ks = 8 c + u of chunk c. AHEAD: steps still to be issued after this one (S - 1 in
    // steady state). SL: this chunk loads the next scale chunk (at u = 0, before the step's
    // own loads); SWAP: this chunk takes over the scale chunk loaded 8 steps ago.
    auto step = [&](int ks, int c, auto u_c, auto ahead_c, auto sl_c, auto swap_c) {
      constexpr int u = decltype(u_c)::value;
      constexpr int AHEAD = decltype(ahead_c)::value;
      constexpr bool SL = decltype(sl_c)::value, SWAP = decltype(swap_c)::value;
      // the weights of step ks and its token stage (issued in that order) have landed once at
      // most the loads issued after them are in flight: those of steps ks + 1 and ks + 2
      // (when issued) and, at u = 1 and 2, the scale loads made at u = 0
      constexpr int LATER = AHEAD >= 2 ? 2 : AHEAD;
      constexpr int EXTRA = (SL && (u == 1 || u == 2)) ? NT : 0;
      wait_vm_known<LATER * OPS + EXTRA>();
      if constexpr (u == 0 && SWAP) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) scur[nt] = snxt[nt];  // complete: loaded 8 steps ago
      }
      barrier_no_fence();
      if constexpr (u == 0 && SL) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) snxt[nt] = sload(nt, c + 1);
        asm volatile("" ::: "memory");
      }
      if constexpr (AHEAD >= S - 1) issue(ks + S - 1, wr[(u + S - 1) % kWRing]);
      const uint8_t* st = lds + (ks % S) * AB;
      const int baddr = (ln + 16 * (u >> 1)) * 4;
      i32x8 wop[NT];
      int wsc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // an FP4 operand takes the low four registers of the tuple; the upper four are left
        // undefined so that no zero registers are kept per tile
        typedef int i32x4v __attribute__((ext_vector_type(4)));
        const i32x4v wi = __builtin_bit_cast(i32x4v, wr[u % kWRing][nt]);
        wop[nt] = __builtin_shufflevector(wi, wi, 0, 1, 2, 3, -1, -1, -1, -1);
        if constexpr (PK)  // this lane's own byte of step u of the chunk
          wsc[nt] = (int)((scur[nt][u >> 2] >> (8 * (u & 3))) & 0xFFu);
        else
          wsc[nt] = (int)(((uint32_t)__builtin_amdgcn_ds_bpermute(baddr, (int)scur[nt][u & 1]) >>
                           (8 * g)) & 0xFFu);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint8_t* xh = st + ((m * 2 + 0) * 2) * 1024 + lane * 16;
        const uint8_t* xl = st + ((m * 2 + 1) * 2) * 1024 + lane * 16;
        const u32x4 h0 = *reinterpret_cast<const u32x4*>(xh), h1 = *reinterpret_cast<const u32x4*>(xh + 1024);
        const u32x4 l0 = *reinterpret_cast<const u32x4*>(xl), l1 = *reinterpret_cast<const u32x4*>(xl + 1024);
        const i32x8 xhi = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
        const i32x8 xlo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xhi, acc[m][nt], 4, 0, 0,
                                                                         wsc[nt], 0, sxh[m]);
          acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xlo, acc[m][nt], 4, 0, 0,
                                                                         wsc[nt], 0, sxl[m]);
        }
      }
    };
    using T0 = std::false_type;
    using T1 = std::true_type;
    (void)T0{};
    // chunk c with `ahead` steps to issue in steady state; the last chunk's last S - 1 steps
    // issue nothing
    auto chunk = [&](int c, auto sl_c, auto swap_c, auto last_c) {
      constexpr bool LAST = decltype(last_c)::value;
      using A = std::integral_constant<int, S - 1>;
      const int ks0 = c * kScaleSteps;
      step(ks0 + 0, c, std::integral_constant<int, 0>{}, A{}, sl_c, swap_c);
      step(ks0 + 1, c, std::integral_constant<int, 1>{}, A{}, sl_c, swap_c);
      step(ks0 + 2, c, std::integral_constant<int, 2>{}, A{}, sl_c, swap_c);
      step(ks0 + 3, c, std::integral_constant<int, 3>{}, A{}, sl_c, swap_c);
      step(ks0 + 4, c, std::integral_constant<int, 4>{}, A{}, sl_c, swap_c);
      step(ks0 + 5, c, std::integral_constant<int, 5>{},
           std::integral_constant<int, LAST ? 2 : S - 1>{}, sl_c, swap_c);
      step(ks0 + 6, c, std::integral_constant<int, 6>{},
           std::integral_constant<int, LAST ? 1 : S - 1>{}, sl_c, swap_c);
      step(ks0 + 7, c, std::integral_constant<int, 7>{},
           std::integral_constant<int, LAST ? 0 : S - 1>{}, sl_c, swap_c);
    };

    // prologue: scale chunk 0 (taken over at step 0), then steps 0 .. S - 2 (nk >= 8 > S - 1)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) snxt[nt] = sload(nt, 0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s2 = 0; s2 < S - 1; ++s2) issue(s2, wr[s2]);
    int c = 0;
    for (; c + 1 < nch; ++c) chunk(c, T1{}, T1{}, T0{});
    chunk(c, T0{}, T1{}, T1{});
  };
  if (wave < 2 * MT) kloop(std::true_type{});
  else kloop(std::false_type{});

  store_h_terms<MT>(a, acc, p0, pn, nb, wave, ln, g);
}

// Down on the block-scaled MFMA: D (FP4, as stored) against h as three E4M3 terms with
// their per-32-block scales (B operand; the scale of block g of pair column x comes from
// lane (x, g)). Per stage a wave DMAs its share of the h tile (a term's 128 bytes per pair
// in the FP8 operand lane order, and each pair's 4 scale bytes of every term), its 4
// weight tiles and their scales; each wave waits on its own DMA count. 3 MFMAs per
// (M subtile, N tile, step).
// Packed weights (PK): each tile's step is one contiguous 1-KB DMA; each wave's scale bytes
// of its 4 tiles for 8 steps come in two 1-KB DMAs into a 2-KB slot, two groups in the ring.
constexpr int kPkSGroup = kWaves * 2048;

template <int MT, bool SG4, bool PK = false>
struct MxDownPipe {
  static constexpr int ADATA = MT * 6 * 1024;      // [m][term][half] 1-KB blocks
  static constexpr int ABYTES = ADATA + MT * 256;  // + scale words [m][term x 16 pairs]
  static constexpr int BYTES = ABYTES + kBStage + (SG4 ? 0 : kSStage);
  static constexpr int RING = PK ? 2 * kPkSGroup : (SG4 ? 2 * kSGroup : 0);
  static constexpr int S0 = (kLdsBytes - RING) / BYTES;
  static constexpr int S = S0 < 4 ? S0 : 4;
  static_assert(S >= 2, "pipeline needs two stages");
  static constexpr int A_PER_WAVE = (6 * MT + kWaves - 1) / kWaves;
};

template <int MT, bool SG4, bool PK, int CP>
__device__ __forceinline__ void mx_down_tile(const MfmaArgs& a, uint8_t* lds, int e, int p0, int pn,
                                             int nb) {
  static_assert(!PK || SG4, "packed scales use the ring");
  using PP = MxDownPipe<MT, SG4, PK>;
  constexpr int S = PP::S, SB = PP::BYTES, AB = PP::ABYTES, AW = PP::A_PER_WAVE;
  const int P = a.T * a.k;
  const int K = a.f, NR = a.d, KB = K >> 5;
  const size_t F = (size_t)K, rq = (size_t)(K >> 1);
  const int nk = K / BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, g = lane >> 4;
  uint8_t* const sring = lds + S * SB;

  // term rows (x3) of this lane's pair in each M subtile; rows past the tile's end repeat
  // its last row (their results are never stored)
  size_t hrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) hrow[m] = (size_t)(p0 + min(16 * m + ln, pn - 1)) * 3;
  const uint8_t* hlane = a.h8 + 32 * (g >> 1) + 16 * (g & 1);
  // scale-word lanes: pair ln, term lane >> 4 (the fourth group repeats term 2)
  const int sw_t = min(lane >> 4, 2);
  const uint8_t* bsrc[NT];
  const uint8_t* ssrc;
  const int nch = (nk + 7) >> 3;
  if constexpr (PK) {
    // tile t's step ks is 1 KB at (t nk + ks) KB in lane order; its scale chunk c is 512 B at
    // (t nch + c) 512 B, 8 bytes per lane
    const size_t qb = (size_t)NR * rq, sbytes = (size_t)(NR / 16) * nch * 512;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const size_t t = (size_t)min(nb * 32 + wave * 4 + nt, NR / 16 - 1);
      bsrc[nt] = a.q0 + (size_t)e * qb + (t * nk * 64 + lane) * 16;
    }
    // scale DMA lane l of copy q: tile 2 q + (l >> 5), lanes 2 (l & 31) and 2 (l & 31) + 1
    const size_t t0 = (size_t)min(nb * 32 + wave * 4 + (lane >> 5), NR / 16 - 1);
    ssrc = a.s0 + (size_t)e * sbytes + (t0 * nch * 64 + 2 * (lane & 31)) * 8;
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = min(nb * 512 + wave * 64 + nt * 16 + ln, NR - 1);
      bsrc[nt] = a.q0 + ((size_t)e * NR + r) * rq + 16 * g;
    }
    const int r = min(nb * 512 + wave * 64 + (lane >> 4) * 16 + (lane & 15), NR - 1);
    ssrc = a.s0 + ((size_t)e * NR + r) * KB;
  }
  // the scale DMA of copy 1 (tiles 2, 3) of the packed layout: tile t0 + 2
  const size_t s_pk_next =
      PK ? ((size_t)min(nb * 32 + wave * 4 + 2 + (lane >> 5), NR / 16 - 1) -
            (size_t)min(nb * 32 + wave * 4 + (lane >> 5), NR / 16 - 1)) * nch * 512
         : 0;
  auto issue = [&](int ks, int slotno) {
    uint8_t* st = lds + slotno * SB;
#pragma unroll
    for (int j = 0; j < AW; ++j) {
      const int b = wave + kWaves * j;
      if (b < 6 * MT) {
        const int m = b / 6, t = (b % 6) >> 1, hh = b & 1;
        dma16(hlane + (hrow[m] + t) * F + (size_t)ks * BK + 64 * hh, st + b * 1024);
      }
    }
    if (wave < MT) {
      const size_t row = (size_t)(p0 + min(16 * wave + ln, pn - 1)) * 3 + sw_t;
      dma4(a.hs8 + row * KB + 4 * ks, st + PP::ADATA + wave * 256);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      dma16p<CP>(bsrc[nt] + (size_t)ks * (PK ? 1024 : 64), st + AB + (wave * NT + nt) * 1024);
    if (PK) {
      if ((ks & 7) == 0) {
        uint8_t* slot = sring + ((ks >> 3) & 1) * kPkSGroup + wave * 2048;
        dma16(ssrc + (size_t)(ks >> 3) * 512, slot);
        dma16(ssrc + s_pk_next + (size_t)(ks >> 3) * 512, slot + 1024);
      }
    } else if (SG4) {
      if ((ks & 3) == 0) dma16(ssrc + ks * 4, sring + ((ks >> 2) & 1) * kSGroup + wave * 1024);
    } else {
      dma4(ssrc + ks * 4, st + AB + kBStage + wave * 256);
    }
  };
  // this wave's DMAs per stage: its h blocks, the scale words of subtile `wave`, weights
  int na = 0;
#pragma unroll
  for (int j = 0; j < AW; ++j) na += (wave + kWaves * j < 6 * MT) ? 1 : 0;
  const int ops = na + (wave < MT ? 1 : 0) + NT + (SG4 ? 0 : 1);
  auto wait_stage = [&](int ks) {
    if (ks + S - 2 >= nk) {
      wait_vm<0>();
      return;
    }
    const int extra = PK ? 2 * (((ks + S - 2) >> 3) - (ks >> 3))
                         : (SG4 ? ((ks + S - 2) >> 2) - (ks >> 2) : 0);
    wait_vm_n((S - 2) * ops + extra);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);

  for (int ks = 0; ks < nk; ++ks) {
    wait_stage(ks);
    barrier_no_fence();
    if (ks + S - 1 < nk) issue(ks + S - 1, (ks + S - 1) % S);

    const uint8_t* st = lds + (ks % S) * SB;
    i32x8 wop[NT];
    int wsc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(st + AB + (wave * NT + nt) * 1024 + lane * 16);
      wop[nt] = i32x8{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
      if (PK)  // this lane's byte of step ks in tile nt's 8-byte entry
        wsc[nt] = sring[((ks >> 3) & 1) * kPkSGroup + wave * 2048 + nt * 512 + lane * 8 + (ks & 7)];
      else
        wsc[nt] = SG4 ? sring[((ks >> 2) & 1) * kSGroup + wave * 1024 + 16 * (nt * 16 + ln) + 4 * (ks & 3) + g]
                      : st[AB + kBStage + wave * 256 + 4 * (nt * 16 + ln) + g];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const uint8_t* xb = st + ((m * 3 + t) * 2) * 1024 + lane * 16;
        const u32x4 h0 = *reinterpret_cast<const u32x4*>(xb), h1 = *reinterpret_cast<const u32x4*>(xb + 1024);
        const i32x8 xop = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
        const int xsc = st[PP::ADATA + m * 256 + (ln + 16 * t) * 4 + g];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xop, acc[m][nt], 4, 0, 0,
                                                                         wsc[nt], 0, xsc);
      }
    }
  }

  // epilogue: lane (ln, g) holds output rows 4 g .. 4 g + 3 of each tile for pair row ln
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = 16 * m + ln;
    if (row >= pn) continue;
    const int pair = a.rows[p0 + row];
    if (pair < 0 || pair >= P) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i0 = nb * 512 + wave * 64 + nt * 16 + 4 * g;  // d % 4 == 0: all four or none
      if (i0 < a.d) *reinterpret_cast<f32x4*>(a.z_out + (size_t)pair * a.d + i0) = acc[m][nt];
    }
  }
}

// Down projection of one tile on the packed layout with the weights fed straight into the
// MFMA's FP4 operand registers: each wave owns NT 16-row tiles of D (64 output rows; the
// block 512), and for K step ks loads its tiles' 1-KB steps with buffer loads into a ring of
// S steps, issued S - 1 steps ahead. Only h passes through LDS: each stage holds the tile's
// three E4M3 terms of h for one K step (MT 16-pair subtiles x 3 terms x 2 x 1 KB) and their
// E8M0 words, S = 4 stages. Every wave issues the same number of h copies per step (the
// last copies are repeated by the waves that have no block of their own: same source, same
// LDS bytes), so each wave's wait for step ks is one compile-time count: its own loads issued
// after those of step ks (steps ks + 1 .. ks + S - 2, and the next scale entries when they
// were loaded in between), then a barrier for the other waves' copies. The K loop is
// unrolled over its NK steps. The weights' scale bytes come 8 steps at a time, 8 bytes per
// lane and tile (the packed scale entry), loaded one chunk ahead.
template <int MT, int NK, int CP>
__device__ __forceinline__ void mx_down_tile_rw(const MfmaArgs& a, uint8_t* lds, int e, int p0,
                                                int pn, int nb) {
  constexpr int S = 4;
  constexpr int ADATA = MT * 6 * 1024;            // [m][term][half] 1-KB blocks
  constexpr int SB = ADATA + MT * 256;            // + scale words [m][term x 16 pairs]
  static_assert(S * SB <= kLdsBytes, "h stages exceed LDS");
  constexpr int NA = (6 * MT + kWaves - 1) / kWaves;  // h blocks per wave and step
  constexpr int OPS = NT + NA + 1;                 // loads per wave and step
  constexpr int NCH = (NK + 7) / 8;                // packed scale entries per tile
  static_assert(NK >= S - 1, "the prologue issues S - 1 steps");
  const int P = a.T * a.k;
  const int K = a.f, NR = a.d, KB = K >> 5;
  const size_t F = (size_t)K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, g = lane >> 4;

  // h term rows (x3) of this lane's pair in each M subtile; rows past the tile's end repeat
  // its last row (their results are never stored)
  size_t hrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) hrow[m] = (size_t)(p0 + min(16 * m + ln, pn - 1)) * 3;
  const uint8_t* hlane = a.h8 + 32 * (g >> 1) + 16 * (g & 1);
  // this wave's h copies: blocks b = wave + 8 j (block b = m 6 + 2 t + hh); past 6 MT, the
  // copy of block b mod 6 MT again. Scale words: subtile wave mod MT, term lane >> 4 (the
  // fourth group repeats term 2).
  const int sw_m = wave % MT, sw_t = min(lane >> 4, 2);
  const uint8_t* swsrc = a.hs8 + ((size_t)(p0 + min(16 * sw_m + ln, pn - 1)) * 3 + sw_t) * KB;
  const uint8_t* hsrc[NA];
  int hdst[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int b = (wave + kWaves * j) % (6 * MT);
    const int m = b / 6, t = (b % 6) >> 1, hh = b & 1;
    hsrc[j] = hlane + (hrow[m] + t) * F + 64 * hh;
    hdst[j] = b * 1024;
  }
  // expert e's D in the packed layout: tile t, step ks at (t NK + ks) KB, lane order; scale
  // chunk c of tile t at (t NCH + c) 512 B, 8 bytes per lane
  const size_t qb = (size_t)NR * (K >> 1), sbytes = (size_t)(NR / 16) * NCH * 512;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(a.q0 + (size_t)e * qb, (uint32_t)qb);
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(a.s0 + (size_t)e * sbytes, (uint32_t)sbytes);
  uint32_t vq[NT], vs[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint32_t t = (uint32_t)min(nb * 32 + wave * 4 + nt, NR / 16 - 1);
    vq[nt] = (t * (uint32_t)NK * 64u + (uint32_t)lane) * 16u;
    vs[nt] = (t * (uint32_t)NCH * 64u + (uint32_t)lane) * 8u;
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x4 wr[S][NT];
  u32x2 scur[NT], snxt[NT];
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // step ks: its weights (ring slot ks mod S), then its h copies into stage ks mod S
  auto issue = [&](auto ks_c) {
    constexpr int KS = decltype(ks_c)::value;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wr[KS % S][nt] = __builtin_amdgcn_raw_buffer_load_b128(rq, vq[nt], KS * 1024, CP);
    asm volatile("" ::: "memory");
    uint8_t* st = lds + (KS % S) * SB;
#pragma unroll
    for (int j = 0; j < NA; ++j) dma16(hsrc[j] + KS * BK, st + hdst[j]);
    dma4(swsrc + 4 * KS, st + ADATA + sw_m * 256);
    asm volatile("" ::: "memory");
  };
  auto sload = [&](int nt, int c) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, vs[nt], 512 * c, CP);
  };
  auto step = [&](auto ks_c) {
    constexpr int KS = decltype(ks_c)::value;
    constexpr int U = KS & 7, C = KS >> 3;
    // loads issued after step KS's: steps KS + 1 .. KS + S - 2 (those issued) and the scale
    // entries of chunk C + 1 when they were loaded (at step 8 C) after step KS's loads
    constexpr int LATER = (NK - 1 - KS) < (S - 2) ? (NK - 1 - KS) : (S - 2);
    constexpr int EXTRA = (U >= 1 && U <= S - 2 && C + 1 < NCH) ? NT : 0;
    wait_vm_known<LATER * OPS + EXTRA>();
    if constexpr (U == 0 && C > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) scur[nt] = snxt[nt];  // loaded 8 steps ago
    }
    barrier_no_fence();
    if constexpr (U == 0 && C + 1 < NCH) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) snxt[nt] = sload(nt, C + 1);
      asm volatile("" ::: "memory");
    }
    if constexpr (KS + S - 1 < NK) issue(std::integral_constant<int, KS + S - 1>{});
    const uint8_t* st = lds + (KS % S) * SB;
    i32x8 wop[NT];
    int wsc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // an FP4 operand takes the low four registers of the tuple; the upper four are left
      // undefined so that no zero registers are kept per tile
      typedef int i32x4v __attribute__((ext_vector_type(4)));
      const i32x4v wi = __builtin_bit_cast(i32x4v, wr[KS % S][nt]);
      wop[nt] = __builtin_shufflevector(wi, wi, 0, 1, 2, 3, -1, -1, -1, -1);
      wsc[nt] = (int)((scur[nt][U >> 2] >> (8 * (U & 3))) & 0xFFu);
    }
    // the step's h scale bytes are read first; then the h operand of the next (m, t) is read
    // before the MFMAs of this one are issued (the scheduling barrier keeps the read there:
    // left free, the scheduler sinks it to just before its own MFMAs and the LDS latency
    // stalls every group). Each accumulator still takes terms 0, 1, 2 in order.
    int xsa[3 * MT];
#pragma unroll
    for (int mt = 0; mt < 3 * MT; ++mt)
      xsa[mt] = st[ADATA + (mt / 3) * 256 + (ln + 16 * (mt % 3)) * 4 + g];
    u32x4 hb0[2], hb1[2];
    auto rd = [&](int mt, int p) {
      const uint8_t* xb = st + mt * 2048 + lane * 16;
      hb0[p] = *reinterpret_cast<const u32x4*>(xb);
      hb1[p] = *reinterpret_cast<const u32x4*>(xb + 1024);
    };
    rd(0, 0);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int mt = m * 3 + t, p = mt & 1;
        const u32x4 h0 = hb0[p], h1 = hb1[p];
        if (mt + 1 < 3 * MT) rd(mt + 1, p ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        const i32x8 xop = {(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
        const int xsc = xsa[mt];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[m][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop[nt], xop, acc[m][nt], 4, 0, 0,
                                                                         wsc[nt], 0, xsc);
          // ties each MFMA to this point, and the next term's LDS reads below it: left free,
          // the scheduler gathers the MFMAs of many steps at the end and holds every operand
          // read before them
          asm volatile("" : "+v"(acc[m][nt])::"memory");
        }
      }
    }
  };

  // prologue: scale chunk 0 (taken over at step 0), then steps 0 .. S - 2
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) scur[nt] = sload(nt, 0);
  asm volatile("" ::: "memory");
  for_each_const(std::make_integer_sequence<int, S - 1>{}, issue);
  for_each_const(std::make_integer_sequence<int, NK>{}, step);

  // epilogue: lane (ln, g) holds output rows 4 g .. 4 g + 3 of each tile for pair row ln
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = 16 * m + ln;
    if (row >= pn) continue;
    const int pair = a.rows[p0 + row];
    if (pair < 0 || pair >= P) continue;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int i0 = nb * 512 + wave * 64 + nt * 16 + 4 * g;  // d % 4 == 0: all four or none
      if (i0 < a.d) *reinterpret_cast<f32x4*>(a.z_out + (size_t)pair * a.d + i0) = acc[m][nt];
    }
  }
}

// Token rows -> two FP8 E4M3 terms with one E8M0 scale per term row. With e the exponent
// that puts the row maximum in [128, 256): y = x 2^-e (exact), hi = RNE_e4m3(y), and the
// remainder y - hi (exact in fp32) is coded the same way against its own maximum. For a
// bf16 row every element is then carried to about 2^-22 of the row maximum. A non-finite
// maximum gives scale byte 255 (NaN). One block per token; each thread holds up to
// kPrepChunks 4-element pieces of the row in registers through the three sweeps (rows
// longer than 256 * 4 * kPrepChunks are read again per sweep).
constexpr int kPrepChunks = 8;
__global__ __launch_bounds__(256) void x8_prep_kernel(int d, const uint16_t* __restrict__ x,
                                                      uint8_t* __restrict__ x8,
                                                      uint8_t* __restrict__ xs8) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint2* xr = reinterpret_cast<const uint2*>(x + (size_t)t * d);  // d % 4 == 0
  const int nq = d >> 2;
  auto block_max = [&](float v) {
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  };
  // exponent putting m in [128, 256), or INT_MIN for m == 0, INT_MAX for non-finite m
  auto top_exp = [](float m) -> int {
    if (!__builtin_isfinite(m)) return 0x7fffffff;
    if (m == 0.0f) return -0x7fffffff;
    return ilogbf(m) - 7;
  };
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  // four E4M3 codes (RNE) in one dword, byte i from v_i
  auto pk_e4m3 = [](float v0, float v1, float v2, float v3) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false),
                                           true);
  };
  auto unpack = [](uint2 v, float f[4]) {
    f[0] = bf16_bits_to_f32(v.x & 0xFFFFu);
    f[1] = bf16_bits_to_f32(v.x >> 16);
    f[2] = bf16_bits_to_f32(v.y & 0xFFFFu);
    f[3] = bf16_bits_to_f32(v.y >> 16);
  };
  const bool cached = nq <= 256 * kPrepChunks;
  uint2 reg[kPrepChunks];
  if (cached) {
#pragma unroll
    for (int c = 0; c < kPrepChunks; ++c) {
      const int q = tid + 256 * c;
      reg[c] = q < nq ? xr[q] : make_uint2(0u, 0u);
    }
  }
  // piece c of this thread (c-th of the sweep), from registers or memory
  auto piece = [&](int c, int q) { return cached ? reg[c] : xr[q]; };

  float mx = 0.0f;
  for (int q0 = 0; q0 < nq; q0 += 256 * kPrepChunks)
#pragma unroll
    for (int c = 0; c < kPrepChunks; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        float f[4];
        unpack(piece(c, q), f);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(f[0]), fabsf(f[1])), fmaxf(fabsf(f[2]), fabsf(f[3]))));
      }
    }
  mx = block_max(mx);
  const int eh0 = top_exp(mx);
  const bool bad = eh0 == 0x7fffffff;
  const int sh = bad ? 255 : min(max(eh0 + 127, 0), 254);
  const int eh = sh - 127;  // exponent actually applied (row maximum may sit below 128)

  float rm = 0.0f;
  for (int q0 = 0; q0 < nq; q0 += 256 * kPrepChunks)
#pragma unroll
    for (int c = 0; c < kPrepChunks; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        float f[4], y[4];
        unpack(piece(c, q), f);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = ldexpf(f[i], -eh);
        // two values per conversion, each way (the same RNE codes as one at a time)
        const int cq = pk_e4m3(y[0], y[1], y[2], y[3]);
        const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(cq, false);
        const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(cq, true);
        rm = fmaxf(rm, fmaxf(fmaxf(fabsf(y[0] - b01[0]), fabsf(y[1] - b01[1])),
                             fmaxf(fabsf(y[2] - b23[0]), fabsf(y[3] - b23[1]))));
      }
    }
  rm = block_max(rm);
  const int er0 = top_exp(rm);  // relative to the hi scale
  const int sl = bad ? 255 : min(max(sh + max(er0, -300), 0), 254);
  const int er = sl - sh;
  uint32_t* hi = reinterpret_cast<uint32_t*>(x8 + (size_t)t * 2 * d);
  uint32_t* lo = reinterpret_cast<uint32_t*>(x8 + (size_t)t * 2 * d + d);
  for (int q0 = 0; q0 < nq; q0 += 256 * kPrepChunks)
#pragma unroll
    for (int c = 0; c < kPrepChunks; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        float f[4], y[4];
        unpack(piece(c, q), f);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = ldexpf(f[i], -eh);
        const int wh = pk_e4m3(y[0], y[1], y[2], y[3]);
        const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(wh, false);
        const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(wh, true);
        const int wl = pk_e4m3(ldexpf(y[0] - b01[0], -er), ldexpf(y[1] - b01[1], -er),
                               ldexpf(y[2] - b23[0], -er), ldexpf(y[3] - b23[1], -er));
        hi[q] = (uint32_t)wh;
        lo[q] = (uint32_t)wl;
      }
    }
  if (tid == 0) {
    xs8[2 * t] = (uint8_t)sh;
    xs8[2 * t + 1] = (uint8_t)sl;
  }
}


// ---- down projection of one token on the block-scaled MFMA (decode) -----------------------
// Persistent: one block per CU, one wave per slot (k <= 16); the block owns an equal range of
// output rows (28 of 7168 on 256 CUs) and walks it in tiles of 16 rows. Wave q:
//  1. loads its expert's 16 rows of the tile as the MFMA's FP4 operand straight into
//     registers: for K step s (128 elements), lane (r, g) = (lane & 15, lane >> 4) takes
//     MXFP4 block 4s + g of row r (the four lanes of a row read 64 contiguous bytes) and the
//     dword with the step's four scale bytes of its row (its own is byte g);
//  2. once per block, while the first tile's loads are in flight, splits the slot's fp32 h
//     into three E4M3 terms with one E8M0 scale per term (for the whole slot, steps of 2^4
//     apart) into its own LDS area (natural order);
//  3. runs one MFMA per step with the three terms as B columns 0..2 (other columns zero), so
//     column c of the result is term c's share of z; z = (C0 + C1) + C2. The next tile's
//     weight loads are issued as soon as the last MFMA has its operands.
// After a barrier the block adds the k slot results of each row in slot order, so y is
// bit-identical from run to run. Weights are multiplied as stored; nothing is decoded.
constexpr int kDecMfmaSlots = 16;
constexpr int kDecMfmaMaxF = 1536;  // K steps <= 12
constexpr int kDecTermBytes = 3 * kDecMfmaMaxF;

struct DownDecMArgs {
  int d, f, k;
  const uint8_t *dq, *ds;
  const float* h;
  const int32_t *pair_pos, *pair_exp;
  const float* gates;
  const float *resid, *shared;
  float* y;
  uint16_t* y_bf16;
  int rpb;  // output rows per block
};

template <int NK, bool PK>
__global__ __launch_bounds__(1024) void down_decode_mfma_kernel(DownDecMArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tb[kDecMfmaSlots][kDecTermBytes];
  __shared__ float zs[2][kDecMfmaSlots][16];
  __shared__ float gsh[kDecMfmaSlots];
  const int F = NK * BK, FB = F >> 5;
  const int tid = threadIdx.x, lane = tid & 63, q = tid >> 6;  // wave = slot
  const int ln = lane & 15, g = lane >> 4;
  // rows [rb0, rb1) of this block, walked in tiles of 16 (the last may be partial)
  const int rb0 = blockIdx.x * a.rpb, rb1 = min(a.d, rb0 + a.rpb);
  int r0 = rb0;
  if (tid < a.k) gsh[tid] = a.gates[tid];
  const int pos = a.pair_pos[q];
  const int e = a.pair_exp[q];
  const bool sv = pos >= 0 && e >= 0;

  // h of the slot first (four values per lane and round), so that waiting for it later
  // leaves the weight loads behind it in flight
  constexpr int NR = (NK * BK / 4 + 63) / 64;
  f32x4 hv[NR];
  const float* hr = a.h + (size_t)(sv ? pos : 0) * F;
#pragma unroll
  for (int v0 = 0; v0 < NR; ++v0) {
    const int c = v0 * 64 + lane;
    hv[v0] = c < (F >> 2) ? reinterpret_cast<const f32x4*>(hr)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // 1. weights of one tile's 16 rows; lanes of rows past the block's range read the last row
  //    of the range again (same addresses as a lane in the same load, so no extra traffic;
  //    their results are never combined). Unconditional loads keep the wait counts exact.
  //    Packed layout: the block's rows are whole 16-row tiles, a tile step is one 1-KB piece
  //    in lane order and a lane's scale bytes of 8 steps are one 8-byte entry.
  constexpr int NCH = (NK + 7) / 8;
  constexpr int NSW = PK ? 2 * NCH : NK;
  const uint8_t* wq0 = PK ? a.dq + (size_t)(sv ? e : 0) * a.d * (size_t)(F >> 1) + 16 * lane
                          : a.dq + (size_t)(sv ? e : 0) * a.d * (size_t)(F >> 1) + 16 * g;
  const uint8_t* ws0 = PK ? a.ds + (size_t)(sv ? e : 0) * (a.d >> 4) * (size_t)(NCH * 512) + 8 * lane
                          : a.ds + (size_t)(sv ? e : 0) * a.d * (size_t)FB;
  u32x4 w[NK];
  uint32_t sw[NSW];
  auto load_tile = [&](int rt) {
    if constexpr (PK) {
      const int tt = rt >> 4;
      const uint2* wsc = reinterpret_cast<const uint2*>(ws0 + (size_t)tt * (NCH * 512));
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint2 v = wsc[c * 64];
        sw[2 * c] = v.x;
        sw[2 * c + 1] = v.y;
      }
      const uint8_t* wq = wq0 + (size_t)tt * NK * 1024;
#pragma unroll
      for (int s = 0; s < NK; ++s) w[s] = load_u32x4_nt(wq + 1024 * s);
    } else {
      const int row = min(rt + ln, rb1 - 1);
      const uint8_t* wq = wq0 + (size_t)row * (size_t)(F >> 1);
      const uint32_t* wsc = reinterpret_cast<const uint32_t*>(ws0 + (size_t)row * (size_t)FB);
#pragma unroll
      for (int s = 0; s < NK; ++s) sw[s] = wsc[s];  // scales first: step s waits for block s only
#pragma unroll
      for (int s = 0; s < NK; ++s) w[s] = load_u32x4_nt(wq + 64 * s);
    }
  };
  load_tile(r0);  // every block has at least one row
  // residual and shared-expert values of this thread's row in the current tile, requested a
  // tile ahead of the combine that adds them (behind that tile's weight loads, so waiting for
  // them leaves the next tile's weights in flight)
  float res_r = 0.0f, res_s = 0.0f;
  auto fetch_res = [&](int rt) {
    if (a.resid && tid < 16) {
      const int r = min(rt + tid, rb1 - 1);
      res_r = a.resid[r];
      res_s = a.shared ? a.shared[r] : 0.0f;
    }
  };
  fetch_res(r0);

  // 2. three E4M3 terms of h with one E8M0 scale per term for the whole slot: 2^(s0-127)
  //    puts the slot maximum in [128, 256), term t has scale s0 - 4t. RNE to E4M3 leaves a
  //    remainder of at most 2^-4 of each value, so 16 x the remainder fits the next term,
  //    and every value is carried to about 2^-12 of itself (subnormal floor 2^-18 of the
  //    slot maximum). A non-finite maximum gives scale bytes 255 (NaN), as does the oracle's
  //    sum over every h value for each output row.
  uint8_t* tq = tb[q];
  float mx = 0.0f;
#pragma unroll
  for (int v0 = 0; v0 < NR; ++v0)
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(hv[v0][0]), fabsf(hv[v0][1])),
                         fmaxf(fabsf(hv[v0][2]), fabsf(hv[v0][3]))));
  mx = fmaxf(mx, lane_xor_f<1>(mx, lane));
  mx = fmaxf(mx, lane_xor_f<2>(mx, lane));
  mx = fmaxf(mx, lane_xor_f<4>(mx, lane));
  mx = fmaxf(mx, lane_xor_f<8>(mx, lane));
  mx = fmaxf(mx, lane_xor_f<16>(mx, lane));
  mx = fmaxf(mx, lane_xor_f<32>(mx, lane));
  const int e0 = top_exp(mx);
  const bool bad = e0 == kExpBad;
  const int s0 = bad ? 255 : min(max(e0 + 127, 0), 254);
  int tsc[3], ter[3];  // term scale byte and its exponent relative to term 0
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    tsc[t] = bad ? 255 : max(s0 - 4 * t, 0);
    ter[t] = tsc[t] - s0;
  }
#pragma unroll
  for (int v0 = 0; v0 < NR; ++v0) {
    const int c = v0 * 64 + lane;
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = ldexpf(hv[v0][i], 127 - s0);  // exact: maximum < 256
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      float ys[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ys[i] = t == 0 ? y[i] : ldexpf(y[i], -ter[t]);
      // two E4M3 codes (RNE) per conversion, written into the term's dword in place
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(ys[0], ys[1], 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(ys[2], ys[3], wd, true);
      if (t < 2) {
        y[0] -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(wd, 0), ter[t]);
        y[1] -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(wd, 1), ter[t]);
        y[2] -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(wd, 2), ter[t]);
        y[3] -= ldexpf(__builtin_amdgcn_cvt_f32_fp8(wd, 3), ter[t]);
      }
      if (c < (F >> 2)) *reinterpret_cast<int*>(tq + t * F + 4 * c) = wd;
    }
  }
  // the wave reads back what its own lanes wrote (LDS operations of a wave are in order)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");

  // 3. one MFMA per K step; B column ln < 3 is term ln, the rest zero with scale 1
  const bool bl = ln < 3;
  const uint8_t* tb_ln = tq + (bl ? ln : 0) * F + 16 * g;
  const int bsc = bl ? tsc[ln == 0 ? 0 : (ln == 1 ? 1 : 2)] : 127;
  for (int it = 0;; ++it) {
    // the B operands are the same for every tile; they are read again per tile from LDS, one
    // step ahead of the MFMA that takes them (the asm statements keep the compiler from
    // gathering all of them into the registers the weights need)
    asm volatile("" ::: "memory");
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    u32x4 b0 = {0u, 0u, 0u, 0u}, b1 = {0u, 0u, 0u, 0u};
    if (bl) {
      b0 = *reinterpret_cast<const u32x4*>(tb_ln);
      b1 = *reinterpret_cast<const u32x4*>(tb_ln + 64);
    }
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      u32x4 n0 = {0u, 0u, 0u, 0u}, n1 = {0u, 0u, 0u, 0u};
      if (s + 1 < NK && bl) {
        n0 = *reinterpret_cast<const u32x4*>(tb_ln + BK * (s + 1));
        n1 = *reinterpret_cast<const u32x4*>(tb_ln + BK * (s + 1) + 64);
      }
      // an FP4 operand occupies the low four registers of the tuple; the upper four are
      // left undefined so that no zero registers are kept per step
      typedef int i32x4v __attribute__((ext_vector_type(4)));
      const i32x4v wi = __builtin_bit_cast(i32x4v, w[s]);
      const i32x8 aop = __builtin_shufflevector(wi, wi, 0, 1, 2, 3, -1, -1, -1, -1);
      const i32x8 bop = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                         (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
      const int asc = PK ? (int)((sw[2 * (s >> 3) + ((s & 7) >> 2)] >> (8 * (s & 3))) & 0xFFu)
                         : (int)((sw[s] >> (8 * g)) & 0xFFu);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc, 4, 0, 0, asc, 0, bsc);
      b0 = n0;
      b1 = n1;
      // ties the MFMA to this point: the next step's LDS reads (and, after the last step,
      // the next tile's weight loads) stay below it
      asm volatile("" : "+v"(acc)::"memory");
    }
    const int next = r0 + 16;
    const bool more = next < rb1;  // on the only path that goes on, w is reloaded
    if (more) load_tile(next);
    // lane (c, g) holds column c of rows 4 g .. 4 g + 3
    float (*zb)[16] = zs[it & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // lane (0, g) takes columns 1 and 2 from lanes (1, g) and (2, g)
      const float c1 = lane_xor_f<1>(acc[i], lane);
      const float c2 = lane_xor_f<2>(acc[i], lane);
      if (ln == 0) zb[q][4 * g + i] = sv ? (acc[i] + c1) + c2 : 0.0f;
    }
    // barrier without draining the next tile's loads: only LDS writes must be complete
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (tid < min(16, rb1 - r0)) {
      const int r = r0 + tid;
      float s2 = 0.0f;
      for (int j = 0; j < a.k; ++j) s2 = fmaf(gsh[j], zb[j][tid], s2);
      float out = s2;
      if (a.resid) out = (res_r + res_s) + s2;
      a.y[r] = out;
      if (a.y_bf16) a.y_bf16[r] = f32_to_bf16_rne(out);
    }
    if (!more) break;
    r0 = next;
    fetch_res(r0);
  }
}

// ---- gate/up of one token on the packed layout, block-scaled MFMA --------------------------
// One block per (slot, 16-row tile of f), one wave per chunk of 8 K steps (1024 elements of d;
// d / 1024 waves). Wave c:
//  1. copies its chunk of the token into LDS (asynchronous copies) and issues all 8 steps of
//     the tile in G and in U (1 KB each: lane (i, g) = row i, MXFP4 block 4 s + g, as the
//     packed layout stores them) and its two packed scale entries, all at once;
//  2. splits the chunk into NTM E4M3 terms with one E8M0 scale per term and 32-element block
//     (lane l takes elements 16 l .. 16 l + 15, two lanes per block): term 0 puts the block
//     maximum in [128, 256), each further term codes what the previous ones left against its
//     own maximum. Two terms carry a bf16 token exactly (to about 2^-22 of the block maximum),
//     three an fp32 one to about 2^-13 of it. The terms overwrite the chunk in LDS (each lane
//     has read its elements first), natural order, scales behind them;
//  3. runs one MFMA per step and matrix with the weights as the FP4 operand as stored and the
//     terms as FP8 B columns 0 .. NTM - 1 (the other columns repeat term 0 and are not read),
//     so column t of the result is term t's share of the row's dot product: (C0 + C1) (+ C2).
// The per-row chunk sums go through LDS and wave 0 adds them in chunk order and writes
// h = silu(gate) * up, so results are the same from run to run. The weights are never
// decoded: the dot products of the one-token GEMV become 16 MFMAs per wave.
struct GateUpPackedArgs {
  int d, f, k;
  const void* x;
  const uint8_t *gq, *gs, *uq, *us;  // packed G and U
  const int32_t *pair_pos, *pair_exp;
  float* h;  // [k][f] by bucket position
};
constexpr int kPkMaxWaves = 16;  // d <= 16384
// LDS bytes per wave: the chunk as copied, or its terms and their scales if that is more
__host__ __device__ constexpr int pk_wave_lds(bool xf32) {
  return xf32 ? 4096 : 2048 + 2 * 32;
}

// Work item `item` = (slot, tile) of the block; xl: the dynamic LDS (nch * AREA bytes);
// part: per-chunk row sums.
template <bool XF32>
__device__ __forceinline__ void gateup_packed_item(int item, const GateUpPackedArgs& a,
                                                   uint8_t* xl, float (*part)[2][16]) {
  constexpr int NTM = XF32 ? 3 : 2;  // E4M3 terms of the token
  constexpr int AREA = pk_wave_lds(XF32);
  const int d = a.d, f = a.f;
  const int lane = threadIdx.x & 63;
  const int c = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's chunk
  const int g = lane >> 4, ln = lane & 15;
  const int ntile = f >> 4, nk = d / 128, nch = nk >> 3;
  const int q = item / ntile, t = item - (item / ntile) * ntile;
  const int pos = __builtin_amdgcn_readfirstlane(a.pair_pos[q]);
  const int e = __builtin_amdgcn_readfirstlane(a.pair_exp[q]);
  if (pos < 0 || e < 0) return;  // block-uniform
  uint8_t* xw = xl + c * AREA;
  // 1. the chunk's 1024 token elements into this wave's LDS area (1 KB per copy), then the
  //    two scale entries and the 8 steps of G and U, in the order they are used
  constexpr int NCOPY = XF32 ? 4 : 2;
#pragma unroll
  for (int u = 0; u < NCOPY; ++u)
    __builtin_amdgcn_global_load_lds(static_cast<const uint8_t*>(a.x) + ((size_t)c * NCOPY + u) * 1024 +
                                         lane * 16,
                                     (lds_void*)(xw + u * 1024), 16, 0, 0);
  asm volatile("" ::: "memory");  // the copies stay the oldest loads
  const size_t qb = (size_t)f * (d >> 1), sb = (size_t)(f >> 4) * nch * 512;
  const size_t qo = (size_t)e * qb + (((size_t)t * nk + 8 * c) * 64 + lane) * 16;
  const size_t so = (size_t)e * sb + (((size_t)t * nch + c) * 64 + lane) * 8;
  const uint64_t sg = *reinterpret_cast<const uint64_t*>(a.gs + so);
  const uint64_t su = *reinterpret_cast<const uint64_t*>(a.us + so);
  asm volatile("" ::: "memory");
  u32x4 wg[8], wu[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    wg[j] = load_u32x4_nt(a.gq + qo + (size_t)j * 1024);
    wu[j] = load_u32x4_nt(a.uq + qo + (size_t)j * 1024);
  }
  asm volatile("" ::: "memory");
  // the token copies are the oldest loads: waiting for them leaves the other 18 in flight (as
  // the builtin, so that the compiler's own waits for the weights stay per step)
  wait_vm_known<18>();
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");

  // 2. terms of this lane's 16 elements
  float y[16];
  if constexpr (XF32) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(xw + 64 * lane + 16 * v);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[4 * v + i] = __uint_as_float(w4[i]);
    }
  } else {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(xw + 32 * lane + 16 * v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[8 * v + 2 * i] = __uint_as_float(w4[i] << 16);
        y[8 * v + 2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
      }
    }
  }
  // every lane holds its elements before any term overwrites the chunk
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  auto bmax = [&](float m) { return fmaxf(m, lane_xor_f<1>(m, lane)); };  // the block's two lanes
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(y[i]));
  mx = bmax(mx);
  const int e0 = top_exp(mx);
  const bool bad = e0 == kExpBad;
  const int s0 = bad ? 255 : min(max(e0 + 127, 0), 254);
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = ldexpf(y[i], 127 - s0);  // exact: the maximum below 256
#pragma unroll
  for (int tm = 0; tm < NTM; ++tm) {
    int sc = s0, er = 0;  // term scale and its exponent relative to term 0
    if (tm > 0) {
      float rm = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) rm = fmaxf(rm, fabsf(y[i]));
      rm = bmax(rm);
      const int ex = top_exp(rm);
      sc = bad ? 255 : min(max(s0 + max(ex, -300), 0), 254);
      er = sc - s0;
    }
    u32x4 codes = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int cq = e4m3_code(ldexpf(y[i], -er));
      y[i] -= ldexpf(e4m3_value(cq), er);
      codes[i >> 2] |= (uint32_t)cq << (8 * (i & 3));
    }
    *reinterpret_cast<u32x4*>(xw + tm * 1024 + 16 * lane) = codes;
    if ((lane & 1) == 0) xw[NTM * 1024 + tm * 32 + (lane >> 1)] = (uint8_t)sc;
  }
  // the wave reads back what its own lanes wrote (LDS operations of a wave are in order)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");

  // 3. one MFMA per step and matrix
  const int tt = ln < NTM ? ln : 0;  // this lane's term (B column)
  const uint8_t* tb = xw + tt * 1024 + 16 * g;
  const uint8_t* ts = xw + NTM * 1024 + tt * 32 + g;
  f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 b0 = *reinterpret_cast<const u32x4*>(tb + 128 * j);
    const u32x4 b1 = *reinterpret_cast<const u32x4*>(tb + 128 * j + 64);
    const int bsc = ts[4 * j];
    const i32x8 bop = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                       (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    // an FP4 operand takes the low four registers of the tuple; the upper four are undefined
    typedef int i32x4v __attribute__((ext_vector_type(4)));
    const i32x4v wgi = __builtin_bit_cast(i32x4v, wg[j]), wui = __builtin_bit_cast(i32x4v, wu[j]);
    const i32x8 ag = __builtin_shufflevector(wgi, wgi, 0, 1, 2, 3, -1, -1, -1, -1);
    const i32x8 au = __builtin_shufflevector(wui, wui, 0, 1, 2, 3, -1, -1, -1, -1);
    const int gsc = (int)((sg >> (8 * j)) & 0xFFu), usc = (int)((su >> (8 * j)) & 0xFFu);
    accg = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ag, bop, accg, 4, 0, 0, gsc, 0, bsc);
    accu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(au, bop, accu, 4, 0, 0, usc, 0, bsc);
  }
  // lane (ln, g) holds column ln (term ln) of tile rows 4 g .. 4 g + 3
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // lane (0, g) takes columns 1 (and 2) from lanes (1, g) (and (2, g))
    float gs = accg[r] + lane_xor_f<1>(accg[r], lane);
    float us = accu[r] + lane_xor_f<1>(accu[r], lane);
    if (NTM == 3) {
      gs += lane_xor_f<2>(accg[r], lane);
      us += lane_xor_f<2>(accu[r], lane);
    }
    if (ln == 0) {
      part[c][0][4 * g + r] = gs;
      part[c][1][4 * g + r] = us;
    }
  }
  __syncthreads();
  if (c == 0 && lane < 16) {
    float gs2 = part[0][0][lane], us2 = part[0][1][lane];
    for (int c2 = 1; c2 < nch; ++c2) {
      gs2 += part[c2][0][lane];
      us2 += part[c2][1][lane];
    }
    a.h[(size_t)pos * f + 16 * t + lane] = silu_f32(gs2) * us2;
  }
}

template <bool XF32>
__global__ __launch_bounds__(64 * kPkMaxWaves) void gateup_decode_packed_kernel(
    GateUpPackedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
  __shared__ float part[kPkMaxWaves][2][16];
  gateup_packed_item<XF32>(blockIdx.x, a, xl, part);
}

// Block mode: the expert items, then the shared expert's down GEMV (out = W hsh, bf16 W
// [d][f]) in the blocks after them, one row group of the block's waves each; its 22 MB at the
// K3 shapes fill the tail of the expert stream.
struct SharedDownArgs {
  int d, f;
  const float* hsh;
  const uint16_t* w;
  float* out;
};
template <bool XF32>
__global__ __launch_bounds__(64 * kPkMaxWaves) void gateup_packed_shared_down_kernel(
    GateUpPackedArgs a, SharedDownArgs sd) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
  __shared__ float part[kPkMaxWaves][2][16];
  const int items = a.k * (a.f >> 4);
  if ((int)blockIdx.x < items) {  // block-uniform
    gateup_packed_item<XF32>(blockIdx.x, a, xl, part);
    return;
  }
  StageRow stg{sd.hsh, sd.f};
  bf16_gemv_rows<false>((int)blockIdx.x - items, (int)gridDim.x - items, 1, sd.d, sd.f, stg, sd.w,
                        nullptr, sd.out, reinterpret_cast<f32x4*>(xl));
}

}  // namespace

int mfma_mtiles_bound(int T, int E, int k) {
  const long P = (long)T * k;
  const long act = P < E ? P : E;
  return (int)(act + P / BM + 1);
}

bool mfma_shape_supported(int d, int f) { return d % BK == 0 && f % BK == 0; }

hipError_t launch_gateup_mfma(int T, int d, int f, int E, int k, const uint16_t* x,
                              const MxPtrs& w, const int32_t* offsets, const int32_t* rows,
                              const int32_t* act, const int32_t* n_act,
                              const int32_t* mtile_off, uint8_t* h8, uint8_t* hs8, uint8_t* x8,
                              uint8_t* xs8, hipStream_t s, bool packed) {
  x8_prep_kernel<<<T, 256, 0, s>>>(d, x, x8, xs8);
  MfmaArgs a{};
  a.T = T; a.d = d; a.f = f; a.k = k; a.x8 = x8; a.xs8 = xs8;
  a.q0 = w.gate_q; a.s0 = w.gate_s; a.q1 = w.up_q; a.s1 = w.up_s;
  a.offsets = offsets; a.rows = rows; a.act = act; a.n_act = n_act; a.mtile_off = mtile_off;
  a.nblk_n = (f + 255) / 256;
  a.packed = packed ? 1 : 0;
  a.hot_tokens = g_hot_tokens.load(std::memory_order_relaxed);
  a.h8 = h8;
  a.hs8 = hs8;
  dim3 grid((unsigned)(mfma_mtiles_bound(T, E, k) * a.nblk_n));
  launch_timed(mfma_ffn_kernel<true>, grid, dim3(512), 0u, s, a);
  return hipGetLastError();
}

bool set_hot_tokens(int n) {
  if (n < 0 || n > kHotTokensMax) return false;
  g_hot_tokens.store(n, std::memory_order_relaxed);
  return true;
}
int hot_tokens() { return g_hot_tokens.load(std::memory_order_relaxed); }

bool packed_shape_supported(int d, int f) { return d % 1024 == 0 && f % 512 == 0; }

hipError_t launch_down_mfma(int T, int d, int f, int E, int k, const MxPtrs& w,
                            const uint8_t* h8, const uint8_t* hs8, const int32_t* offsets,
                            const int32_t* rows, const int32_t* act, const int32_t* n_act,
                            const int32_t* mtile_off, float* z, hipStream_t s, bool packed) {
  MfmaArgs a{};
  a.packed = packed ? 1 : 0;
  a.hot_tokens = g_hot_tokens.load(std::memory_order_relaxed);
  a.T = T; a.d = d; a.f = f; a.k = k;
  a.h8 = const_cast<uint8_t*>(h8);
  a.hs8 = const_cast<uint8_t*>(hs8);
  a.q0 = w.down_q; a.s0 = w.down_s;
  a.offsets = offsets; a.rows = rows; a.act = act; a.n_act = n_act; a.mtile_off = mtile_off;
  a.nblk_n = (d + 511) / 512;
  a.z_out = z;
  dim3 grid((unsigned)(mfma_mtiles_bound(T, E, k) * a.nblk_n));
  launch_timed(mfma_ffn_kernel<false>, grid, dim3(512), 0u, s, a);
  return hipGetLastError();
}


bool down_decode_mfma_supported(int d, int f, int k) {
  return d % 16 == 0 && f % BK == 0 && f <= kDecMfmaMaxF && k >= 1 && k <= kDecMfmaSlots;
}

hipError_t launch_down_decode_mfma(int d, int f, int k, const MxPtrs& w, const float* h,
                                   const int32_t* pair_pos, const int32_t* pair_exp,
                                   const float* gates, const float* resid, const float* shared,
                                   float* y, uint16_t* y_bf16, int n_cu, hipStream_t s,
                                   bool packed) {
  DownDecMArgs a;
  a.d = d; a.f = f; a.k = k; a.dq = w.down_q; a.ds = w.down_s; a.h = h;
  a.pair_pos = pair_pos; a.pair_exp = pair_exp; a.gates = gates;
  a.resid = resid; a.shared = shared; a.y = y; a.y_bf16 = y_bf16;
  // equal row ranges for one block per CU (16 rows at least; whole tiles when packed)
  const int nb = n_cu > 0 ? n_cu : 1;
  if (packed)
    a.rpb = 16 * ((d / 16 + nb - 1) / nb);
  else
    a.rpb = (d + nb - 1) / nb;
  if (a.rpb < 16) a.rpb = 16;
  const dim3 grid((unsigned)((d + a.rpb - 1) / a.rpb)), block((unsigned)(64 * k));
  switch (f / BK) {
#define K3_DM(N)                                                              \
  case N:                                                                     \
    if (packed)                                                               \
      launch_timed(down_decode_mfma_kernel<N, true>, grid, block, 0u, s, a);  \
    else                                                                      \
      launch_timed(down_decode_mfma_kernel<N, false>, grid, block, 0u, s, a); \
    break;
    K3_DM(1) K3_DM(2) K3_DM(3) K3_DM(4) K3_DM(5) K3_DM(6)
    K3_DM(7) K3_DM(8) K3_DM(9) K3_DM(10) K3_DM(11) K3_DM(12)
#undef K3_DM
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gateup_decode_packed(int d, int f, int k, const void* x, int xf32,
                                       const MxPtrs& w, const int32_t* pair_pos,
                                       const int32_t* pair_exp, float* h, hipStream_t s,
                                       const SharedDown* shared) {
  if (d % 1024 != 0 || f % 16 != 0) return hipErrorInvalidValue;
  const int nch = d / 1024;
  if (nch < 1 || nch > kPkMaxWaves) return hipErrorInvalidValue;
  GateUpPackedArgs a;
  a.d = d; a.f = f; a.k = k; a.x = x;
  a.gq = w.gate_q; a.gs = w.gate_s; a.uq = w.up_q; a.us = w.up_s;
  a.pair_pos = pair_pos; a.pair_exp = pair_exp; a.h = h;
  const int items = k * (f / 16);
  const dim3 block((unsigned)(64 * nch));
  const uint32_t lds = (uint32_t)(nch * pk_wave_lds(xf32 != 0));
  if (shared) {
    // the shared down's staged hsh (f floats) fits the expert items' LDS: f <= 16 d / 4
    if ((size_t)f * 4 > lds || f % 8 != 0) return hipErrorInvalidValue;
    SharedDownArgs sd{d, f, shared->hsh, shared->w, shared->out};
    const int rows = gemv_group_rows(f, nch);
    const dim3 grid((unsigned)(items + (d + rows - 1) / rows));
    if (xf32)
      launch_timed(gateup_packed_shared_down_kernel<true>, grid, block, lds, s, a, sd);
    else
      launch_timed(gateup_packed_shared_down_kernel<false>, grid, block, lds, s, a, sd);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)items);
  if (xf32)
    launch_timed(gateup_decode_packed_kernel<true>, grid, block, lds, s, a);
  else
    launch_timed(gateup_decode_packed_kernel<false>, grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace k3moe
