// ffn_mfma.hip — grouped expert GEMMs on bf16 MFMA for many tokens per expert (prefill).
//
// Each tile is 64 tokens of one expert (its bucket rows) times a slice of that expert's
// weight rows. The activation tile (bf16) is staged in LDS; each weight row's 32-element
// MXFP4 block is loaded with one 16-byte load per lane and decoded in registers straight
// into MFMA B operands, the E8M0 scale folded into the gfx950 scaled FP4->bf16
// conversion (exact: E2M1 values times a power of two fit bf16 for normal scales).
// v_mfma_f32_16x16x32_bf16 accumulates in fp32.
//
// K is walked in steps of 128 = 4 scale blocks. Within a step, lane group g = lane/16
// owns block g and feeds its 32 elements to four MFMAs, 8 per MFMA; the activation
// operand uses the same permutation of k, which leaves every dot product unchanged.
//
// Gate/up: h = silu(G x) * (U x), written as a pair of bf16 arrays h_hi = bf16(h),
// h_lo = bf16(h - h_hi), which together carry h to about 2^-16 relative.
// Down: z = D h_hi + D h_lo (two MFMAs per step on the same decoded B operand), fp32,
// one row per (token, slot) pair, combined later in slot order.
// Source of the form: "Kimi K3 纯 C 语言 CPU 推理实战" (chenxutan.com/d/5901.html) §1.2, §2.3.
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = kMfmaTileM;  // 64 tokens per tile
constexpr int BK = 128;         // K per step (4 MXFP4 blocks)
constexpr int APITCH = BK + 8;  // bf16 per LDS row: 272 B, rows land on distinct banks
constexpr int kWaves = 4;

__device__ __forceinline__ int tile_expert(const int32_t* mtile_off, int n_act, int mt) {
  int lo = 0, hi = n_act - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mtile_off[mid] <= mt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One MXFP4 block (16 bytes, 32 elements) with its scale -> 4 MFMA B operands of 8 bf16.
__device__ __forceinline__ void decode_b(const u32x4 q, float sc, bf16x8 out[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 v;
    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 0));
    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 1));
    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 2));
    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], sc, 3));
    out[i] = __builtin_bit_cast(bf16x8, v);
  }
}

struct MfmaArgs {
  int T, d, f, k;
  const uint16_t* a_src;  // gate/up: x [T][d]; down: h_hi [P][f]
  const uint16_t* a_lo;   // down: h_lo [P][f]
  const uint8_t *q0, *s0, *q1, *s1;  // gate/up: G and U; down: D (q1 unused)
  const int32_t *offsets, *rows, *act, *n_act, *mtile_off;
  int nblk_n;
  uint16_t* h_out;  // gate/up output: h_hi
  uint16_t* h_lo;   // gate/up output: h_lo
  float* z_out;     // down output
};

// GATEUP: N slice = 128 rows j (each wave 32 j, as 2 gate + 2 up 16-wide tiles).
// DOWN:   N slice = 256 rows i (each wave 64 i, as 4 tiles).
template <bool GATEUP>
__global__ __launch_bounds__(256) void mfma_ffn_kernel(MfmaArgs a) {
  constexpr int NA = GATEUP ? 1 : 2;  // activation tiles per stage: x, or h_hi and h_lo
  __shared__ __attribute__((aligned(16))) uint16_t As[2][NA][BM * APITCH];
  const int n_act = *a.n_act;
  const int mt_glob = blockIdx.x / a.nblk_n;
  const int nb = blockIdx.x - mt_glob * a.nblk_n;
  if (n_act <= 0 || mt_glob >= a.mtile_off[n_act]) return;
  const int ai = tile_expert(a.mtile_off, n_act, mt_glob);
  const int e = a.act[ai];
  const int P = a.T * a.k;
  const int pe0 = min(max(a.offsets[e], 0), P), pe1 = min(max(a.offsets[e + 1], pe0), P);
  const int p0 = pe0 + (mt_glob - a.mtile_off[ai]) * BM;
  const int pn = max(0, min(BM, pe1 - p0));
  const int K = GATEUP ? a.d : a.f;     // contraction length
  const int NR = GATEUP ? a.f : a.d;    // weight rows of one matrix
  const int KB = K >> 5;                // scale blocks per weight row
  const size_t rq = (size_t)(K >> 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, g = lane >> 4;

  // staging assignment: 4 threads per tile row, 32 k (64 bytes) each
  const int sr = tid >> 2, sq = tid & 3;
  const uint16_t* srow[NA];
#pragma unroll
  for (int v = 0; v < NA; ++v) srow[v] = nullptr;
  if (sr < pn) {
    if (GATEUP) {
      const int pair = a.rows[p0 + sr];
      if (pair >= 0 && pair < P) srow[0] = a.a_src + (size_t)(pair / a.k) * a.d;
    } else {
      srow[0] = a.a_src + (size_t)(p0 + sr) * a.f;
      srow[NA - 1] = a.a_lo + (size_t)(p0 + sr) * a.f;
    }
  }

  // weight rows of this lane's N tiles
  constexpr int NT = 4;
  const uint8_t* wq[NT];
  const uint8_t* wsc[NT];
  bool wv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int r;
    const uint8_t *qb, *sb;
    if (GATEUP) {
      // tiles 0,1: gate rows; tiles 2,3: the same rows of up
      r = nb * 128 + wave * 32 + (nt & 1) * 16 + ln;
      qb = (nt < 2) ? a.q0 : a.q1;
      sb = (nt < 2) ? a.s0 : a.s1;
    } else {
      r = nb * 256 + wave * 64 + nt * 16 + ln;
      qb = a.q0;
      sb = a.s0;
    }
    wv[nt] = r < NR;
    const size_t row = (size_t)e * NR + (wv[nt] ? r : 0);
    wq[nt] = qb + row * rq;
    wsc[nt] = sb + row * KB;
  }

  f32x4 acc[4][NT];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[m][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  u32x4 stg[NA][4];
  auto load_a = [&](int ks) {
    const int k0 = ks * BK + sq * 32;
#pragma unroll
    for (int v = 0; v < NA; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = srow[v] != nullptr && (k0 + 8 * c) < K;
        stg[v][c] = ok ? *reinterpret_cast<const u32x4*>(srow[v] + k0 + 8 * c)
                       : u32x4{0u, 0u, 0u, 0u};
      }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int v = 0; v < NA; ++v) {
      uint16_t* dst = &As[buf][v][sr * APITCH + sq * 32];
#pragma unroll
      for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(dst + 8 * c) = stg[v][c];
    }
  };
  u32x4 bq[NT];
  uint32_t bs[NT];
  auto load_b = [&](int ks) {
    const int kb = ks * 4 + g;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bool ok = wv[nt] && kb < KB;
      bq[nt] = ok ? load_u32x4_nt(wq[nt] + (size_t)kb * 16) : u32x4{0u, 0u, 0u, 0u};
      bs[nt] = ok ? (uint32_t)wsc[nt][kb] : 127u;
    }
  };

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    bf16x8 bop[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) decode_b(bq[nt], e8m0_to_f32(bs[nt]), bop[nt]);
    if (ks + 1 < nk) {
      load_a(ks + 1);
      load_b(ks + 1);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int v = 0; v < NA; ++v) {
        const uint16_t* arow = &As[buf][v][(16 * m + ln) * APITCH + 32 * g];
        bf16x8 aop[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) aop[i] = *reinterpret_cast<const bf16x8*>(arow + 8 * i);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[m][nt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[i], bop[nt][i], acc[m][nt], 0, 0, 0);
      }
    }
    if (ks + 1 < nk) {
      store_a(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds rows 4*g .. 4*g+3 of column ln of each 16x16 tile
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * m + 4 * g + r;
      if (row >= pn) continue;
      if (GATEUP) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int j = nb * 128 + wave * 32 + nt * 16 + ln;
          if (j < a.f) {
            const float hv = silu_f32(acc[m][nt][r]) * acc[m][nt + 2][r];
            const uint16_t hi = f32_to_bf16_rne(hv);
            const size_t o = (size_t)(p0 + row) * a.f + j;
            a.h_out[o] = hi;
            a.h_lo[o] = f32_to_bf16_rne(hv - bf16_bits_to_f32(hi));
          }
        }
      } else {
        const int pair = a.rows[p0 + row];
        if (pair < 0 || pair >= P) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int i = nb * 256 + wave * 64 + nt * 16 + ln;
          if (i < a.d) a.z_out[(size_t)pair * a.d + i] = acc[m][nt][r];
        }
      }
    }
  }
}

}  // namespace

int mfma_mtiles_bound(int T, int E, int k) {
  const long P = (long)T * k;
  const long act = P < E ? P : E;
  return (int)(act + P / BM + 1);
}

bool mfma_shape_supported(int d, int f) { return d % 32 == 0 && f % 32 == 0; }

hipError_t launch_gateup_mfma(int T, int d, int f, int E, int k, const uint16_t* x,
                              const MxPtrs& w, const int32_t* offsets, const int32_t* rows,
                              const int32_t* act, const int32_t* n_act,
                              const int32_t* mtile_off, uint16_t* h, hipStream_t s) {
  MfmaArgs a{};
  a.T = T; a.d = d; a.f = f; a.k = k; a.a_src = x;
  a.q0 = w.gate_q; a.s0 = w.gate_s; a.q1 = w.up_q; a.s1 = w.up_s;
  a.offsets = offsets; a.rows = rows; a.act = act; a.n_act = n_act; a.mtile_off = mtile_off;
  a.nblk_n = (f + 127) / 128;
  a.h_out = h;
  a.h_lo = h + (size_t)T * k * f;
  dim3 grid((unsigned)(mfma_mtiles_bound(T, E, k) * a.nblk_n));
  mfma_ffn_kernel<true><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_mfma(int T, int d, int f, int E, int k, const MxPtrs& w,
                            const uint16_t* h, const int32_t* offsets, const int32_t* rows,
                            const int32_t* act, const int32_t* n_act, const int32_t* mtile_off,
                            float* z, hipStream_t s) {
  MfmaArgs a{};
  a.T = T; a.d = d; a.f = f; a.k = k; a.a_src = h;
  a.a_lo = h + (size_t)T * k * f;
  a.q0 = w.down_q; a.s0 = w.down_s;
  a.offsets = offsets; a.rows = rows; a.act = act; a.n_act = n_act; a.mtile_off = mtile_off;
  a.nblk_n = (d + 255) / 256;
  a.z_out = z;
  dim3 grid((unsigned)(mfma_mtiles_bound(T, E, k) * a.nblk_n));
  mfma_ffn_kernel<false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace k3moe
