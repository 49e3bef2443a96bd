// block_dev.h — device routines of the decoder-block extras, shared by their standalone
// kernels (block.hip) and by the routing launches that carry them at one token (router.hip):
// the RMSNorm of the residual and the bf16-weight GEMV of the shared expert.
//
// RMSNorm ("P053 FareedKhan-dev/kimi-k3-in-c", architecture section: an RMSNorm kernel among
// the engine's ops): xhat = h / sqrt(mean(h^2) + eps) * gamma, the sum of squares in fp64.
// Shared expert ("Kimi K3 纯 C 语言 CPU 推理实战", chenxutan.com/d/5901.html, §1.2 and §2.3:
// kept at higher precision than the routed ones): bf16 weights read once with 16-byte loads,
// widened to fp32 and multiplied against an fp32 activation row staged in LDS.
#pragma once
#include "k3moe_device.h"

namespace k3moe {
namespace {

// ---- RMSNorm of one fp32 row by a block of 256 threads ------------------------------------
// Thread tid holds the 4-element pieces q = tid + 256 c of the row and of gamma (16-byte loads
// of h, all requested at once), for rows up to kNormMaxD elements (d % 4 == 0).
constexpr int kNormPieces = 8;
constexpr int kNormMaxD = 256 * 4 * kNormPieces;
struct NormPieces {
  f32x4 v[kNormPieces];
  uint32_t gm[kNormPieces][2];  // gamma of the same pieces, two bf16 per word (low first)
};
__device__ __forceinline__ void norm_load_h(const float* __restrict__ h, int d,
                                            f32x4 (&v)[kNormPieces]) {
  const f32x4* h4 = reinterpret_cast<const f32x4*>(h);
  const int nq = d >> 2, tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < kNormPieces; ++c) {
    const int q = tid + 256 * c;
    v[c] = q < nq ? h4[q] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}
__device__ __forceinline__ void norm_load(const float* __restrict__ h,
                                          const uint16_t* __restrict__ gamma, int d,
                                          NormPieces& p) {
  norm_load_h(h, d, p.v);
  const int nq = d >> 2, tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < kNormPieces; ++c) {
    const int q = tid + 256 * c;
    const int qc = q < nq ? q : 0;
    p.gm[c][0] = (uint32_t)gamma[4 * qc] | ((uint32_t)gamma[4 * qc + 1] << 16);
    p.gm[c][1] = (uint32_t)gamma[4 * qc + 2] | ((uint32_t)gamma[4 * qc + 3] << 16);
  }
}
// 1 / sqrt(mean(h^2) + eps): per thread the squares of its pieces in order, an xor tree over
// the wave, then the four wave sums in a fixed order (the same value in every block that runs
// it on the same row). red: 4 doubles of LDS, not in use by the caller.
__device__ __forceinline__ double norm_inv(const f32x4 (&v)[kNormPieces], int d, float eps,
                                           double* red) {
  const int nq = d >> 2, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < kNormPieces; ++c)
    if (tid + 256 * c < nq)
#pragma unroll
      for (int i = 0; i < 4; ++i) ss += (double)v[c][i] * (double)v[c][i];
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  return 1.0 / sqrt(((red[0] + red[1]) + (red[2] + red[3])) / (double)d + (double)eps);
}
__device__ __forceinline__ float norm_value(float hv, uint32_t g16, double inv) {
  return (float)((double)hv * inv * (double)bf16_bits_to_f32(g16));
}
// xhat of element i of piece c
__device__ __forceinline__ float norm_out(const NormPieces& p, int c, int i, double inv) {
  return norm_value(p.v[c][i], (p.gm[c][i >> 1] >> (16 * (i & 1))) & 0xFFFFu, inv);
}

// ---- bf16 GEMV --------------------------------------------------------------------------
// LDS layout of an fp32 activation row for 8-element chunks: chunk c = sub + lpr*i,
// half hh (4 floats) goes to slot ((i*2 + hh)*lpr + sub), so a lane group reads
// consecutive 16-byte slots.
__device__ __forceinline__ int xs_slot(int c, int hh, int lpr) {
  const int i = c / lpr, sub = c - i * lpr;
  return (i * 2 + hh) * lpr + sub;
}

__device__ __forceinline__ float bf16x8_dot(const u32x4 w, const f32x4 a, const f32x4 b, float acc) {
  acc = fmaf(__uint_as_float(w[0] << 16), a[0], acc);
  acc = fmaf(__uint_as_float(w[0] & 0xFFFF0000u), a[1], acc);
  acc = fmaf(__uint_as_float(w[1] << 16), a[2], acc);
  acc = fmaf(__uint_as_float(w[1] & 0xFFFF0000u), a[3], acc);
  acc = fmaf(__uint_as_float(w[2] << 16), b[0], acc);
  acc = fmaf(__uint_as_float(w[2] & 0xFFFF0000u), b[1], acc);
  acc = fmaf(__uint_as_float(w[3] << 16), b[2], acc);
  acc = fmaf(__uint_as_float(w[3] & 0xFFFF0000u), b[3], acc);
  return acc;
}

// Stage one fp32 row (n elements, n % 8 == 0) into the slot layout.
__device__ __forceinline__ void stage_row(const float* src, int n, int lpr, f32x4* xs) {
  const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
  for (int v = threadIdx.x; v < n / 4; v += blockDim.x) {
    const int c = v >> 1, hh = v & 1;
    xs[xs_slot(c, hh, lpr)] = s4[v];
  }
}

// Lane-group width for a row of nch 8-element chunks: the largest power of two <= 64
// dividing nch that still leaves each lane at least 8 chunks (short rows get narrower
// groups and more rows per wave).
__host__ __device__ inline int gemv_lanes(int nch) {
  int l = lanes_per_row(nch);
  while (l > 1 && nch / l < 8) l >>= 1;
  return l;
}
// Rows one row group covers: one row group of nw waves, rpw rows per wave.
__host__ __device__ inline int gemv_group_rows(int ncols, int nw) {
  return nw * (64 / gemv_lanes(ncols >> 3));
}

// Token staging for bf16_gemv_rows: issue() runs before the block's first weights are
// requested, stage(t, lpr, xs) between two block barriers and writes token t into the slot
// layout. StageRow copies an fp32 row from memory; StageNormRow (one token, 256 threads)
// writes the RMSNorm of the residual row h, from pieces requested in issue().
struct StageRow {
  const float* x;
  int ncols;
  __device__ __forceinline__ void issue() {}
  __device__ __forceinline__ void stage(int t, int lpr, f32x4* xs) {
    stage_row(x + (size_t)t * ncols, ncols, lpr, xs);
  }
};
struct StageNormRow {
  const float* h;
  const uint16_t* gamma;
  int d;
  float eps;
  double* red;  // 4 doubles of LDS
  NormPieces p;
  __device__ __forceinline__ void issue() { norm_load(h, gamma, d, p); }
  __device__ __forceinline__ void stage(int, int lpr, f32x4* xs) {
    const double inv = norm_inv(p.v, d, eps, red);
    const int nq = d >> 2;
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = threadIdx.x + 256 * c;  // piece q = half q & 1 of 8-element chunk q >> 1
      if (q < nq) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = norm_out(p, c, i, inv);
        xs[xs_slot(q >> 1, q & 1, lpr)] = o;
      }
    }
  }
};

// out[t][r] = sum_c W[r][c] * x[t][c] for the row groups bid, bid + nblk, ... of this block
// (a row group = one row slice per wave, all waves of the block); two weight matrices at once
// when SWIGLU (gate and up share the activation), epilogue silu(a) * b. A lane takes chunks
// sub, sub + lpr, ... in rounds of kGemvChunks whose loads all go out before their math (the
// first round of the block's first group before the token is staged).
// xs: LDS for one staged activation row (ncols floats); stg stages the token (StageRow,
// StageNormRow). Every thread of the block calls it (it has block barriers); each row's sum
// depends only on the lane-group layout, not on the block size.
constexpr int kGemvChunks = 8;
template <bool SWIGLU, class Stager>
__device__ __forceinline__ void bf16_gemv_rows(int bid, int nblk, int T, int nrows, int ncols,
                                               Stager& stg, const uint16_t* __restrict__ W1,
                                               const uint16_t* __restrict__ W2,
                                               float* __restrict__ out, f32x4* xs) {
  const int nch = ncols >> 3;
  const int lpr = gemv_lanes(nch), cpl = nch / lpr, rpw = 64 / lpr;
  const int nw = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const int ngroups = (nrows + nw * rpw - 1) / (nw * rpw);
  int r = 0;
  bool rv = false;
  const uint16_t *w1 = W1, *w2 = W2;
  u32x4 v1[kGemvChunks], v2[kGemvChunks];
  auto setup = [&](int grp) {
    r = (grp * nw + wave) * rpw + rsel;
    rv = r < nrows;
    const int rr = rv ? r : nrows - 1;  // loads stay in bounds; results of !rv are dropped
    w1 = W1 + (size_t)rr * ncols + (size_t)sub * 8;
    if (SWIGLU) w2 = W2 + (size_t)rr * ncols + (size_t)sub * 8;
  };
  auto load_round = [&](int i0) {
#pragma unroll
    for (int i = 0; i < kGemvChunks; ++i) {
      if (i0 + i < cpl) {
        const size_t off = (size_t)lpr * (i0 + i) * 8;
        v1[i] = load_u32x4_nt(reinterpret_cast<const uint8_t*>(w1 + off));
        if (SWIGLU) v2[i] = load_u32x4_nt(reinterpret_cast<const uint8_t*>(w2 + off));
      }
    }
  };
  for (int t = 0; t < T; ++t) {
    // the first round of weights of the block's first group goes out before the token is
    // staged (the weights do not depend on it), so the two round trips overlap
    if (t == 0) stg.issue();
    if (bid < ngroups) {
      setup(bid);
      load_round(0);
    }
    // the token is staged once per block and token; every group of the block uses it
    __syncthreads();  // the previous token's LDS reads are done
    stg.stage(t, lpr, xs);
    __syncthreads();
    for (int grp = bid; grp < ngroups; grp += nblk) {
      if (grp != bid) {
        setup(grp);
        load_round(0);
      }
      float a1 = 0.0f, a2 = 0.0f;
      for (int i0 = 0; i0 < cpl; i0 += kGemvChunks) {
        if (i0 > 0) load_round(i0);
#pragma unroll
        for (int i = 0; i < kGemvChunks; ++i) {
          if (i0 + i < cpl) {
            const int c = sub + lpr * (i0 + i);
            const f32x4 xa = xs[xs_slot(c, 0, lpr)], xb = xs[xs_slot(c, 1, lpr)];
            a1 = bf16x8_dot(v1[i], xa, xb, a1);
            if (SWIGLU) a2 = bf16x8_dot(v2[i], xa, xb, a2);
          }
        }
      }
      a1 = group_sum_rt(a1, lpr);
      if (SWIGLU) a2 = group_sum_rt(a2, lpr);
      if (rv && sub == 0) out[(size_t)t * nrows + r] = SWIGLU ? silu_f32(a1) * a2 : a1;
    }
  }
}

}  // namespace
}  // namespace k3moe
