// gemv_bf16.h — the bf16-weight GEMV of the shared expert as a block-level routine, so that
// the standalone shared-expert kernels (block.hip) and the routing launches that carry the
// shared expert beside the router and the top-k (router.hip) run the same code.
//
// bf16 weights are read once with 16-byte loads, widened to fp32 and multiplied against an
// fp32 activation row staged in LDS ("Kimi K3 纯 C 语言 CPU 推理实战", chenxutan.com/d/5901.html,
// §1.2 and §2.3: the shared expert is kept at higher precision than the routed ones).
#pragma once
#include "k3moe_device.h"

namespace k3moe {
namespace {

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

// out[t][r] = sum_c W[r][c] * x[t][c] for the row groups bid, bid + nblk, ... of this block
// (a row group = one row slice per wave, all waves of the block); two weight matrices at once
// when SWIGLU (gate and up share the activation), epilogue silu(a) * b. A lane takes chunks
// sub, sub + lpr, ... in rounds of kGemvChunks whose loads all go out before their math.
// xs: LDS for one staged activation row (ncols floats). Every thread of the block calls it
// (it has block barriers); each row's sum depends only on the lane-group layout, not on the
// block size.
constexpr int kGemvChunks = 8;
template <bool SWIGLU>
__device__ __forceinline__ void bf16_gemv_rows(int bid, int nblk, int T, int nrows, int ncols,
                                               const float* __restrict__ x,
                                               const uint16_t* __restrict__ W1,
                                               const uint16_t* __restrict__ W2,
                                               float* __restrict__ out, f32x4* xs) {
  const int nch = ncols >> 3;
  const int lpr = gemv_lanes(nch), cpl = nch / lpr, rpw = 64 / lpr;
  const int nw = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const int ngroups = (nrows + nw * rpw - 1) / (nw * rpw);
  for (int t = 0; t < T; ++t) {
    // the token is staged once per block and token; every group of the block uses it
    __syncthreads();  // the previous token's LDS reads are done
    stage_row(x + (size_t)t * ncols, ncols, lpr, xs);
    __syncthreads();
    for (int grp = bid; grp < ngroups; grp += nblk) {
      const int r = (grp * nw + wave) * rpw + rsel;
      const bool rv = r < nrows;
      const int rr = rv ? r : nrows - 1;  // loads stay in bounds; results of !rv are dropped
      const uint16_t* w1 = W1 + (size_t)rr * ncols + (size_t)sub * 8;
      const uint16_t* w2 = SWIGLU ? W2 + (size_t)rr * ncols + (size_t)sub * 8 : nullptr;
      u32x4 v1[kGemvChunks], v2[kGemvChunks];
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
      float a1 = 0.0f, a2 = 0.0f;
      for (int i0 = 0; i0 < cpl; i0 += kGemvChunks) {
        load_round(i0);
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
