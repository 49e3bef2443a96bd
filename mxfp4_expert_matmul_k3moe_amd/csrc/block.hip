// block.hip — the extras of a full decoder block around the routed experts:
// RMSNorm of the residual and the always-active bf16 shared expert (SwiGLU).
//
// The pages describe each MoE layer as the routed top-16 plus one shared expert kept
// at higher precision ("Kimi K3 纯 C 语言 CPU 推理实战", chenxutan.com/d/5901.html, §1.2
// and §2.3) and list an RMSNorm kernel among the engine's ops (project card "P053
// FareedKhan-dev/kimi-k3-in-c", architecture section). Both are HBM-streaming GEMVs at
// decode: bf16 weights are read once with 16-byte loads, widened to fp32 and
// multiplied against an fp32 activation staged in LDS.
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

// xhat = h / sqrt(mean(h^2) + eps) * gamma; the sum of squares runs in fp64 with a
// fixed per-thread order and reduction tree. Each thread holds its 4-element pieces of
// the row (16-byte loads, all in flight at once) through both passes.
constexpr int kNormPieces = 8;  // rows up to 256 * 4 * 8 = 8192 elements stay in registers
__global__ __launch_bounds__(256) void rmsnorm_kernel(int d, const float* __restrict__ h,
                                                      const uint16_t* __restrict__ gamma,
                                                      float eps, float* __restrict__ xhat) {
  __shared__ double red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const f32x4* ht = reinterpret_cast<const f32x4*>(h + (size_t)t * d);  // d % 8 == 0
  const int nq = d >> 2;
  const bool cached = nq <= 256 * kNormPieces;
  f32x4 v[kNormPieces];
  uint32_t gm[kNormPieces][4];  // gamma of the same pieces, requested with them
  if (cached) {
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = tid + 256 * c;
      const int qc = q < nq ? q : 0;
      v[c] = q < nq ? ht[q] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) gm[c][i] = gamma[4 * qc + i];
    }
  }
  double ss = 0.0;
  for (int q0 = 0; q0 < nq; q0 += 256 * kNormPieces)
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        const f32x4 a = cached ? v[c] : ht[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += (double)a[i] * (double)a[i];
      }
    }
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double inv = 1.0 / sqrt(((red[0] + red[1]) + (red[2] + red[3])) / (double)d + (double)eps);
  f32x4* out = reinterpret_cast<f32x4*>(xhat + (size_t)t * d);
  for (int q0 = 0; q0 < nq; q0 += 256 * kNormPieces)
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        const f32x4 a = cached ? v[c] : ht[q];
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = (float)((double)a[i] * inv *
                         (double)bf16_bits_to_f32(cached ? gm[c][i] : gamma[4 * q + i]));
        out[q] = o;
      }
    }
}

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

// out[t][r] = sum_c W[r][c] * x[t][c], one row group (rpw rows) per wave; two weight
// matrices at once when W2 is given (gate and up share the activation). Epilogue:
// SWIGLU ? silu(a)*b : a. A lane takes chunks sub, sub + lpr, ... in rounds of
// kGemvChunks whose loads all go out before their math. The grid may
// be smaller than the row groups: blocks then walk groups gridDim.x apart (the shared
// expert runs beside the routed path and is given a fraction of the CUs, so that the
// latency-bound router and top-k find room on every CU).
constexpr int kGemvChunks = 8;
template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void bf16_gemv_kernel(int T, int nrows, int ncols,
                                                           const float* __restrict__ x,
                                                           const uint16_t* __restrict__ W1,
                                                           const uint16_t* __restrict__ W2,
                                                           float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) f32x4 xs[];
  const int nch = ncols >> 3;
  const int lpr = gemv_lanes(nch), cpl = nch / lpr, rpw = 64 / lpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const int ngroups = (nrows + 4 * rpw - 1) / (4 * rpw);  // row groups of 4 waves
  for (int t = 0; t < T; ++t) {
    // the token is staged once per block and token; every group of the block uses it
    __syncthreads();  // the previous token's LDS reads are done
    stage_row(x + (size_t)t * ncols, ncols, lpr, xs);
    __syncthreads();
    for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
      const int r = (grp * 4 + wave) * rpw + rsel;
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

hipError_t launch_rmsnorm(int T, int d, const float* h, const uint16_t* gamma, float eps,
                          float* xhat, hipStream_t s) {
  rmsnorm_kernel<<<T, 256, 0, s>>>(d, h, gamma, eps, xhat);
  return hipGetLastError();
}

hipError_t launch_dense_swiglu(int T, int d, int f, const float* x, const uint16_t* wg,
                               const uint16_t* wu, const uint16_t* wd, float* hbuf, float* out,
                               hipStream_t s, int max_blocks) {
  // one row group per wave: at d = 7168, f = 1536 that is 384 and 448 groups of 4 waves,
  // walked by at most max_blocks blocks (0: one block per group)
  auto blocks = [&](int groups) {
    return (unsigned)(max_blocks > 0 && groups > max_blocks ? max_blocks : groups);
  };
  {
    const int rows = 4 * (64 / gemv_lanes(d >> 3));
    dim3 grid(blocks((f + rows - 1) / rows));
    bf16_gemv_kernel<true><<<grid, 256, (size_t)d * 4, s>>>(T, f, d, x, wg, wu, hbuf);
  }
  {
    const int rows = 4 * (64 / gemv_lanes(f >> 3));
    dim3 grid(blocks((d + rows - 1) / rows));
    bf16_gemv_kernel<false><<<grid, 256, (size_t)f * 4, s>>>(T, d, f, hbuf, wd, nullptr, out);
  }
  return hipGetLastError();
}

}  // namespace k3moe
