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
// fixed per-thread order and reduction tree.
__global__ __launch_bounds__(256) void rmsnorm_kernel(int d, const float* __restrict__ h,
                                                      const uint16_t* __restrict__ gamma,
                                                      float eps, float* __restrict__ xhat) {
  __shared__ double red[256];
  const int t = blockIdx.x;
  const float* ht = h + (size_t)t * d;
  double ss = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) {
    const double v = (double)ht[i];
    ss += v * v;
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  const double r = sqrt(red[0] / (double)d + (double)eps);
  for (int i = threadIdx.x; i < d; i += 256)
    xhat[(size_t)t * d + i] = (float)((double)ht[i] / r * (double)bf16_bits_to_f32(gamma[i]));
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

// out[t][r] = sum_c W[r][c] * x[t][c] for a chunk of rows; two weight matrices at once
// when W2 is given (gate and up share the activation). Epilogue: SWIGLU ? silu(a)*b : a.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void bf16_gemv_kernel(int T, int nrows, int ncols,
                                                        const float* __restrict__ x,
                                                        const uint16_t* __restrict__ W1,
                                                        const uint16_t* __restrict__ W2,
                                                        int rc, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) f32x4 xs[];
  const int nch = ncols >> 3;
  const int lpr = lanes_per_row(nch), cpl = nch / lpr, rpw = 64 / lpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const int r0 = blockIdx.x * rc, r1 = min(nrows, r0 + rc);
  for (int t = 0; t < T; ++t) {
    __syncthreads();
    stage_row(x + (size_t)t * ncols, ncols, lpr, xs);
    __syncthreads();
    for (int rb = r0 + wave * rpw; rb < r1; rb += 4 * rpw) {
      const int r = rb + rsel;
      const bool rv = r < r1;
      float a1 = 0.0f, a2 = 0.0f;
      if (rv) {
        const uint16_t* w1 = W1 + (size_t)r * ncols;
        const uint16_t* w2 = SWIGLU ? W2 + (size_t)r * ncols : nullptr;
        int i = 0;
        for (; i + 4 <= cpl; i += 4) {
          u32x4 v1[4], v2[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = sub + lpr * (i + u);
            v1[u] = load_u32x4_nt(reinterpret_cast<const uint8_t*>(w1 + (size_t)c * 8));
            if (SWIGLU) v2[u] = load_u32x4_nt(reinterpret_cast<const uint8_t*>(w2 + (size_t)c * 8));
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = sub + lpr * (i + u);
            const f32x4 xa = xs[xs_slot(c, 0, lpr)], xb = xs[xs_slot(c, 1, lpr)];
            a1 = bf16x8_dot(v1[u], xa, xb, a1);
            if (SWIGLU) a2 = bf16x8_dot(v2[u], xa, xb, a2);
          }
        }
        for (; i < cpl; ++i) {
          const int c = sub + lpr * i;
          const u32x4 v1 = load_u32x4_nt(reinterpret_cast<const uint8_t*>(w1 + (size_t)c * 8));
          const f32x4 xa = xs[xs_slot(c, 0, lpr)], xb = xs[xs_slot(c, 1, lpr)];
          a1 = bf16x8_dot(v1, xa, xb, a1);
          if (SWIGLU) {
            const u32x4 v2 = load_u32x4_nt(reinterpret_cast<const uint8_t*>(w2 + (size_t)c * 8));
            a2 = bf16x8_dot(v2, xa, xb, a2);
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
                               hipStream_t s) {
  {
    const int lpr = lanes_per_row(d >> 3), rpw = 64 / lpr;
    const int rc = 4 * rpw * 2;
    dim3 grid((unsigned)((f + rc - 1) / rc));
    bf16_gemv_kernel<true><<<grid, 256, (size_t)d * 4, s>>>(T, f, d, x, wg, wu, rc, hbuf);
  }
  {
    const int lpr = lanes_per_row(f >> 3), rpw = 64 / lpr;
    const int rc = 4 * rpw * 2;
    dim3 grid((unsigned)((d + rc - 1) / rc));
    bf16_gemv_kernel<false><<<grid, 256, (size_t)f * 4, s>>>(T, d, f, hbuf, wd, nullptr, rc, out);
  }
  return hipGetLastError();
}

}  // namespace k3moe
