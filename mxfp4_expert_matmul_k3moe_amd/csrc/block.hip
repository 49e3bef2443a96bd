// block.hip — the extras of a full decoder block around the routed experts:
// RMSNorm of the residual and the always-active bf16 shared expert (SwiGLU).
//
// The pages describe each MoE layer as the routed top-16 plus one shared expert kept
// at higher precision ("Kimi K3 纯 C 语言 CPU 推理实战", chenxutan.com/d/5901.html, §1.2
// and §2.3) and list an RMSNorm kernel among the engine's ops (project card "P053
// FareedKhan-dev/kimi-k3-in-c", architecture section). Both are HBM-streaming GEMVs at
// decode: bf16 weights are read once with 16-byte loads, widened to fp32 and
// multiplied against an fp32 activation staged in LDS.
#include "block_dev.h"
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

// xhat = h / sqrt(mean(h^2) + eps) * gamma, one block of 256 threads per row; rows up to
// kNormMaxD elements stay in registers between the two passes (norm_load / norm_inv), longer
// ones are read again with the same per-thread order and reduction tree.
__global__ __launch_bounds__(256) void rmsnorm_kernel(int d, const float* __restrict__ h,
                                                      const uint16_t* __restrict__ gamma,
                                                      float eps, float* __restrict__ xhat) {
  __shared__ double red[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* ht = h + (size_t)t * d;  // d % 8 == 0
  f32x4* out = reinterpret_cast<f32x4*>(xhat + (size_t)t * d);
  const int nq = d >> 2;
  if (d <= kNormMaxD) {
    NormPieces p;
    norm_load(ht, gamma, d, p);
    const double inv = norm_inv(p.v, d, eps, red);
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = tid + 256 * c;
      if (q < nq) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = norm_out(p, c, i, inv);
        out[q] = o;
      }
    }
    return;
  }
  const f32x4* h4 = reinterpret_cast<const f32x4*>(ht);
  double ss = 0.0;
  for (int q0 = 0; q0 < nq; q0 += 256 * kNormPieces)
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        const f32x4 a = h4[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += (double)a[i] * (double)a[i];
      }
    }
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double inv = 1.0 / sqrt(((red[0] + red[1]) + (red[2] + red[3])) / (double)d + (double)eps);
  for (int q0 = 0; q0 < nq; q0 += 256 * kNormPieces)
#pragma unroll
    for (int c = 0; c < kNormPieces; ++c) {
      const int q = q0 + tid + 256 * c;
      if (q < nq) {
        const f32x4 a = h4[q];
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = norm_value(a[i], gamma[4 * q + i], inv);
        out[q] = o;
      }
    }
}

// out[t][r] = W[r] . x[t] for every row, one row group (4 waves) per block when the grid
// covers the groups; a smaller grid walks them gridDim.x apart (the shared expert beside the
// routed path on a side stream takes a fraction of the CUs, so that the latency-bound router
// and top-k find room on every CU).
template <bool SWIGLU>
__global__ __launch_bounds__(256, 2) void bf16_gemv_kernel(int T, int nrows, int ncols,
                                                           const float* __restrict__ x,
                                                           const uint16_t* __restrict__ W1,
                                                           const uint16_t* __restrict__ W2,
                                                           float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) f32x4 xs[];
  StageRow stg{x, ncols};
  bf16_gemv_rows<SWIGLU>(blockIdx.x, gridDim.x, T, nrows, ncols, stg, W1, W2, out, xs);
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
    const int rows = gemv_group_rows(d, 4);
    dim3 grid(blocks((f + rows - 1) / rows));
    bf16_gemv_kernel<true><<<grid, 256, (size_t)d * 4, s>>>(T, f, d, x, wg, wu, hbuf);
  }
  {
    const int rows = gemv_group_rows(f, 4);
    dim3 grid(blocks((d + rows - 1) / rows));
    bf16_gemv_kernel<false><<<grid, 256, (size_t)f * 4, s>>>(T, d, f, hbuf, wd, nullptr, out);
  }
  return hipGetLastError();
}

}  // namespace k3moe
