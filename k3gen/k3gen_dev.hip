/*
 * k3gen_dev.hip — device-side fill of the integer draws of k3gen.h, so that
 * multi-gigabyte synthetic expert tensors can be produced directly in HBM
 * instead of being copied over PCIe. It implements the same SplitMix64
 * counter form as k3gen.c (published definition), and a GPU test checks the
 * two bit for bit. Input drawing only: nothing here decodes or multiplies.
 *
 * Layout written: dst[e * per_expert + j] = draw j of the stream keyed by
 * k3gen_key(seed, layer, tag, e), for e in [0, E) and j in [0, per_expert).
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t at(uint64_t key, uint64_t i) {
  return mix(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

__global__ void fill_bytes_kernel(uint64_t seed, uint64_t layer, uint64_t tag,
                                  uint64_t per_expert, uint8_t* __restrict__ dst) {
  const uint64_t e = blockIdx.y;
  const uint64_t key = at(at(at(seed, layer), tag), e);
  uint8_t* out = dst + e * per_expert;
  const uint64_t nwords = (per_expert + 7) >> 3;
  const bool aligned = ((reinterpret_cast<uintptr_t>(out) & 7) == 0);
  for (uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t v = at(key, w);
    uint64_t b0 = w << 3;
    if (aligned && b0 + 8 <= per_expert) {
      *reinterpret_cast<uint64_t*>(out + b0) = v;
    } else {
      for (int b = 0; b < 8 && b0 + b < per_expert; ++b) out[b0 + b] = (uint8_t)(v >> (8 * b));
    }
  }
}

__global__ void fill_e8m0_kernel(uint64_t seed, uint64_t layer, uint64_t tag,
                                 uint64_t per_expert, int lo, int count,
                                 uint8_t* __restrict__ dst) {
  const uint64_t e = blockIdx.y;
  const uint64_t key = at(at(at(seed, layer), tag), e);
  uint8_t* out = dst + e * per_expert;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < per_expert;
       j += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t hi = at(key, j) >> 32;
    out[j] = (uint8_t)(lo + (int)((hi * (uint64_t)count) >> 32));
  }
}

unsigned grid_x(uint64_t items) {
  uint64_t g = (items + 255) / 256;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

/* Returns 0 on success, -1 on bad arguments, -4 on a HIP launch error. */
int k3gen_dev_fill_bytes(uint64_t seed, uint64_t layer, uint64_t tag, int32_t E,
                         uint64_t per_expert, uint8_t* dst, void* stream) {
  if (E < 0 || E > 65535 || (dst == nullptr && E > 0 && per_expert > 0)) return -1;
  if (E == 0 || per_expert == 0) return 0;
  dim3 grid(grid_x((per_expert + 7) >> 3), (unsigned)E);
  hipLaunchKernelGGL(fill_bytes_kernel, grid, dim3(256), 0, (hipStream_t)stream, seed,
                     layer, tag, per_expert, dst);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int k3gen_dev_fill_e8m0(uint64_t seed, uint64_t layer, uint64_t tag, int32_t E,
                        uint64_t per_expert, int lo, int count, uint8_t* dst,
                        void* stream) {
  if (E < 0 || E > 65535 || count < 1 || lo < 0 || lo + count > 256) return -1;
  if (dst == nullptr && E > 0 && per_expert > 0) return -1;
  if (E == 0 || per_expert == 0) return 0;
  dim3 grid(grid_x(per_expert), (unsigned)E);
  hipLaunchKernelGGL(fill_e8m0_kernel, grid, dim3(256), 0, (hipStream_t)stream, seed,
                     layer, tag, per_expert, lo, count, dst);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
