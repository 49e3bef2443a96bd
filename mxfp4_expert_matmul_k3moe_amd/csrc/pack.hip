// pack.hip — the packed ("tiled") MXFP4 layout of the expert matrices.
//
// The row-major layout puts each weight row's 32-element blocks one after another, so the 16
// rows that one block-scaled MFMA takes as its FP4 operand lie 3584 bytes (gate/up) or 768
// bytes (down) apart and one operand load can read only 64 contiguous bytes per row. The
// packed layout stores each operand tile contiguously, in the order the MFMA's lanes hold it,
// so that one 16-byte-per-lane load reads 1 KB in one piece. Nothing is decoded: the bytes are
// the same 4-bit codes and E8M0 scales, permuted.
//
// For an MXFP4 matrix [R][K] (R % 16 == 0, K % 128 == 0), nk = K / 128 steps of 128 elements
// and nch = ceil(nk / 8) chunks of 8 steps, tile t holding rows 16 t .. 16 t + 15:
//   codes   [R/16][nk][64][16 B]: entry (t, s, L), L = i + 16 g (i < 16, g < 4), holds bytes
//           [64 s + 16 g, 64 s + 16 g + 16) of row 16 t + i (elements 128 s + 32 g .. + 31);
//   scales  [R/16][nch][64][8 B]: byte j of entry (t, c, L) is the E8M0 scale of block
//           4 (8 c + j) + g of row 16 t + i, 0 where 8 c + j >= nk.
// The scale format and the element order inside a 16-byte piece are those of the row-major
// layout ("Kimi K3 纯 C 语言 CPU 推理实战" §2.3: [N][K] weights with one scale per 32 consecutive
// K elements; project card "P053 FareedKhan-dev/kimi-k3-in-c", core features: MXFP4).
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

// One 16-byte piece of the packed codes per thread, over `n_mat` stacked matrices.
__global__ __launch_bounds__(256) void pack_codes_kernel(int R, int K, long long total,
                                                         const uint8_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst) {
  const long long o = (long long)blockIdx.x * 256 + threadIdx.x;  // piece index
  if (o >= total) return;
  const int nk = K / 128;
  const long long per_mat = (long long)R * K / 32;  // pieces per matrix
  const long long mat = o / per_mat;
  long long r = o - mat * per_mat;
  const int L = (int)(r & 63);
  r >>= 6;
  const int s = (int)(r % nk);
  const long long t = r / nk;
  const int i = L & 15, g = L >> 4;
  const size_t row = (size_t)(t * 16 + i);
  const uint8_t* p = src + (size_t)mat * R * (K / 2) + row * (K / 2) + 64 * s + 16 * g;
  *reinterpret_cast<u32x4*>(dst + (size_t)o * 16) = *reinterpret_cast<const u32x4*>(p);
}

// One 8-byte scale entry per thread.
__global__ __launch_bounds__(256) void pack_scales_kernel(int R, int K, long long total,
                                                          const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst) {
  const long long o = (long long)blockIdx.x * 256 + threadIdx.x;  // entry index
  if (o >= total) return;
  const int nk = K / 128, nch = (nk + 7) / 8, KB = K / 32;
  const long long per_mat = (long long)(R / 16) * nch * 64;
  const long long mat = o / per_mat;
  long long r = o - mat * per_mat;
  const int L = (int)(r & 63);
  r >>= 6;
  const int c = (int)(r % nch);
  const long long t = r / nch;
  const int i = L & 15, g = L >> 4;
  const uint8_t* rowp = src + (size_t)mat * R * KB + (size_t)(t * 16 + i) * KB;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int s = 8 * c + j;
    const uint32_t b = s < nk ? rowp[4 * s + g] : 0u;
    w[j >> 2] |= b << (8 * (j & 3));
  }
  *reinterpret_cast<uint2*>(dst + (size_t)o * 8) = make_uint2(w[0], w[1]);
}

}  // namespace

size_t packed_scale_bytes(int R, int K) {
  const int nk = K / 128, nch = (nk + 7) / 8;
  return (size_t)(R / 16) * nch * 512;
}

hipError_t launch_pack_matrix(int R, int K, int n_mat, const uint8_t* q, const uint8_t* s,
                              uint8_t* pq, uint8_t* ps, hipStream_t st) {
  const long long nq = (long long)n_mat * R * K / 32;
  const long long ns = (long long)n_mat * (R / 16) * ((K / 128 + 7) / 8) * 64;
  if (nq > 0)
    pack_codes_kernel<<<(unsigned)((nq + 255) / 256), 256, 0, st>>>(R, K, nq, q, pq);
  if (ns > 0)
    pack_scales_kernel<<<(unsigned)((ns + 255) / 256), 256, 0, st>>>(R, K, ns, s, ps);
  return hipGetLastError();
}

}  // namespace k3moe
