// router.hip — router logits (fp64 accumulation), softmax and top-k on gfx950.
//
// Follows "Kimi K3 纯 C 语言 CPU 推理实战" (chenxutan.com/d/5901.html) §2.4: logits are
// the GEMV of the token against the [hidden][experts] gate matrix, the softmax is
// max-subtracted over all experts, and top-k picks the largest logits with the lower
// index winning a tie; the gate of a chosen expert is its full-softmax probability.
// Every product bf16*bf16 or bf16*fp32 is exact in fp64, and the sums are carried in
// fp64, so the ranking is that of the exact logits barring ties closer than fp64
// rounding.
#include "block_dev.h"
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

constexpr int kRouterRows = 512;  // W rows per partial chunk (4 waves x 128)
constexpr int kRouterCols = 64;   // W columns per block (one lane each)
constexpr int kTokGroup = 4;      // tokens per pass over a chunk
constexpr int kRouterTokMinT = 10;  // from here on the in-lane-reduction kernel
constexpr int kRouterTokWaves = 4;  // its waves per block

template <bool XF32>
__device__ __forceinline__ double load_x(const void* x, size_t i) {
  if (XF32) return (double)static_cast<const float*>(x)[i];
  return (double)bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
}

// part[chunk][t][e] = sum over rows k of this chunk of x[t][k] * W[k][e].
// Block: 4 waves; lane = column; wave w sums rows [w*128, w*128+128) of the chunk; the
// four wave sums are added in wave order. Grid: (chunks, column blocks).
template <bool XF32, int NT>
__global__ __launch_bounds__(256) void router_gemv_kernel(int T, int d, int E,
                                                          const void* __restrict__ x,
                                                          const uint16_t* __restrict__ w,
                                                          double* __restrict__ part) {
  __shared__ double xs[kRouterRows][NT];
  __shared__ double ws[4][NT][kRouterCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  const int k0 = chunk * kRouterRows;
  const int nrows = min(kRouterRows, d - k0);
  const int col = blockIdx.y * kRouterCols + lane;
  const int r0 = wave * (kRouterRows / 4);
  const int r1 = min(r0 + kRouterRows / 4, nrows);
  for (int t0 = 0; t0 < T; t0 += NT) {
    const int nt = min(NT, T - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < nrows * NT; i += 256) {
      const int r = i / NT, tt = i % NT;
      xs[r][tt] = (tt < nt) ? load_x<XF32>(x, (size_t)(t0 + tt) * d + k0 + r) : 0.0;
    }
    __syncthreads();
    double acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = 0.0;
    if (col < E) {
      const uint16_t* wp = w + (size_t)k0 * E + col;
      int r = r0;
      for (; r + 8 <= r1; r += 8) {
        uint16_t wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) wv[u] = wp[(size_t)(r + u) * E];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double wd = (double)bf16_bits_to_f32(wv[u]);
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[tt] = fma(xs[r + u][tt], wd, acc[tt]);
        }
      }
      for (; r < r1; ++r) {
        const double wd = (double)bf16_bits_to_f32(wp[(size_t)r * E]);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) acc[tt] = fma(xs[r][tt], wd, acc[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) ws[wave][tt][lane] = acc[tt];
    __syncthreads();
    if (wave == 0 && col < E) {
      for (int tt = 0; tt < nt; ++tt) {
        const double s = ((ws[0][tt][lane] + ws[1][tt][lane]) + ws[2][tt][lane]) + ws[3][tt][lane];
        part[((size_t)chunk * T + t0 + tt) * E + col] = s;
      }
    }
  }
}

// Same partials with 16-byte loads: a block covers 512 rows x 64 columns; lane l reads
// columns 8*(l%8) .. +7 of rows l/8, l/8 + 8, ... (16 rows per lane, all loads issued
// before the first FMA). Row sums: per lane in row order, then a fixed xor tree over
// the 8 lanes sharing a column group, then the four waves in order. Needs E % 8 == 0.
// (chunk, cblk): the block's row chunk and column block (the grid's x and y). Needs 256
// threads. One token: xl supplies the chunk's activations: issue(t, ra, rb) before the
// weight loads (rows ra, rb of the chunk, in range), get(xa, xb) after them (XRow reads
// x; the block-mode launch's form normalises the residual there).
template <bool XF32>
struct XRow {
  const void* x;
  int d, k0;
  double xa, xb;
  __device__ __forceinline__ void issue(int t, int ra, int rb) {
    xa = load_x<XF32>(x, (size_t)t * d + k0 + ra);
    xb = load_x<XF32>(x, (size_t)t * d + k0 + rb);
  }
  __device__ __forceinline__ void get(double& a, double& b) {
    a = xa;
    b = xb;
  }
};

template <bool XF32, int NT, class XL>
__device__ __forceinline__ void router_gemv_vec_block(int chunk, int cblk, int T, int d, int E,
                                                      XL& xl, const uint16_t* __restrict__ w,
                                                      double* __restrict__ part) {
  constexpr int RPL = kRouterRows / 4 / 8;  // rows per lane (16)
  __shared__ double xs[kRouterRows][NT];
  __shared__ double wsum[4][NT][kRouterCols];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = chunk * kRouterRows;
  const int nrows = min(kRouterRows, d - k0);
  const int cg = lane & 7, rl = lane >> 3;
  const int col0 = cblk * kRouterCols + cg * 8;
  const bool cv = col0 < E;
  u32x4 wv[RPL];
  if constexpr (NT > 1) {
    // several tokens: the block's weights are loaded once (clamped to valid rows/columns,
    // masked below) and stay in registers for every token group
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int r = min(wave * (kRouterRows / 4) + rl + 8 * u, nrows - 1);
      wv[u] = *reinterpret_cast<const u32x4*>(w + (size_t)(k0 + r) * E + (cv ? col0 : 0));
    }
  }
  for (int t0 = 0; t0 < T; t0 += NT) {
    const int nt = min(NT, T - t0);
    if constexpr (NT == 1) {
      // one token: the chunk's activations first (rows tid and tid + 256, loads clamped and
      // masked), then every weight load; the activations go to LDS as soon as their own
      // loads land and the barrier waits only for LDS, so all weight loads stay in flight
      if (t0 > 0) __syncthreads();
      const int ra = threadIdx.x, rb = threadIdx.x + 256;
      xl.issue(t0, min(ra, nrows - 1), min(rb, nrows - 1));
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < RPL; ++u) {
        const int r = min(wave * (kRouterRows / 4) + rl + 8 * u, nrows - 1);
        wv[u] = *reinterpret_cast<const u32x4*>(w + (size_t)(k0 + r) * E + (cv ? col0 : 0));
      }
      double xa, xb;
      xl.get(xa, xb);
      xs[ra][0] = ra < nrows ? xa : 0.0;
      xs[rb][0] = rb < nrows ? xb : 0.0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      // no barrier before refilling xs: every wave finished reading it before the barrier
      // that publishes the previous group's wave sums.
      // Activations of the group: one 16-byte load (8 bf16 or 4 fp32 values) per thread and
      // step, all issued before any is used (one element per load made every element its
      // own round trip to L2); x rows and the chunk start are 16-byte aligned and nrows is
      // a multiple of 32
      const void* x = xl.x;
      constexpr int VPL = XF32 ? 4 : 8;
      constexpr int LPT = kRouterRows / VPL;              // loads per token
      constexpr int ITER = (NT * LPT + 255) / 256;        // loads per thread
      u32x4 xq[ITER];
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int i = threadIdx.x + 256 * it;
        const int tt = i / LPT, r0 = (i - tt * LPT) * VPL;
        const bool ok = i < NT * LPT && tt < nt && r0 < nrows;
        const size_t el = (size_t)(t0 + (ok ? tt : 0)) * d + k0 + (ok ? r0 : 0);
        xq[it] = XF32 ? *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + el)
                      : *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + el);
      }
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int i = threadIdx.x + 256 * it;
        if (i >= NT * LPT) continue;
        const int tt = i / LPT, r0 = (i - tt * LPT) * VPL;
        const bool ok = tt < nt && r0 < nrows;
        double v[VPL];
        if (XF32) {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = (double)__uint_as_float(xq[it][u]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[2 * u] = (double)__uint_as_float(xq[it][u] << 16);
            v[2 * u + 1] = (double)__uint_as_float(xq[it][u] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int u = 0; u < VPL; ++u) xs[r0 + u][tt] = ok ? v[u] : 0.0;
      }
      __syncthreads();
    }
    double acc[NT][8];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[tt][c] = 0.0;
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
      const int r = wave * (kRouterRows / 4) + rl + 8 * u;
      if (r < nrows) {
        double wd[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          wd[2 * c] = (double)__uint_as_float(wv[u][c] << 16);
          wd[2 * c + 1] = (double)__uint_as_float(wv[u][c] & 0xFFFF0000u);
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const double xv = xs[r][tt];
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[tt][c] = fma(xv, wd[c], acc[tt][c]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        double v = acc[tt][c];
        v += lane_xor_d<8>(v, lane);
        v += lane_xor_d<16>(v, lane);
        v += lane_xor_d<32>(v, lane);
        acc[tt][c] = v;
      }
    if (rl == 0) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int c = 0; c < 8; ++c) wsum[wave][tt][cg * 8 + c] = acc[tt][c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt * kRouterCols; i += 256) {
      const int tt = i / kRouterCols, c = i % kRouterCols;
      const int col = cblk * kRouterCols + c;
      if (col < E) {
        const double s = ((wsum[0][tt][c] + wsum[1][tt][c]) + wsum[2][tt][c]) + wsum[3][tt][c];
        part[((size_t)chunk * T + t0 + tt) * E + col] = s;
      }
    }
  }
}

template <bool XF32, int NT>
__global__ __launch_bounds__(256) void router_gemv_vec_kernel(int T, int d, int E,
                                                              const void* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              double* __restrict__ part) {
  XRow<XF32> xl{x, d, (int)blockIdx.x * kRouterRows, 0.0, 0.0};
  router_gemv_vec_block<XF32, NT>(blockIdx.x, blockIdx.y, T, d, E, xl, w, part);
}

// Several tokens: the K reduction stays inside each lane (no cross-lane sums). A work item
// is (512-row chunk, 512-column slab, group of 4 tokens); its block of NW waves gives wave w
// the chunk's rows [w R, w R + R), R = 512 / NW, and lane l the columns slab * 512 + 8 l .. + 7.
// A lane accumulates its 4 x 8 outputs over its rows in row order, reading rows in batches
// of 8 with the next batch in flight; the wave sums are then added by a fixed pairwise tree
// (wave w + wave w + NW/2, then halves again). Consecutive work items (the token groups of
// one weight tile first) are given to blocks on the same XCD (blocks are dealt to the 8
// XCDs round robin), so a weight tile is read from HBM once and then from that XCD's L2.
// Needs E % 8 == 0, 16-byte aligned W and x.
typedef double f64x2 __attribute__((ext_vector_type(2)));
constexpr int kRtSlab = 512;   // columns per work item (64 lanes x 8)
constexpr int kRtTok = 4;      // tokens per work item
constexpr int kRtBatch = 8;    // W rows per load batch
// x of a work item in LDS: row r, token t at r * 4 + t + 2 * (r / 8) doubles (the pad keeps
// the staging writes of neighbouring lanes on different banks, and rows 16-byte aligned)
__device__ __forceinline__ int rt_xs_at(int r) { return r * kRtTok + 2 * (r >> 3); }
constexpr int kRtXsLen = kRouterRows * kRtTok + 2 * (kRouterRows / 8);
constexpr int kRtAcc = kRtTok * 8;  // outputs per lane

__host__ __device__ inline int rt_slabs(int E) { return (E + kRtSlab - 1) / kRtSlab; }

template <bool XF32, int NW>
__global__ __launch_bounds__(64 * NW) void router_tok_kernel(int T, int d, int E, int n_tg,
                                                             int n_items,
                                                             const void* __restrict__ x,
                                                             const uint16_t* __restrict__ w,
                                                             double* __restrict__ part) {
  constexpr int NTH = 64 * NW, WROWS = kRouterRows / NW;
  constexpr int RED = (NW / 2) * kRtAcc * 64;  // first reduction stage
  // the activations while the waves accumulate, then the reduction stages (after a barrier
  // that every read of the activations precedes)
  __shared__ __align__(16) double lds[RED > kRtXsLen ? RED : kRtXsLen];
  double* xs = lds;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x, n8 = n_items / 8, rem = n_items % 8, xcd = b % 8;
  const int item = xcd * n8 + min(xcd, rem) + b / 8;
  const int n_slab = rt_slabs(E);
  const int tg = item % n_tg, slab = (item / n_tg) % n_slab, chunk = item / (n_tg * n_slab);
  const int t0 = tg * kRtTok, nt = min(kRtTok, T - t0);
  const int k0 = chunk * kRouterRows, nrows = min(kRouterRows, d - k0);
  const int col0 = slab * kRtSlab + lane * 8;
  const bool cv = col0 < E;  // E % 8 == 0: a lane's 8 columns are all valid or none
  const int rw0 = wave * WROWS;
  const uint16_t* wcol = w + (cv ? col0 : 0);

  u32x4 wa[kRtBatch], wb[kRtBatch];
  // rows clamped to the chunk's last valid row; batches past it are skipped below
  auto load = [&](u32x4 (&dst)[kRtBatch], int bi) {
#pragma unroll
    for (int i = 0; i < kRtBatch; ++i) {
      const int r = min(rw0 + kRtBatch * bi + i, nrows - 1);
      dst[i] = *reinterpret_cast<const u32x4*>(wcol + (size_t)(k0 + r) * E);
    }
  };
  load(wa, 0);

  // the work item's activations: one 16-byte load (8 bf16 or 4 fp32 values) per thread
  {
    constexpr int VPL = XF32 ? 4 : 8;
    constexpr int LPT = kRouterRows / VPL;  // loads per token
    constexpr int NLD = kRtTok * LPT;
    constexpr int ITER = (NLD + NTH - 1) / NTH;
    u32x4 xq[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int i = min((int)threadIdx.x + NTH * it, NLD - 1);
      const int tt = i / LPT, r0 = (i - tt * LPT) * VPL;
      const bool ok = tt < nt && r0 < nrows;
      const size_t el = (size_t)(t0 + (ok ? tt : 0)) * d + k0 + (ok ? r0 : 0);
      xq[it] = XF32 ? *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + el)
                    : *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + el);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int i = threadIdx.x + NTH * it;
      if (i >= NLD) break;
      const int tt = i / LPT, r0 = (i - tt * LPT) * VPL;
      const bool ok = tt < nt && r0 < nrows;
      double v[VPL];
      if (XF32) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (double)__uint_as_float(xq[it][u]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[2 * u] = (double)__uint_as_float(xq[it][u] << 16);
          v[2 * u + 1] = (double)__uint_as_float(xq[it][u] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int u = 0; u < VPL; ++u) xs[rt_xs_at(r0 + u) + tt] = ok ? v[u] : 0.0;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  double acc[kRtAcc];
#pragma unroll
  for (int i = 0; i < kRtAcc; ++i) acc[i] = 0.0;
  auto fma_batch = [&](const u32x4 (&src)[kRtBatch], int bi) {
    const int rb = rw0 + kRtBatch * bi;
    if (rb >= nrows) return;  // wave-uniform: nrows is a multiple of 32
#pragma unroll
    for (int i = 0; i < kRtBatch; ++i) {
      const f64x2* xr = reinterpret_cast<const f64x2*>(&xs[rt_xs_at(rb + i)]);
      const f64x2 x01 = xr[0], x23 = xr[1];
      const double xv[kRtTok] = {x01[0], x01[1], x23[0], x23[1]};
      double wd[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        wd[2 * c] = (double)__uint_as_float(src[i][c] << 16);
        wd[2 * c + 1] = (double)__uint_as_float(src[i][c] & 0xFFFF0000u);
      }
#pragma unroll
      for (int tt = 0; tt < kRtTok; ++tt)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[tt * 8 + c] = fma(xv[tt], wd[c], acc[tt * 8 + c]);
    }
  };
  constexpr int NB = WROWS / kRtBatch;
  static_assert(NB % 2 == 0, "batches are taken in pairs");
  for (int bi = 0; bi < NB; bi += 2) {
    load(wb, bi + 1);
    fma_batch(wa, bi);
    load(wa, min(bi + 2, NB - 1));  // the last pair reloads a batch it does not use
    fma_batch(wb, bi + 1);
  }

  // wave sums: wave w takes wave w + half, for half = NW/2, NW/4, ..., 1
#pragma unroll
  for (int half = NW / 2; half >= 1; half /= 2) {
    __syncthreads();  // the previous stage's (or the activations') readers are done
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int i = 0; i < kRtAcc; ++i) lds[((wave - half) * kRtAcc + i) * 64 + lane] = acc[i];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int i = 0; i < kRtAcc; ++i) acc[i] += lds[(wave * kRtAcc + i) * 64 + lane];
    }
  }
  if (wave == 0 && cv) {
#pragma unroll
    for (int tt = 0; tt < kRtTok; ++tt) {
      if (tt < nt) {
        f64x2* dst = reinterpret_cast<f64x2*>(part + ((size_t)chunk * T + t0 + tt) * E + col0);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = f64x2{acc[tt * 8 + 2 * c], acc[tt * 8 + 2 * c + 1]};
      }
    }
  }
}

// Many-token router on fp64 MFMA: part[c][t][e] = sum over the c-th K chunk of
// x[t][k] * W[k][e], with v_mfma_f64_16x16x4_f64 (fp64 products and sums, like the
// scalar paths). Block: 64 tokens x 64 experts x one K chunk, 4 waves of 32 x 32
// (2 x 2 MFMA tiles). Both operands (bf16, or fp32 tokens) are exact in fp32, so LDS holds
// them as fp32 (four blocks fit on a CU) and each MFMA operand is widened to fp64 as it is
// read. K advances 32 per stage, double-buffered: the next stage's global loads go out as raw
// words before the current stage's MFMAs and are converted and stored after them, one block
// barrier per stage. Within a stage, lane group g = lane/16 feeds k = 4 j + g to the j-th
// MFMA of every tile (A and B alike).
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kRmBK = 32;        // K per stage
constexpr int kRmAP = kRmBK + 4; // A: token-major, pitch 36 floats (lane (ln, g) -> bank 4 ln + g)
constexpr int kRmBP = 64 + 16;   // B: k-major, pitch 80 floats (lane groups 16 banks apart)

template <bool XF32>
__global__ __launch_bounds__(256) void router_mfma_kernel(int T, int d, int E, int kc,
                                                          const void* __restrict__ x,
                                                          const uint16_t* __restrict__ w,
                                                          double* __restrict__ part) {
  __shared__ __align__(16) float As[2][64 * kRmAP];
  __shared__ __align__(16) float Bs[2][kRmBK * kRmBP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int c = blockIdx.z;
  const int kbeg = c * kc, kend = min(d, kbeg + kc);
  const int nst = (kend - kbeg + kRmBK - 1) / kRmBK;

  // staging: thread -> (A row ar, 8 k at ak) and (B k-row bk, 8 experts at be)
  const int ar = tid >> 2, ak = (tid & 3) * 8;
  const int bk = tid >> 3, be = (tid & 7) * 8;
  const int arow = min(t0 + ar, T - 1);  // rows past T load row T - 1 and store zeros
  const bool arow_ok = t0 + ar < T;
  // 16-byte loads where the 8 values are contiguous and aligned (k chunks are multiples
  // of 32 and x rows are 16-byte aligned; W rows need E % 8 == 0 and an aligned base)
  const bool wvec = (E % 8) == 0 && (reinterpret_cast<uintptr_t>(w) & 15u) == 0;
  // raw words of the next stage: A as 8 fp32 (qa0, qa1) or 8 bf16 (qa0); B as 8 bf16
  u32x4 qa0, qa1 = u32x4{0u, 0u, 0u, 0u}, qb;
  bool aok, bok;
  auto load = [&](int st) {
    const int k = kbeg + st * kRmBK;
    const int ka = k + ak, kb = k + bk;
    aok = arow_ok && ka < kend;
    // out-of-range pieces read an in-range address and are zeroed when stored, so no load
    // sits behind a branch that would make the compiler wait for it there
    const size_t aoff = (size_t)arow * d + (ka < kend ? ka : kbeg);
    if (XF32) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + aoff);
      qa0 = src[0];
      qa1 = src[1];
    } else {
      qa0 = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + aoff);
    }
    const int eb = e0 + be;
    if (wvec) {
      bok = kb < kend && eb + 8 <= E;
      qb = *reinterpret_cast<const u32x4*>(w + (size_t)(kb < kend ? kb : kbeg) * E +
                                           (eb + 8 <= E ? eb : 0));
    } else {
      bok = true;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t lo = (kb < kend && eb + 2 * u < E) ? w[(size_t)kb * E + eb + 2 * u] : 0u;
        const uint32_t hi =
            (kb < kend && eb + 2 * u + 1 < E) ? w[(size_t)kb * E + eb + 2 * u + 1] : 0u;
        qb[u] = lo | (hi << 16);
      }
    }
  };
  auto store = [&](int buf) {
    f32x4 a0, a1, b0, b1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (XF32) {
        a0[u] = __uint_as_float(qa0[u]);
        a1[u] = __uint_as_float(qa1[u]);
      } else {
        const uint32_t q = qa0[u >> 1] >> (16 * (u & 1)), r = qa0[2 + (u >> 1)] >> (16 * (u & 1));
        a0[u] = __uint_as_float(q << 16);
        a1[u] = __uint_as_float(r << 16);
      }
      b0[u] = __uint_as_float((qb[u >> 1] >> (16 * (u & 1))) << 16);
      b1[u] = __uint_as_float((qb[2 + (u >> 1)] >> (16 * (u & 1))) << 16);
    }
    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4* ad = reinterpret_cast<f32x4*>(&As[buf][ar * kRmAP + ak]);
    f32x4* bd = reinterpret_cast<f32x4*>(&Bs[buf][bk * kRmBP + be]);
    ad[0] = aok ? a0 : z;
    ad[1] = aok ? a1 : z;
    bd[0] = bok ? b0 : z;
    bd[1] = bok ? b1 : z;
  };

  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load(st + 1);
#pragma unroll
    for (int j = 0; j < kRmBK / 4; ++j) {
      const int kk = 4 * j + g;
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = (double)As[buf][(wm * 32 + i * 16 + ln) * kRmAP + kk];
#pragma unroll
      for (int i = 0; i < 2; ++i) b[i] = (double)Bs[buf][kk * kRmBP + wn * 32 + i * 16 + ln];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    // buffer buf ^ 1 was last read in stage st - 1, before every wave passed the previous
    // barrier, so it can be refilled without another one
    if (st + 1 < nst) {
      store(buf ^ 1);
      __syncthreads();
    }
  }
  // fp64 16 x 16 result: value r of lane (ln, g) is row g + 4 r, column ln
  double* out = part + (size_t)c * T * E;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + wm * 32 + mi * 16 + g + 4 * r;
        const int e = e0 + wn * 32 + ni * 16 + ln;
        if (t < T && e < E) out[(size_t)t * E + e] = acc[mi][ni][r];
      }
}

// Total-order key of an fp64 logit: larger logit -> larger key; +0 and -0 share a
// key; NaN gets key 0, below every number.
__device__ __forceinline__ uint64_t order_key(double v) {
  if (v != v) return 0ull;
  v = v + 0.0;  // -0 -> +0
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ bool better(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

constexpr int kMaxE = 4096;
constexpr int kMaxSlots = 32;

// One block per token of NT = blockDim.x threads (a multiple of 64, at most 256): thread t
// holds the logits of experts t + NT*j (j < KPT) in registers. WIDE: the block has 1024
// threads, which form the logits one expert per thread into LDS (every partial in flight
// at once); the first 256 threads then read their keys back and the rest only keep the
// block's barrier count.
//  1. logits = sum of the fp64 partials in chunk order (+ bias), as order keys;
//  2. each wave sorts the upper 32 bits of its 64 lane maxima (bitonic network over
//     lanes): the k-th best of them is at most the upper bits of the k-th best of all E,
//     so the best such bound over the waves is a valid threshold, and every top-k element
//     has its upper bits at or above it;
//  3. candidates at or above the threshold are compacted into LDS (ballot counts) and ranked
//     exactly against each other; the softmax denominator is a per-thread ordered sum and
//     a fixed reduction tree.
// With `bk` (T == 1) the same block also writes the expert bucket of the single token.
constexpr int kTopkMaxWaves = 4;
struct Bucket1 {
  int32_t *offsets, *rows, *act, *n_act, *pair_pos, *pair_exp, *mtile_off;
};

__device__ __forceinline__ double key_to_double(uint64_t kv) {
  const uint64_t b = (kv >> 63) ? (kv & 0x7FFFFFFFFFFFFFFFull) : ~kv;
  return __longlong_as_double((long long)b);
}

// Token t of the block; WIDE needs 1024 threads, the other form at most 256.
template <int KPT, bool WIDE>
__device__ __forceinline__ void route_topk_block(int t, int T, int E, int k,
                                                 const double* __restrict__ part, int nsum,
                                                 const float* __restrict__ bias,
                                                 int32_t* __restrict__ ids,
                                                 float* __restrict__ gates, Bucket1 bk) {
  // every expert's key, and room for every candidate (E <= 256 KPT)
  constexpr int NKEY = 256 * KPT;
  __shared__ uint64_t keys[NKEY];
  __shared__ uint64_t ckey[NKEY];
  __shared__ int cid[NKEY];
  __shared__ uint32_t w_tk[kTopkMaxWaves], w_mk[kTopkMaxWaves];
  __shared__ int w_ok[kTopkMaxWaves], w_cnt[kTopkMaxWaves], w_nan[kTopkMaxWaves];
  __shared__ double w_sum[kTopkMaxWaves];
  __shared__ int s_ids[kMaxSlots];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NT = WIDE ? 256 : blockDim.x, nw = NT >> 6;

  uint64_t key[KPT];
  int nan_here = 0;
  uint64_t bkey = 0;
  int bi = -1;
  if (WIDE) {
    // 1. logits, one expert per thread of the whole block (every chunk's load in flight at
    //    once), chunks summed in order; the first NT threads carry on from the LDS keys
    for (int e = tid; e < E; e += blockDim.x) {
      const float b = bias ? bias[e] : 0.0f;
      double l = 0.0;
      for (int c0 = 0; c0 < nsum; c0 += 16) {
        double v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = part[((size_t)min(c0 + u, nsum - 1) * T + t) * E + e];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (c0 + u < nsum) l = (c0 + u == 0) ? v[u] : l + v[u];
      }
      if (bias) l += (double)b;
      keys[e] = order_key(l);  // NaN -> key 0, which no number maps to
    }
    __syncthreads();
    if (tid >= NT) {
      // loader-only waves: match the three block barriers below (four with a bucket)
      __syncthreads();
      __syncthreads();
      __syncthreads();
      if (bk.offsets) __syncthreads();
      return;
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int e = tid + NT * j;
      if (e < E) {
        key[j] = keys[e];
        nan_here |= (key[j] == 0ull);
        if (bi < 0 || better(key[j], e, bkey, bi)) { bkey = key[j]; bi = e; }
      } else {
        key[j] = 0;
      }
    }
  } else {
    // 1. logits: all loads of a chunk issued before any add; chunks summed in order
    constexpr int CB = (64 / KPT) > 1 ? (64 / KPT) : 1;  // chunks whose loads go out together
    float bv[KPT];  // bias requested together with the first partials
#pragma unroll
    for (int j = 0; j < KPT; ++j) bv[j] = bias ? bias[min(tid + NT * j, E - 1)] : 0.0f;
    double acc[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) acc[j] = 0.0;
    for (int c0 = 0; c0 < nsum; c0 += CB) {
      double v[CB][KPT];
#pragma unroll
      for (int u = 0; u < CB; ++u)
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const int e = min(tid + NT * j, E - 1);
          const int c = min(c0 + u, nsum - 1);
          v[u][j] = part[((size_t)c * T + t) * E + e];  // clamped: always a valid address
        }
#pragma unroll
      for (int u = 0; u < CB; ++u)
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (c0 + u < nsum) acc[j] = (c0 + u == 0) ? v[u][j] : acc[j] + v[u][j];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int e = tid + NT * j;
      if (e < E) {
        const double l = bias ? acc[j] + (double)bv[j] : acc[j];
        nan_here |= (l != l);
        key[j] = order_key(l);
        keys[e] = key[j];
        if (bi < 0 || better(key[j], e, bkey, bi)) { bkey = key[j]; bi = e; }
      } else {
        key[j] = 0;
      }
    }
  }

  // 2. per-wave threshold on the upper 32 bits of the keys (a monotone map, so the bound
  //    below stays valid and candidates are ranked on the full keys): the 64 lane maxima
  //    sorted best-first by a bitonic network over the lanes; lane 0 then holds the wave's
  //    best and lane k-1 its k-th best
  {
    uint32_t sk = (bi >= 0) ? (uint32_t)(bkey >> 32) : 0u;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const uint32_t pk = lane_xor_rt(sk, stride, lane);  // a constant stride once unrolled
        const bool desc = (lane & size) == 0;  // this run of `size` lanes sorts best-first
        const bool low = (lane & stride) == 0;
        sk = (low == desc) ? (pk > sk ? pk : sk) : (pk < sk ? pk : sk);
      }
    }
    const int nvalid = __popcll(__ballot(bi >= 0));
    const bool anyn = __any(nan_here);
    if (lane == 0) {
      w_ok[wave] = nvalid >= k;
      w_nan[wave] = anyn ? 1 : 0;
      w_mk[wave] = nvalid > 0 ? sk : 0u;
    }
    if (lane == k - 1) w_tk[wave] = sk;
  }
  __syncthreads();
  // threshold: the best wave bound (0 admits every expert when no wave has k valid lanes)
  uint32_t tk = 0, mk = 0;
  int anynan = 0;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    if (w_ok[w] && w_tk[w] > tk) tk = w_tk[w];
    mk = (w_mk[w] > mk) ? w_mk[w] : mk;
    anynan |= w_nan[w];
  }
  // softmax shift: the largest logit with the low 32 key bits cleared, at most 2^-20 of its
  // magnitude below it (any shift near the maximum gives the same quotients)
  const double m = key_to_double((uint64_t)mk << 32);

  // 3. candidates (wave scan) and softmax denominator
  int mine = 0;
  double se = 0.0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int e = tid + NT * j;
    if (e < E) {
      mine += ((uint32_t)(key[j] >> 32) >= tk) ? 1 : 0;
      se += exp(key_to_double(key[j]) - m);
    }
  }
  // exclusive prefix of `mine` (at most KPT) over the wave's lanes and the wave's total, from
  // the ballots of its bits
  int pre = 0, wtot = 0;
#pragma unroll
  for (int bit = 0; (1 << bit) <= KPT; ++bit) {
    const uint64_t bm = __ballot((mine >> bit) & 1);
    pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u)) << bit;
    wtot += __popcll(bm) << bit;
  }
  se += lane_xor_d<32>(se, lane);
  se += lane_xor_d<16>(se, lane);
  se += lane_xor_d<8>(se, lane);
  se += lane_xor_d<4>(se, lane);
  se += lane_xor_d<2>(se, lane);
  se += lane_xor_d<1>(se, lane);
  if (lane == 0) {
    w_cnt[wave] = wtot;
    w_sum[wave] = se;
  }
  __syncthreads();
  int base = 0, total = 0;
  double wsum = 0.0;
  for (int w = 0; w < nw; ++w) {
    base += (w < wave) ? w_cnt[w] : 0;
    total += w_cnt[w];
    wsum += w_sum[w];
  }
  const double sum = anynan ? __builtin_nan("") : wsum;
  pre += base;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int e = tid + NT * j;
    if (e < E && (uint32_t)(key[j] >> 32) >= tk) {
      cid[pre] = e;
      ckey[pre] = key[j];
      ++pre;
    }
  }
  __syncthreads();

  // 4. exact ranks of the candidates: with at most NT/4 of them, four threads share a
  //    candidate, each comparing it with every fourth other one, and add their counts
  if (4 * total <= NT) {
    const int c = tid >> 2, part = tid & 3;
    const bool has = c < total;
    const uint64_t kv = has ? ckey[c] : 0ull;
    const int id = has ? cid[c] : 0;
    int r = 0;
    if (has) {
#pragma unroll 4
      for (int j = part; j < total; j += 4) r += better(ckey[j], cid[j], kv, id) ? 1 : 0;
    }
    r += (int)lane_xor<1>((uint32_t)r, lane);
    r += (int)lane_xor<2>((uint32_t)r, lane);
    if (has && part == 0 && r < k) {
      ids[(size_t)t * k + r] = id;
      gates[(size_t)t * k + r] = (float)(exp(key_to_double(kv) - m) / sum);
      if (bk.offsets) s_ids[r] = id;
    }
  } else {
    for (int c = tid; c < total; c += NT) {
      const int id = cid[c];
      const uint64_t kv = ckey[c];
      int r = 0;
#pragma unroll 8
      for (int j = 0; j < total; ++j) r += better(ckey[j], cid[j], kv, id) ? 1 : 0;
      if (r < k) {
        ids[(size_t)t * k + r] = id;
        gates[(size_t)t * k + r] = (float)(exp(key_to_double(kv) - m) / sum);
        if (bk.offsets) s_ids[r] = id;
      }
    }
  }
  if (!bk.offsets) return;
  // 5. T == 1: bucket of the single token (ranks of the k ids in ascending id order)
  __syncthreads();
  if (tid < k) {
    const int id = s_ids[tid];
    int pos = 0;
    for (int j = 0; j < k; ++j) pos += (s_ids[j] < id) ? 1 : 0;
    bk.rows[pos] = tid;
    bk.act[pos] = id;
    bk.pair_pos[tid] = pos;
    bk.pair_exp[tid] = id;
    bk.mtile_off[pos] = pos;
  }
  if (tid == 0) {
    *bk.n_act = k;
    bk.mtile_off[k] = k;
  }
  // only the selected experts' offsets are read on the single-token path
  if (tid < k) {
    const int id = s_ids[tid];
    int pos = 0;
    for (int j = 0; j < k; ++j) pos += (s_ids[j] < id) ? 1 : 0;
    bk.offsets[id] = pos;
    bk.offsets[id + 1] = pos + 1;
  }
}

template <int KPT, bool WIDE>
__global__ __launch_bounds__(WIDE ? 1024 : 256) void route_topk_kernel(int T, int E, int k,
                                                          const double* __restrict__ part,
                                                          int nsum, const float* __restrict__ bias,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ gates, Bucket1 bk) {
  route_topk_block<KPT, WIDE>(blockIdx.x, T, E, k, part, nsum, bias, ids, gates, bk);
}

// One token of block mode: the router's chunk rows are the RMSNorm of the residual h, formed
// in every router block (the sum of squares over the whole row as in the standalone RMSNorm,
// so every block gets the same values); the blocks of column block 0 also store their chunk
// of xhat for the expert kernels.
struct XNormRow {
  const float* h;
  const uint16_t* gamma;
  float* xhat;  // nullable: where to store the chunk's rows
  int d, k0;
  float eps;
  double* red;  // 4 doubles of LDS
  f32x4 v[kNormPieces];  // this thread's pieces of h, for the sum of squares
  float ha, hb;
  uint32_t ga, gb;
  int rowa, rowb;
  __device__ __forceinline__ void issue(int, int ra, int rb) {
    norm_load_h(h, d, v);
    rowa = k0 + ra;
    rowb = k0 + rb;
    ha = h[rowa];
    hb = h[rowb];
    ga = gamma[rowa];
    gb = gamma[rowb];
  }
  __device__ __forceinline__ void get(double& a, double& b) {
    const double inv = norm_inv(v, d, eps, red);
    const float xa = norm_value(ha, ga, inv), xb = norm_value(hb, gb, inv);
    if (xhat) {  // rows past the chunk's end are clamped to its last row: same value
      xhat[rowa] = xa;
      xhat[rowb] = xb;
    }
    a = (double)xa;
    b = (double)xb;
  }
};

// ---- block mode, one token: the routing launches carry the shared expert ------------------
// The shared expert's two bf16 GEMVs need only the normalised token. Rather than running on
// a second stream (whose fork and join cost more than the GEMVs themselves at this size),
// they ride in the two routing launches, which are latency-bound and leave most of the HBM
// bandwidth idle, and the RMSNorm rides in the first: blocks [0, nrb) of the first launch
// are the router GEMV's (chunk, column block), in the standalone grid's order, each forming
// its chunk of xhat itself (XNormRow; column block 0 also stores it for the expert kernels);
// the others walk the shared gate/up row groups (silu(G xhat) * (U xhat) into hsh) on a
// token they normalise themselves (StageNormRow). Block 0 of the second launch is the
// top-k's (with the token's bucket), the others walk the shared down row groups (D hsh into
// ssh). Each part runs the code of its standalone kernel, so every value is the same bit for
// bit as with the separate launches.
struct RouteSharedArgs {
  int d, f, E, k;
  const float* h;            // residual [d] (block input)
  const uint16_t* gamma;     // RMSNorm weight [d]
  float eps;
  float* xhat;               // normalised token [d] (written)
  const uint16_t* w_router;  // [d][E]
  double* part;              // router partial sums [nchunk][E]
  int nchunk, nrb;           // router chunks; router blocks (chunks x column blocks)
  const uint16_t *sh_gate, *sh_up, *sh_down;
  float *hsh, *ssh;          // shared expert's h [f] and output [d]
  const float* bias;
  int32_t* ids;
  float* gates;
  Bucket1 bk;
};

// Three waves per SIMD (168 registers, two of them spilled): the 196 router and 384 shared
// blocks of the K3 layer are then all resident at once (two waves per SIMD left 68 blocks for
// a second round; 0.649-0.654 against 0.657-0.660 ms per token on the 8-block stack).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void
router_shared_gateup_kernel(RouteSharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) f32x4 xs[];
  __shared__ double red[4];
  const int b = blockIdx.x;
  if (b < a.nrb) {  // block-uniform
    const int chunk = b % a.nchunk, cblk = b / a.nchunk;
    XNormRow xl{a.h, a.gamma, cblk == 0 ? a.xhat : nullptr, a.d, chunk * kRouterRows, a.eps, red};
    router_gemv_vec_block<true, 1>(chunk, cblk, 1, a.d, a.E, xl, a.w_router, a.part);
    return;
  }
  StageNormRow stg{a.h, a.gamma, a.d, a.eps, red};
  bf16_gemv_rows<true>(b - a.nrb, (int)gridDim.x - a.nrb, 1, a.f, a.d, stg, a.sh_gate, a.sh_up,
                       a.hsh, xs);
}

template <int KPT>
__global__ __launch_bounds__(1024) void topk_shared_down_kernel(RouteSharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) f32x4 xs[];
  if (blockIdx.x == 0) {
    route_topk_block<KPT, true>(0, 1, a.E, a.k, a.part, a.nchunk, a.bias, a.ids, a.gates, a.bk);
    return;
  }
  StageRow stg{a.hsh, a.f};
  bf16_gemv_rows<false>((int)blockIdx.x - 1, (int)gridDim.x - 1, 1, a.d, a.f, stg, a.sh_down,
                        nullptr, a.ssh, xs);
}

// Packed experts at one token: the router launch carries only the RMSNorm (router_norm_kernel),
// the top-k launch the shared gate/up (topk_shared_gateup_kernel: block 0 the top-k of 256
// threads, the others the shared gate/up row groups on the xhat the router blocks stored), and
// the shared down rides in the expert gate/up launch (ffn_mfma.hip): the top-k leaves a whole
// launch of HBM bandwidth idle that the 44 MB of shared gate/up weights fill, and the router
// launch, the critical one, no longer waits for them.
__global__ __launch_bounds__(256) void router_norm_kernel(RouteSharedArgs a) {
  __shared__ double red[4];
  const int b = blockIdx.x;
  const int chunk = b % a.nchunk, cblk = b / a.nchunk;
  XNormRow xl{a.h, a.gamma, cblk == 0 ? a.xhat : nullptr, a.d, chunk * kRouterRows, a.eps, red};
  router_gemv_vec_block<true, 1>(chunk, cblk, 1, a.d, a.E, xl, a.w_router, a.part);
}

template <int KPT>
__global__ __launch_bounds__(256) void topk_shared_gateup_kernel(RouteSharedArgs a) {
  extern __shared__ __attribute__((aligned(16))) f32x4 xs[];
  if (blockIdx.x == 0) {
    route_topk_block<KPT, false>(0, 1, a.E, a.k, a.part, a.nchunk, a.bias, a.ids, a.gates, a.bk);
    return;
  }
  StageRow stg{a.xhat, a.d};
  bf16_gemv_rows<true>((int)blockIdx.x - 1, (int)gridDim.x - 1, 1, a.f, a.d, stg, a.sh_gate,
                       a.sh_up, a.hsh, xs);
}

}  // namespace

int router_chunk_rows(int) { return kRouterRows; }
int router_num_chunks(int d) { return (d + kRouterRows - 1) / kRouterRows; }

hipError_t launch_router_gemv(int T, int d, int E, const void* x, int xf32, const uint16_t* w,
                              double* part, hipStream_t s) {
  dim3 grid(router_num_chunks(d), (E + kRouterCols - 1) / kRouterCols);
  // 16-byte loads: W rows (and, for several tokens, x rows) must start on 16 bytes
  const bool a16w = (reinterpret_cast<uintptr_t>(w) & 15u) == 0;
  const bool a16x = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  if (E % 8 == 0 && a16w && T >= kRouterTokMinT && a16x) {
    const int n_tg = (T + kRtTok - 1) / kRtTok;
    const int n_items = router_num_chunks(d) * rt_slabs(E) * n_tg;
    constexpr int NW = kRouterTokWaves;
    if (xf32)
      router_tok_kernel<true, NW><<<n_items, 64 * NW, 0, s>>>(T, d, E, n_tg, n_items, x, w, part);
    else
      router_tok_kernel<false, NW><<<n_items, 64 * NW, 0, s>>>(T, d, E, n_tg, n_items, x, w, part);
    return hipGetLastError();
  }
  if (E % 8 == 0 && a16w && (T == 1 || a16x)) {
    if (T == 1) {
      if (xf32) router_gemv_vec_kernel<true, 1><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
      else router_gemv_vec_kernel<false, 1><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
    } else {
      if (xf32) router_gemv_vec_kernel<true, kTokGroup><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
      else router_gemv_vec_kernel<false, kTokGroup><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
    }
    return hipGetLastError();
  }
  if (T == 1) {
    if (xf32) router_gemv_kernel<true, 1><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
    else router_gemv_kernel<false, 1><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
  } else {
    if (xf32) router_gemv_kernel<true, kTokGroup><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
    else router_gemv_kernel<false, kTokGroup><<<grid, 256, 0, s>>>(T, d, E, x, w, part);
  }
  return hipGetLastError();
}

// K chunks: about 2048 blocks of 64 x 64 over the chunks (a few waves of work on 256
// CUs), at most 8, each chunk at least 512 deep. T * splits never exceeds
// max(T, min(8 T, router_split_budget(E))), which sizes the partial-sum workspace.
int router_split_budget(int E) { return 131072 / ((E + 63) / 64); }

int router_mfma_splits(int T, int d, int E) {
  long ks = (long)router_split_budget(E) / (T > 0 ? T : 1);
  const long kmax = (d + 511) / 512;
  if (ks > kmax) ks = kmax;
  if (ks > 8) ks = 8;
  return ks < 1 ? 1 : (int)ks;
}

hipError_t launch_router_gemm(int T, int d, int E, const void* x, int xf32, const uint16_t* w,
                              double* part, int* nsum, hipStream_t s) {
  const int ks = router_mfma_splits(T, d, E);
  const int kc = ((d + ks - 1) / ks + kRmBK - 1) / kRmBK * kRmBK;
  const int nch = (d + kc - 1) / kc;
  *nsum = nch;
  dim3 grid((T + 63) / 64, (E + 63) / 64, nch);
  if (xf32) router_mfma_kernel<true><<<grid, 256, 0, s>>>(T, d, E, kc, x, w, part);
  else router_mfma_kernel<false><<<grid, 256, 0, s>>>(T, d, E, kc, x, w, part);
  return hipGetLastError();
}

hipError_t launch_route_topk(int T, int E, int k, const double* part, int nsum,
                             const float* bias, int32_t* ids, float* gates,
                             const BucketOut* bucket1, hipStream_t s) {
  Bucket1 b{};
  if (bucket1 && T == 1) {
    b.offsets = bucket1->offsets; b.rows = bucket1->rows; b.act = bucket1->act;
    b.n_act = bucket1->n_act; b.pair_pos = bucket1->pair_pos; b.pair_exp = bucket1->pair_exp;
    b.mtile_off = bucket1->mtile_off;
  }
  // four waves per token, up to 16 experts per thread; for few tokens (latency-bound) and
  // more than 256 experts the logits are first formed by a 1024-thread block, one expert
  // per thread
  const int kpt = (E + 255) / 256;
  const int nt = 256;
  if (kpt > 1 && T <= kRouterGemvMaxT) {
    if (kpt <= 2) route_topk_kernel<2, true><<<T, 1024, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
    else if (kpt <= 4) route_topk_kernel<4, true><<<T, 1024, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
    else if (kpt <= 8) route_topk_kernel<8, true><<<T, 1024, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
    else route_topk_kernel<16, true><<<T, 1024, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
    return hipGetLastError();
  }
  if (kpt <= 1) route_topk_kernel<1, false><<<T, nt, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
  else if (kpt <= 2) route_topk_kernel<2, false><<<T, nt, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
  else if (kpt <= 4) route_topk_kernel<4, false><<<T, nt, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
  else if (kpt <= 8) route_topk_kernel<8, false><<<T, nt, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
  else route_topk_kernel<16, false><<<T, nt, 0, s>>>(T, E, k, part, nsum, bias, ids, gates, b);
  return hipGetLastError();
}

bool route_shared_supported(int d, int E, int k, const uint16_t* w_router) {
  return d % 8 == 0 && d <= kNormMaxD && E % 8 == 0 && E > 256 && E <= kMaxE && k >= 1 &&
         k <= kMaxSlots && k <= E && (reinterpret_cast<uintptr_t>(w_router) & 15u) == 0;
}

namespace {
RouteSharedArgs route_shared_args(int d, int f, int E, int k, const float* h,
                                  const uint16_t* gamma, float eps, float* xhat,
                                  const uint16_t* w_router, const float* bias, double* part,
                                  const uint16_t* sh_gate, const uint16_t* sh_up,
                                  const uint16_t* sh_down, float* hsh, float* ssh, int32_t* ids,
                                  float* gates, const BucketOut& bucket1) {
  RouteSharedArgs a;
  a.d = d; a.f = f; a.E = E; a.k = k; a.h = h; a.gamma = gamma; a.eps = eps; a.xhat = xhat;
  a.w_router = w_router; a.part = part;
  a.nchunk = router_num_chunks(d);
  a.nrb = a.nchunk * ((E + kRouterCols - 1) / kRouterCols);
  a.sh_gate = sh_gate; a.sh_up = sh_up; a.sh_down = sh_down; a.hsh = hsh; a.ssh = ssh;
  a.bias = bias; a.ids = ids; a.gates = gates;
  a.bk = Bucket1{bucket1.offsets, bucket1.rows, bucket1.act, bucket1.n_act, bucket1.pair_pos,
                 bucket1.pair_exp, bucket1.mtile_off};
  return a;
}
}  // namespace

hipError_t launch_route_shared(int d, int f, int E, int k, const float* h,
                               const uint16_t* gamma, float eps, float* xhat,
                               const uint16_t* w_router, const float* bias, double* part,
                               const uint16_t* sh_gate, const uint16_t* sh_up,
                               const uint16_t* sh_down, float* hsh, float* ssh, int32_t* ids,
                               float* gates, const BucketOut& bucket1, int gateup_blocks,
                               hipStream_t s) {
  if (!route_shared_supported(d, E, k, w_router)) return hipErrorInvalidValue;
  const RouteSharedArgs a = route_shared_args(d, f, E, k, h, gamma, eps, xhat, w_router, bias,
                                              part, sh_gate, sh_up, sh_down, hsh, ssh, ids,
                                              gates, bucket1);
  // shared gate/up: one block per row group of 4 waves (gateup_blocks > 0 caps the count);
  // shared down: one block per row group of the top-k block's 16 waves
  const int rows_gu = gemv_group_rows(d, 4), rows_dn = gemv_group_rows(f, 16);
  int nsb = (f + rows_gu - 1) / rows_gu;
  if (gateup_blocks > 0 && nsb > gateup_blocks) nsb = gateup_blocks;
  router_shared_gateup_kernel<<<a.nrb + nsb, 256, (size_t)d * 4, s>>>(a);
  const int ndb = (d + rows_dn - 1) / rows_dn;
  const int kpt = (E + 255) / 256;
  const size_t lds = (size_t)f * 4;
  if (kpt <= 2) topk_shared_down_kernel<2><<<1 + ndb, 1024, lds, s>>>(a);
  else if (kpt <= 4) topk_shared_down_kernel<4><<<1 + ndb, 1024, lds, s>>>(a);
  else if (kpt <= 8) topk_shared_down_kernel<8><<<1 + ndb, 1024, lds, s>>>(a);
  else topk_shared_down_kernel<16><<<1 + ndb, 1024, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_norm_shared_gateup(int d, int f, int E, int k, const float* h,
                                           const uint16_t* gamma, float eps, float* xhat,
                                           const uint16_t* w_router, const float* bias,
                                           double* part, const uint16_t* sh_gate,
                                           const uint16_t* sh_up, float* hsh, int32_t* ids,
                                           float* gates, const BucketOut& bucket1,
                                           hipStream_t s) {
  if (!route_shared_supported(d, E, k, w_router)) return hipErrorInvalidValue;
  const RouteSharedArgs a = route_shared_args(d, f, E, k, h, gamma, eps, xhat, w_router, bias,
                                              part, sh_gate, sh_up, nullptr, hsh, nullptr, ids,
                                              gates, bucket1);
  router_norm_kernel<<<a.nrb, 256, 0, s>>>(a);
  const int rows_gu = gemv_group_rows(d, 4);
  const int nsb = (f + rows_gu - 1) / rows_gu;
  const int kpt = (E + 255) / 256;
  const size_t lds = (size_t)d * 4;
  if (kpt <= 2) topk_shared_gateup_kernel<2><<<1 + nsb, 256, lds, s>>>(a);
  else if (kpt <= 4) topk_shared_gateup_kernel<4><<<1 + nsb, 256, lds, s>>>(a);
  else if (kpt <= 8) topk_shared_gateup_kernel<8><<<1 + nsb, 256, lds, s>>>(a);
  else topk_shared_gateup_kernel<16><<<1 + nsb, 256, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace k3moe
