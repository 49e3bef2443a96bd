// bucket.hip — stable counting sort of (token, slot) pairs by expert on gfx950.
//
// Tokens are taken in blocks of 64. Within a block, each expert gets a 64-bit mask of
// the local tokens that chose it; since a token picks an expert at most once, the rank
// of pair (t, slot) inside its expert's list is the popcount of the mask bits below t.
// Per-block counts are scanned along the block axis (ascending token order) and then
// along experts, which yields offsets and the position of every pair. Only integer
// operations are involved, so the result is the same on every run.
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

constexpr int kMaxE = 4096;

// Exclusive scan of 4 consecutive values per thread across a 1024-thread block.
// Returns the exclusive prefix of this thread's first value; *total gets the sum.
__device__ int block_scan4(const int v[4], int out[4], int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sum = v[0] + v[1] + v[2] + v[3];
  int incl = sum;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int c = s_wave[w];
      s_wave[w] = run;
      run += c;
    }
    s_wave[16] = run;
  }
  __syncthreads();
  int ex = s_wave[wave] + incl - sum;
  for (int i = 0; i < 4; ++i) {
    out[i] = ex;
    ex += v[i];
  }
  *total = s_wave[16];
  __syncthreads();
  return out[0];
}

// Masks of one 64-token block into LDS.
__device__ void build_masks(int T, int E, int k, int b, const int32_t* ids,
                            unsigned long long* mask) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  const int t0 = b * kBucketTokens;
  const int t1 = min(T, t0 + kBucketTokens);
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicOr(&mask[e], 1ull << (p / k - t0));
  }
  __syncthreads();
}

__device__ void place_pairs(int T, int E, int k, int b, const int32_t* ids,
                            const unsigned long long* mask, const int32_t* base_of_e,
                            int32_t* rows, int32_t* pair_pos, int32_t* pair_exp) {
  const int t0 = b * kBucketTokens;
  const int t1 = min(T, t0 + kBucketTokens);
  for (int p = t0 * k + threadIdx.x; p < t1 * k; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int tl = p / k - t0;
      const unsigned long long below = (tl == 0) ? 0ull : (mask[e] & ((1ull << tl) - 1ull));
      const int pos = base_of_e[e] + __popcll(below);
      rows[pos] = p;
      pair_pos[p] = pos;
      pair_exp[p] = e;
    } else {
      pair_pos[p] = -1;
      pair_exp[p] = -1;
    }
  }
}

// Active-expert list and M-tile prefix of the grouped GEMM from per-expert counts v[].
__device__ void active_and_tiles(int E, const int v[4], int32_t* act, int32_t* n_act,
                                 int32_t* mtile_off, int* s_wave) {
  int f[4], fo[4], mt[4], mo[4];
  const int e0 = threadIdx.x * 4;
  for (int i = 0; i < 4; ++i) {
    f[i] = (e0 + i < E && v[i] > 0) ? 1 : 0;
    mt[i] = f[i] ? mfma_tiles_of(v[i]) : 0;
  }
  int nact, ntiles;
  block_scan4(f, fo, s_wave, &nact);
  block_scan4(mt, mo, s_wave, &ntiles);
  for (int i = 0; i < 4; ++i)
    if (f[i]) {
      act[fo[i]] = e0 + i;
      mtile_off[fo[i]] = mo[i];
    }
  if (threadIdx.x == 0) {
    *n_act = nact;
    mtile_off[nact] = ntiles;
  }
  __syncthreads();
}

// Counts per expert -> offsets [E+1], active list, n_act, M-tile prefix (one 1024-thread
// block). cnt_to_base: on return holds the first position of each expert.
__device__ void offsets_and_active(int E, int* cnt_to_base, const BucketOut& ob, int* s_wave) {
  int v[4], o[4];
  const int e0 = threadIdx.x * 4;
  for (int i = 0; i < 4; ++i) v[i] = (e0 + i < E) ? cnt_to_base[e0 + i] : 0;
  int total;
  block_scan4(v, o, s_wave, &total);
  active_and_tiles(E, v, ob.act, ob.n_act, ob.mtile_off, s_wave);
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    if (e < E) {
      ob.offsets[e] = o[i];
      cnt_to_base[e] = o[i];
    }
  }
  if (threadIdx.x == 0) ob.offsets[E] = total;
  __syncthreads();
}

// T <= 64: everything in one 1024-thread block.
__global__ __launch_bounds__(1024) void bucket_single_kernel(int T, int E, int k,
                                                             const int32_t* __restrict__ ids,
                                                             BucketOut o) {
  __shared__ unsigned long long mask[kMaxE];
  __shared__ int cnt[kMaxE];
  __shared__ int s_wave[17];
  build_masks(T, E, k, 0, ids, mask);
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = __popcll(mask[e]);
  __syncthreads();
  offsets_and_active(E, cnt, o, s_wave);
  place_pairs(T, E, k, 0, ids, mask, cnt, o.rows, o.pair_pos, o.pair_exp);
}

__global__ __launch_bounds__(256) void bucket_hist_kernel(int T, int E, int k,
                                                          const int32_t* __restrict__ ids,
                                                          uint32_t* __restrict__ hist,
                                                          uint64_t* __restrict__ masks) {
  __shared__ unsigned long long mask[kMaxE];
  const int b = blockIdx.x;
  build_masks(T, E, k, b, ids, mask);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    masks[(size_t)b * E + e] = mask[e];
    hist[(size_t)b * E + e] = (uint32_t)__popcll(mask[e]);
  }
}

__global__ __launch_bounds__(1024) void bucket_scan_kernel(int NB, int E,
                                                           const uint32_t* __restrict__ hist,
                                                           uint32_t* __restrict__ base,
                                                           BucketOut o) {
  __shared__ int cnt[kMaxE];
  __shared__ int s_wave[17];
  // totals first (independent loads, eight blocks' counts in flight at once), then the
  // offsets, then each block's base in one pass: no read-modify-write chains on base
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
#pragma unroll 8
    for (int b = 0; b < NB; ++b) run += (int)hist[(size_t)b * E + e];
    cnt[e] = run;
  }
  __syncthreads();
  offsets_and_active(E, cnt, o, s_wave);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    uint32_t run = (uint32_t)cnt[e];
#pragma unroll 8
    for (int b = 0; b < NB; ++b) {
      base[(size_t)b * E + e] = run;
      run += hist[(size_t)b * E + e];
    }
  }
}

__global__ __launch_bounds__(256) void bucket_place_kernel(int T, int E, int k,
                                                           const int32_t* __restrict__ ids,
                                                           const uint32_t* __restrict__ base,
                                                           const uint64_t* __restrict__ masks,
                                                           BucketOut o) {
  __shared__ unsigned long long mask[kMaxE];
  __shared__ int32_t bs[kMaxE];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    mask[e] = masks[(size_t)b * E + e];
    bs[e] = (int32_t)base[(size_t)b * E + e];
  }
  __syncthreads();
  place_pairs(T, E, k, b, ids, mask, bs, o.rows, o.pair_pos, o.pair_exp);
}

// Caller-supplied bucket -> active list and per-pair position/expert.
__global__ __launch_bounds__(1024) void pairs_from_bucket_kernel(int T, int E, int k,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ rows,
                                                                 BucketOut o) {
  __shared__ int cnt[kMaxE];
  __shared__ int s_wave[17];
  const int P = T * k;
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    o.pair_pos[p] = -1;
    o.pair_exp[p] = -1;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int a = min(max(offsets[e], 0), P), z = min(max(offsets[e + 1], 0), P);
    cnt[e] = max(z - a, 0);
  }
  __syncthreads();
  // the caller's offsets stay as they are; only the active list and tiles are derived
  int v[4];
  const int e0 = threadIdx.x * 4;
  for (int i = 0; i < 4; ++i) v[i] = (e0 + i < E) ? cnt[e0 + i] : 0;
  active_and_tiles(E, v, o.act, o.n_act, o.mtile_off, s_wave);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int a = min(max(offsets[e], 0), P), z = min(max(offsets[e + 1], 0), P);
    for (int p = a; p < z; ++p) {
      const int pr = rows[p];
      if (pr >= 0 && pr < P) {
        o.pair_pos[pr] = p;
        o.pair_exp[pr] = e;
      }
    }
  }
}

}  // namespace

hipError_t launch_bucket(int T, int E, int k, const int32_t* ids, const BucketOut& o,
                         uint32_t* hist, uint32_t* base, uint64_t* masks, hipStream_t s) {
  const int NB = (T + kBucketTokens - 1) / kBucketTokens;
  if (NB <= 1) {
    bucket_single_kernel<<<1, 1024, 0, s>>>(T, E, k, ids, o);
    return hipGetLastError();
  }
  bucket_hist_kernel<<<NB, 256, 0, s>>>(T, E, k, ids, hist, masks);
  bucket_scan_kernel<<<1, 1024, 0, s>>>(NB, E, hist, base, o);
  bucket_place_kernel<<<NB, 256, 0, s>>>(T, E, k, ids, base, masks, o);
  return hipGetLastError();
}

hipError_t launch_pairs_from_bucket(int T, int E, int k, const int32_t* offsets,
                                    const int32_t* rows, const BucketOut& o, hipStream_t s) {
  pairs_from_bucket_kernel<<<1, 1024, 0, s>>>(T, E, k, offsets, rows, o);
  return hipGetLastError();
}

}  // namespace k3moe
