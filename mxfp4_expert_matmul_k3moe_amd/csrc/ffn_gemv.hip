// ffn_gemv.hip — MXFP4 expert GEMVs for few tokens per expert (decode, batched decode).
//
// The expert weights are streamed from HBM with 16-byte loads: one load is one
// 32-element MXFP4 block of one row (16 packed bytes), whose E8M0 scale is one more
// byte. The block is decoded in registers (gfx950 scaled FP4 conversion), multiplied
// against 32 activations, summed, and only then scaled by the block's power of two.
// Nothing dequantised is written anywhere. Rows are split over aligned groups of
// `lpr` lanes (the largest power of two dividing the row's block count), so a row's
// partial sums are reduced inside its lane group with a fixed shuffle tree.
//
// Expert form: E(x) = D (silu(G x) * (U x)) (SwiGLU without biases); combine:
// y_t = sum over slots in slot order of gate * E(x_t), following "Kimi K3 纯 C 语言 CPU
// 推理实战" (chenxutan.com/d/5901.html) §1.2 and §2.4, with the weight layout [N][K] and
// 32-element scale groups of its §2.3 quantised GEMM.
#include "k3moe_device.h"
#include "k3moe_launch.h"

namespace k3moe {
namespace {

constexpr int kGateUpWaves = 4;
constexpr int kMaxTokGroup = 4;
constexpr int kLdsBudget = 64 * 1024;

struct GateUpArgs {
  int T, d, f, k;
  const void* x;
  const uint8_t *gq, *gs, *uq, *us;
  const int32_t *offsets, *rows, *act, *n_act;
  int nchunk, rc, tg;
  float* h;
};

// LDS layout of one staged activation row: block cb = sub + lpr*i, 16-byte piece qq of
// that block goes to chunk ((i*Q + qq)*lpr + sub), so the lanes of a row group read
// consecutive 16-byte chunks (no bank conflicts). Q = pieces per block (4 bf16 / 8 f32).
__device__ __forceinline__ int x_chunk(int cb, int qq, int lpr, int Q) {
  const int i = cb / lpr, sub = cb - i * lpr;
  return (i * Q + qq) * lpr + sub;
}

template <bool XF32, int BPLC, int TGM>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(GateUpArgs a) {
  extern __shared__ __attribute__((aligned(16))) u32x4 xs[];
  constexpr int Q = XF32 ? 8 : 4;  // 16-byte pieces per 32-element block
  const int item = blockIdx.x;
  const int ai = item / a.nchunk, c = item - ai * a.nchunk;
  if (ai >= *a.n_act) return;
  const int e = a.act[ai];
  const int P = a.T * a.k;
  const int p0 = min(max(a.offsets[e], 0), P), p1 = min(max(a.offsets[e + 1], p0), P);
  const int d = a.d, f = a.f;
  const int NB = d >> 5;
  const int lpr = lanes_per_row(NB), bpl = NB / lpr, rpw = 64 / lpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const int j0 = c * a.rc, j1 = min(f, j0 + a.rc);
  const size_t rq = (size_t)(d >> 1), rs = (size_t)NB;
  const uint8_t* gq = a.gq + (size_t)e * f * rq;
  const uint8_t* uq = a.uq + (size_t)e * f * rq;
  const uint8_t* gs = a.gs + (size_t)e * f * rs;
  const uint8_t* us = a.us + (size_t)e * f * rs;
  const int chunks_per_tok = NB * Q;

  for (int pg = p0; pg < p1; pg += a.tg) {
    const int ntok = min(a.tg, p1 - pg);
    __syncthreads();
    for (int tok = 0; tok < ntok; ++tok) {
      const int pair = a.rows[pg + tok];
      const bool ok = pair >= 0 && pair < P;  // caller-supplied buckets are not trusted
      const int t = ok ? pair / a.k : 0;
      const u32x4* src = reinterpret_cast<const u32x4*>(
          static_cast<const uint8_t*>(a.x) + (size_t)t * d * (XF32 ? 4 : 2));
      for (int v = threadIdx.x; v < chunks_per_tok; v += 256) {
        const int cb = v / Q, qq = v - cb * Q;
        xs[tok * chunks_per_tok + x_chunk(cb, qq, lpr, Q)] = ok ? src[v] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();
    for (int jb = j0 + wave * rpw; jb < j1; jb += kGateUpWaves * rpw) {
      const int j = jb + rsel;
      const bool rv = j < j1;
      float gacc[TGM], uacc[TGM];
#pragma unroll
      for (int tk = 0; tk < TGM; ++tk) gacc[tk] = uacc[tk] = 0.0f;
      for (int i0 = 0; i0 < bpl; i0 += BPLC) {
        u32x4 gw[BPLC], uw[BPLC];
        uint32_t gsc[BPLC], usc[BPLC];
#pragma unroll
        for (int ii = 0; ii < BPLC; ++ii) {
          const int i = i0 + ii;
          const int cb = sub + lpr * i;
          if (rv && i < bpl) {
            gw[ii] = load_u32x4_nt(gq + (size_t)j * rq + (size_t)cb * 16);
            uw[ii] = load_u32x4_nt(uq + (size_t)j * rq + (size_t)cb * 16);
            gsc[ii] = gs[(size_t)j * rs + cb];
            usc[ii] = us[(size_t)j * rs + cb];
          }
        }
#pragma unroll
        for (int tk = 0; tk < TGM; ++tk) {
          if (tk < ntok) {
            const u32x4* xt = xs + tk * chunks_per_tok;
#pragma unroll
            for (int ii = 0; ii < BPLC; ++ii) {
              const int i = i0 + ii;
              if (rv && i < bpl) {
                const int cb = sub + lpr * i;
                if constexpr (XF32) {
                  float xv[32];
#pragma unroll
                  for (int qq = 0; qq < 8; ++qq) {
                    const u32x4 v = xt[x_chunk(cb, qq, lpr, 8)];
                    xv[4 * qq + 0] = __uint_as_float(v[0]);
                    xv[4 * qq + 1] = __uint_as_float(v[1]);
                    xv[4 * qq + 2] = __uint_as_float(v[2]);
                    xv[4 * qq + 3] = __uint_as_float(v[3]);
                  }
                  gacc[tk] = fmaf(e8m0_to_f32(gsc[ii]), block_dot_f32(gw[ii], xv), gacc[tk]);
                  uacc[tk] = fmaf(e8m0_to_f32(usc[ii]), block_dot_f32(uw[ii], xv), uacc[tk]);
                  // keeps the next block's 32 activations from being read early: holding
                  // every block's would cost 32 registers each
                  asm volatile("" ::: "memory");
                } else {
                  uint32_t xp[16];
#pragma unroll
                  for (int qq = 0; qq < 4; ++qq) {
                    const u32x4 v = xt[x_chunk(cb, qq, lpr, 4)];
                    xp[4 * qq + 0] = v[0];
                    xp[4 * qq + 1] = v[1];
                    xp[4 * qq + 2] = v[2];
                    xp[4 * qq + 3] = v[3];
                  }
                  gacc[tk] = fmaf(e8m0_to_f32(gsc[ii]), block_dot_bf16(gw[ii], xp), gacc[tk]);
                  uacc[tk] = fmaf(e8m0_to_f32(usc[ii]), block_dot_bf16(uw[ii], xp), uacc[tk]);
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int tk = 0; tk < TGM; ++tk) {
        if (tk < ntok) {
          const float g = group_sum_rt(gacc[tk], lpr);
          const float u = group_sum_rt(uacc[tk], lpr);
          if (rv && sub == 0) a.h[(size_t)(pg + tk) * f + j] = silu_f32(g) * u;
        }
      }
    }
  }
}

struct DownT1Args {
  int d, f, k;
  const uint8_t *dq, *ds;
  const float* h;
  const int32_t *pair_pos, *pair_exp;
  const float* gates;
  const float *resid, *shared;
  float* y;
  uint16_t* y_bf16;
  int rc;
};

constexpr int kMaxSlots = 32;

// ---- gate/up, T == 1: one token, persistent over (expert, row group) ----------------------
// The token is staged in LDS once per block. Each wave walks row groups (rpw rows of G and
// the same rows of U of one selected expert) with a stride of all waves in the grid, and
// issues the loads of its next group before computing the current one.
struct GateUpDecodeArgs {
  int d, f;
  const void* x;
  const uint8_t *gq, *gs, *uq, *us;
  const int32_t *offsets, *act, *n_act;
  float* h;
};

template <bool XF32, int BPL>
__global__ __launch_bounds__(256, 2) void gateup_decode_kernel(GateUpDecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) u32x4 xs[];
  constexpr int Q = XF32 ? 8 : 4;
  const int d = a.d, f = a.f;
  const int NB = d >> 5;
  const int lpr = lanes_per_row(NB), rpw = 64 / lpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const size_t rq = (size_t)(d >> 1), rs = (size_t)NB;
  {
    const u32x4* src = static_cast<const u32x4*>(a.x);
    for (int v = threadIdx.x; v < NB * Q; v += 256) {
      const int cb = v / Q, qq = v - cb * Q;
      xs[x_chunk(cb, qq, lpr, Q)] = src[v];
    }
  }
  __syncthreads();
  const int rgpe = (f + rpw - 1) / rpw;  // row groups per expert
  const int total = *a.n_act * rgpe;
  const int stride = gridDim.x * kGateUpWaves;
  for (int rg = blockIdx.x * kGateUpWaves + wave; rg < total; rg += stride) {
    const int ai = rg / rgpe;
    const int j = (rg - ai * rgpe) * rpw + rsel;
    const int e = a.act[ai];
    const bool rv = j < f;
    const size_t row = (size_t)e * f + (rv ? j : 0);
    u32x4 gw[BPL], uw[BPL];
    uint32_t gsc[BPL], usc[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const size_t cb = (size_t)(sub + lpr * i);
      gw[i] = load_u32x4_nt(a.gq + row * rq + cb * 16);
      uw[i] = load_u32x4_nt(a.uq + row * rq + cb * 16);
      gsc[i] = a.gs[row * rs + cb];
      usc[i] = a.us[row * rs + cb];
    }
    float gacc = 0.0f, uacc = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const u32x4* xb = xs + (i * Q) * lpr + sub;  // piece qq of this lane's block i
      if constexpr (XF32) {
        float xv[32];
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          const u32x4 v = xb[qq * lpr];
          xv[4 * qq + 0] = __uint_as_float(v[0]);
          xv[4 * qq + 1] = __uint_as_float(v[1]);
          xv[4 * qq + 2] = __uint_as_float(v[2]);
          xv[4 * qq + 3] = __uint_as_float(v[3]);
        }
        gacc = fmaf(e8m0_to_f32(gsc[i]), block_dot_f32(gw[i], xv), gacc);
        uacc = fmaf(e8m0_to_f32(usc[i]), block_dot_f32(uw[i], xv), uacc);
        // one block at a time: the next block's weights are converted (and its 32
        // activations read) only after this block's sums; converting every block first
        // would hold 64 fp32 values per block and halve the occupancy
        if (i + 1 < BPL) asm volatile("" : "+v"(gacc), "+v"(uacc), "+v"(gw[i + 1]), "+v"(uw[i + 1])::"memory");
      } else {
        uint32_t xp[16];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const u32x4 v = xb[qq * lpr];
          xp[4 * qq + 0] = v[0];
          xp[4 * qq + 1] = v[1];
          xp[4 * qq + 2] = v[2];
          xp[4 * qq + 3] = v[3];
        }
        gacc = fmaf(e8m0_to_f32(gsc[i]), block_dot_bf16(gw[i], xp), gacc);
        uacc = fmaf(e8m0_to_f32(usc[i]), block_dot_bf16(uw[i], xp), uacc);
        // likewise one block at a time (converting all blocks first takes 247 registers)
        if (i + 1 < BPL) asm volatile("" : "+v"(gacc), "+v"(uacc), "+v"(gw[i + 1]), "+v"(uw[i + 1])::"memory");
      }
    }
    const float g = group_sum_rt(gacc, lpr);
    const float u = group_sum_rt(uacc, lpr);
    if (sub == 0 && rv) a.h[(size_t)a.offsets[e] * f + j] = silu_f32(g) * u;
  }
}

// ---- down, T == 1: all slots of the token, ordered combine ---------------------------------
// Lane group q (lpr lanes) owns slot q and keeps that slot's slice of h in registers. A
// block owns `rpb` consecutive output rows: it walks them R rows at a time (all R*BPL
// loads of a step issued together), parks each row's k partial results in LDS, and after
// one barrier adds them per row in slot order. No barrier and no global store sits inside
// the row loop, so loads of consecutive steps overlap across the block's waves.
constexpr int kDecMaxRows = 64;  // rows per block (LDS holds k x rpb partials)

template <int BPL, int R>
__global__ __launch_bounds__(512) void down_decode_kernel(DownT1Args a) {
  __shared__ float zs[kMaxSlots][kDecMaxRows];
  __shared__ float gsh[kMaxSlots];
  const int d = a.d, f = a.f, k = a.k;
  const int NB = f >> 5;
  const int lpr = lanes_per_row(NB);
  const int tid = threadIdx.x, lane = tid & 63;
  const int q = tid / lpr, sub = lane & (lpr - 1);
  if (tid < k) gsh[tid] = a.gates[tid];
  const int pos = (q < k) ? a.pair_pos[q] : -1;
  const int e = (q < k) ? a.pair_exp[q] : -1;
  const bool sv = pos >= 0 && e >= 0;
  // loads are unconditional (clamped to valid addresses) and masked afterwards, so the
  // compiler can keep many of them in flight
  const float hmask = sv ? 1.0f : 0.0f;
  float hv[BPL][32];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int cb = sub + lpr * i;
    const f32x4* src = reinterpret_cast<const f32x4*>(a.h + (size_t)(sv ? pos : 0) * f + cb * 32);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f32x4 t = src[v];
      hv[i][4 * v + 0] = t[0] * hmask;
      hv[i][4 * v + 1] = t[1] * hmask;
      hv[i][4 * v + 2] = t[2] * hmask;
      hv[i][4 * v + 3] = t[3] * hmask;
    }
  }
  const size_t rq = (size_t)(f >> 1), rs = (size_t)NB;
  const uint8_t* dq = a.dq + (size_t)(sv ? e : 0) * d * rq;
  const uint8_t* dsc = a.ds + (size_t)(sv ? e : 0) * d * rs;
  const int r0 = blockIdx.x * a.rc;
  const int r1 = min(d, r0 + a.rc);
  for (int rb = r0; rb < r1; rb += R) {
    u32x4 w[R][BPL];
    uint32_t sc[R][BPL];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int r = min(rb + u, r1 - 1);
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const int cb = sub + lpr * i;
        w[u][i] = load_u32x4_nt(dq + (size_t)r * rq + (size_t)cb * 16);
        sc[u][i] = dsc[(size_t)r * rs + cb];
      }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int r = rb + u;
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) p = fmaf(e8m0_to_f32(sc[u][i]), block_dot_f32(w[u][i], hv[i]), p);
      const float zz = group_sum_rt(p, lpr);
      if (q < k && sub == 0 && r < r1) zs[q][r - r0] = sv ? zz : 0.0f;
    }
  }
  __syncthreads();
  for (int rl = tid; rl < r1 - r0; rl += blockDim.x) {
    const int r = r0 + rl;
    float acc = 0.0f;
    for (int s2 = 0; s2 < k; ++s2) acc = fmaf(gsh[s2], zs[s2][rl], acc);
    float out = acc;
    if (a.resid) out = (a.resid[r] + (a.shared ? a.shared[r] : 0.0f)) + acc;
    a.y[r] = out;
    if (a.y_bf16) a.y_bf16[r] = f32_to_bf16_rne(out);
  }
}

// ---- down projection per expert (any T) into pair-indexed z --------------------------------
struct DownArgs {
  int T, d, f, k;
  const uint8_t *dq, *ds;
  const float* h;
  const int32_t *offsets, *rows, *act, *n_act;
  int nchunk, rc;
  float* z;
};

template <int BPL>
__global__ __launch_bounds__(256) void down_gemv_kernel(DownArgs a) {
  const int item = blockIdx.x;
  const int ai = item / a.nchunk, c = item - ai * a.nchunk;
  if (ai >= *a.n_act) return;
  const int e = a.act[ai];
  const int P = a.T * a.k;
  const int p0 = min(max(a.offsets[e], 0), P), p1 = min(max(a.offsets[e + 1], p0), P);
  const int d = a.d, f = a.f;
  const int NB = f >> 5;
  const int lpr = lanes_per_row(NB), rpw = 64 / lpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1), rsel = lane / lpr;
  const int i0r = c * a.rc, i1r = min(d, i0r + a.rc);
  const size_t rq = (size_t)(f >> 1), rs = (size_t)NB;
  const uint8_t* dq = a.dq + (size_t)e * d * rq;
  const uint8_t* dsc = a.ds + (size_t)e * d * rs;
  for (int p = p0; p < p1; ++p) {
    const int pair = a.rows[p];
    if (pair < 0 || pair >= P) continue;
    float hv[BPL][32];
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int cb = sub + lpr * i;
      const f32x4* src = reinterpret_cast<const f32x4*>(a.h + (size_t)p * f + cb * 32);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const f32x4 t = src[v];
        hv[i][4 * v + 0] = t[0];
        hv[i][4 * v + 1] = t[1];
        hv[i][4 * v + 2] = t[2];
        hv[i][4 * v + 3] = t[3];
      }
    }
    for (int rb = i0r + wave * rpw; rb < i1r; rb += 4 * rpw) {
      const int r = rb + rsel;
      const bool rv = r < i1r;
      u32x4 w[BPL];
      uint32_t sc[BPL];
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const int cb = sub + lpr * i;
        if (rv) {
          w[i] = load_u32x4(dq + (size_t)r * rq + (size_t)cb * 16);
          sc[i] = dsc[(size_t)r * rs + cb];
        }
      }
      float acc = 0.0f;
      if (rv) {
#pragma unroll
        for (int i = 0; i < BPL; ++i) acc = fmaf(e8m0_to_f32(sc[i]), block_dot_f32(w[i], hv[i]), acc);
      }
      const float zz = group_sum_rt(acc, lpr);
      if (rv && sub == 0) a.z[(size_t)pair * d + r] = zz;
    }
  }
}

// ---- combine -----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(int T, int d, int k, const float* __restrict__ z,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ resid,
                                                      const float* __restrict__ shared,
                                                      float* __restrict__ y,
                                                      uint16_t* __restrict__ y_bf16, int bf16_vec,
                                                      int nbx) {
  // four consecutive outputs per thread (16-byte loads of z); the z rows of up to 8 slots
  // are requested before any of them is added, and slots are added in slot order. One
  // grid dimension: token t takes blocks [t nbx, (t + 1) nbx), so T is not bound by the
  // 65536 blocks the device reports for its other grid dimensions.
  const int t = (int)(blockIdx.x / (unsigned)nbx);
  const int i = ((int)(blockIdx.x - (unsigned)t * (unsigned)nbx) * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < k; s0 += 8) {
    f32x4 v[8];
    float g[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pr = t * k + min(s0 + u, k - 1);  // clamped: always a valid row
      ok[u] = (s0 + u < k) && pair_pos[pr] >= 0;
      g[u] = gates[pr];
      v[u] = *reinterpret_cast<const f32x4*>(z + (size_t)pr * d + i);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (ok[u]) {
        acc[0] = fmaf(g[u], v[u][0], acc[0]);
        acc[1] = fmaf(g[u], v[u][1], acc[1]);
        acc[2] = fmaf(g[u], v[u][2], acc[2]);
        acc[3] = fmaf(g[u], v[u][3], acc[3]);
      }
  }
  const size_t o = (size_t)t * d + i;
  f32x4 out = acc;
  if (resid) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(resid + o);
    const f32x4 sh = shared ? *reinterpret_cast<const f32x4*>(shared + o) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = (r[c] + sh[c]) + acc[c];
  }
  *reinterpret_cast<f32x4*>(y + o) = out;
  if (y_bf16) {
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(out[0]) | ((uint32_t)f32_to_bf16_rne(out[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(out[2]) | ((uint32_t)f32_to_bf16_rne(out[3]) << 16);
    if (bf16_vec) {
      *reinterpret_cast<uint2*>(y_bf16 + o) = make_uint2(lo, hi);
    } else {
      y_bf16[o] = (uint16_t)lo;
      y_bf16[o + 1] = (uint16_t)(lo >> 16);
      y_bf16[o + 2] = (uint16_t)hi;
      y_bf16[o + 3] = (uint16_t)(hi >> 16);
    }
  }
}

int bpl_of(int nb) { return nb / lanes_per_row(nb); }

constexpr int kMaxDecodeBpl = 8;

}  // namespace

bool down_fused_supported(int f, int k) { return k * lanes_per_row(f >> 5) <= 512; }

// The T == 1 gate/up kernel holds all of a lane's blocks of one row at once (one pass, at
// most 8 per lane); wider rows (e.g. d_model = 288, 2304, 4608: 9 blocks per lane) take the
// per-expert GEMV kernel, which walks the row in groups of 8.
bool gateup_decode_supported(int d) { return bpl_of(d >> 5) <= kMaxDecodeBpl; }

bool gemv_shape_supported(int d, int f) {
  // down projections keep a row slice of h in registers: at most 4 blocks per lane
  const int bd = bpl_of(f >> 5);
  return (d % 32 == 0) && (f % 32 == 0) && bd >= 1 && bd <= 4 &&
         (size_t)d * 4 <= (size_t)kLdsBudget;
}

hipError_t launch_gateup_gemv(int T, int d, int f, int E, int k, const void* x, int xf32,
                              const MxPtrs& w, const int32_t* offsets, const int32_t* rows,
                              const int32_t* act, const int32_t* n_act, int max_act, float* h,
                              hipStream_t s) {
  GateUpArgs a;
  a.T = T; a.d = d; a.f = f; a.k = k; a.x = x;
  a.gq = w.gate_q; a.gs = w.gate_s; a.uq = w.up_q; a.us = w.up_s;
  a.offsets = offsets; a.rows = rows; a.act = act; a.n_act = n_act; a.h = h;
  const int NB = d >> 5;
  const int lpr = lanes_per_row(NB), bpl = NB / lpr, rpw = 64 / lpr;
  const size_t xrow = (size_t)d * (xf32 ? 4 : 2);
  int tg = (T == 1) ? 1 : (int)(kLdsBudget / xrow);
  tg = tg < 1 ? 1 : (tg > kMaxTokGroup ? kMaxTokGroup : tg);
  a.tg = tg;
  // rows per block: two row-iterations per wave
  a.rc = kGateUpWaves * rpw * 2;
  a.nchunk = (f + a.rc - 1) / a.rc;
  const size_t lds = (size_t)tg * xrow;
  dim3 grid((unsigned)(max_act * a.nchunk));
  const int bplc = bpl <= 8 ? bpl : 8;
#define K3_GU(XF, B, TG) \
  gateup_gemv_kernel<XF, B, TG><<<grid, 256, lds, s>>>(a)
#define K3_GU_B(XF, TG)                   \
  switch (bplc) {                         \
    case 1: K3_GU(XF, 1, TG); break;      \
    case 2: K3_GU(XF, 2, TG); break;      \
    case 3: K3_GU(XF, 3, TG); break;      \
    case 4: K3_GU(XF, 4, TG); break;      \
    case 5: K3_GU(XF, 5, TG); break;      \
    case 6: K3_GU(XF, 6, TG); break;      \
    case 7: K3_GU(XF, 7, TG); break;      \
    default: K3_GU(XF, 8, TG); break;     \
  }
  if (xf32) {
    if (tg == 1) { K3_GU_B(true, 1) } else { K3_GU_B(true, 4) }
  } else {
    if (tg == 1) { K3_GU_B(false, 1) } else { K3_GU_B(false, 4) }
  }
#undef K3_GU_B
#undef K3_GU
  return hipGetLastError();
}

hipError_t launch_gateup_decode(int d, int f, int k, const void* x, int xf32, const MxPtrs& w,
                                const int32_t* offsets, const int32_t* act, const int32_t* n_act,
                                float* h, int n_cu, hipStream_t s, int blocks_per_cu) {
  GateUpDecodeArgs a;
  a.d = d; a.f = f; a.x = x;
  a.gq = w.gate_q; a.gs = w.gate_s; a.uq = w.up_q; a.us = w.up_s;
  a.offsets = offsets; a.act = act; a.n_act = n_act; a.h = h;
  const int NB = d >> 5;
  const int lpr = lanes_per_row(NB), bpl = NB / lpr, rpw = 64 / lpr;
  const int rgpe = (f + rpw - 1) / rpw;
  const int waves = k * rgpe;  // upper bound of row groups
  int grid = (waves + kGateUpWaves - 1) / kGateUpWaves;
  // resident blocks per CU: 4 for bf16 tokens (127 registers, four waves per SIMD; 2 / 3 /
  // 4 blocks measured 42.7 / 37.9 / 36.4 us on the K3 decode layer), 2 for fp32 tokens (177
  // registers leave room for two)
  if (blocks_per_cu <= 0) blocks_per_cu = xf32 ? 2 : 4;
  const int cap = blocks_per_cu * n_cu;
  if (grid > cap) grid = cap;
  if (bpl > kMaxDecodeBpl) return hipErrorInvalidValue;  // see gateup_decode_supported
  const size_t lds = (size_t)d * (xf32 ? 4 : 2);
#define K3_GD(XF, B) \
  launch_timed(gateup_decode_kernel<XF, B>, dim3(grid), dim3(256), (uint32_t)lds, s, a)
#define K3_GD_B(XF)                   \
  switch (bpl) {                      \
    case 1: K3_GD(XF, 1); break;      \
    case 2: K3_GD(XF, 2); break;      \
    case 3: K3_GD(XF, 3); break;      \
    case 4: K3_GD(XF, 4); break;      \
    case 5: K3_GD(XF, 5); break;      \
    case 6: K3_GD(XF, 6); break;      \
    case 7: K3_GD(XF, 7); break;      \
    default: K3_GD(XF, 8); break;     \
  }
  if (xf32) { K3_GD_B(true) } else { K3_GD_B(false) }
#undef K3_GD_B
#undef K3_GD
  return hipGetLastError();
}

hipError_t launch_down_decode(int d, int f, int k, const MxPtrs& w, const float* h,
                              const int32_t* pair_pos, const int32_t* pair_exp,
                              const float* gates, const float* resid, const float* shared,
                              float* y, uint16_t* y_bf16, int n_cu, hipStream_t s,
                              int rows_per_block, int rows_per_step) {
  // the MFMA kernel reads the scales as dwords: it needs them 4-byte aligned
  if (rows_per_block == 0 && (reinterpret_cast<uintptr_t>(w.down_s) & 3u) == 0 &&
      down_decode_mfma_supported(d, f, k))
    return launch_down_decode_mfma(d, f, k, w, h, pair_pos, pair_exp, gates, resid, shared, y,
                                   y_bf16, n_cu, s);
  DownT1Args a;
  a.d = d; a.f = f; a.k = k; a.dq = w.down_q; a.ds = w.down_s; a.h = h;
  a.pair_pos = pair_pos; a.pair_exp = pair_exp; a.gates = gates;
  a.resid = resid; a.shared = shared; a.y = y; a.y_bf16 = y_bf16;
  const int NB = f >> 5;
  const int lpr = lanes_per_row(NB);
  const int threads = ((k * lpr + 63) / 64) * 64;
  int rpb = rows_per_block;
  if (rpb <= 0) {  // about two blocks per CU
    rpb = (d + 2 * n_cu - 1) / (2 * n_cu);
    rpb = (rpb + 3) / 4 * 4;
  }
  if (rpb > kDecMaxRows) rpb = kDecMaxRows;
  if (rpb < 1) rpb = 1;
  a.rc = rpb;
  const int grid = (d + rpb - 1) / rpb;
#define K3_DD(B, R) down_decode_kernel<B, R><<<grid, threads, 0, s>>>(a)
#define K3_DD_R(B)                         \
  switch (rows_per_step) {                 \
    case 2: K3_DD(B, 2); break;            \
    case 8: K3_DD(B, 8); break;            \
    default: K3_DD(B, 4); break;           \
  }
  switch (bpl_of(NB)) {
    case 1: K3_DD_R(1) break;
    case 2: K3_DD_R(2) break;
    case 3: K3_DD_R(3) break;
    default: K3_DD_R(4) break;
  }
#undef K3_DD_R
#undef K3_DD
  return hipGetLastError();
}

hipError_t launch_down_gemv(int T, int d, int f, int E, int k, const MxPtrs& w, const float* h,
                            const int32_t* offsets, const int32_t* rows, const int32_t* act,
                            const int32_t* n_act, int max_act, float* z, hipStream_t s) {
  DownArgs a;
  a.T = T; a.d = d; a.f = f; a.k = k; a.dq = w.down_q; a.ds = w.down_s; a.h = h;
  a.offsets = offsets; a.rows = rows; a.act = act; a.n_act = n_act; a.z = z;
  const int NB = f >> 5;
  const int rpw = 64 / lanes_per_row(NB);
  a.rc = 4 * rpw * 4;
  a.nchunk = (d + a.rc - 1) / a.rc;
  dim3 grid((unsigned)(max_act * a.nchunk));
  switch (bpl_of(NB)) {
    case 1: down_gemv_kernel<1><<<grid, 256, 0, s>>>(a); break;
    case 2: down_gemv_kernel<2><<<grid, 256, 0, s>>>(a); break;
    case 3: down_gemv_kernel<3><<<grid, 256, 0, s>>>(a); break;
    default: down_gemv_kernel<4><<<grid, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(int T, int d, int k, const float* z, const float* gates,
                          const int32_t* pair_pos, const float* resid, const float* shared,
                          float* y, uint16_t* y_bf16, hipStream_t s) {
  // d is a multiple of 32; y and resid are 16-byte aligned (checked at the boundary)
  const int nbx = (d / 4 + 255) / 256;
  const dim3 grid((unsigned)nbx * (unsigned)T);  // T <= 2^20, nbx <= 16
  const int bf16_vec = (reinterpret_cast<uintptr_t>(y_bf16) & 7u) == 0;
  combine_kernel<<<grid, 256, 0, s>>>(T, d, k, z, gates, pair_pos, resid, shared, y, y_bf16,
                                      bf16_vec, nbx);
  return hipGetLastError();
}

}  // namespace k3moe
