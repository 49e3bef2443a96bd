// k3moe_device.h — device-side helpers shared by the gfx950 kernels of libk3moe.
//
// MXFP4 element decoding uses the gfx950 scaled FP4 conversions, which map one
// byte (two E2M1 nibbles) to a packed pair. E8M0 scale bytes are turned into fp32
// powers of two and applied once per 32-element block after the block's own
// sum (the pages' "accumulate on the packed codes, multiply by the scale once").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k3moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 byte -> 2^(s-127) as fp32: s=0 is the subnormal 2^-127, s=255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7FC00000u : bits;
  return __uint_as_float(bits);
}

// Unscaled E2M1 pair of byte `B` of `w`: element 2j (low nibble) in .x, 2j+1 in .y.
template <int B>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// Sum of one 32-element MXFP4 block (16 packed bytes in q) against 32 bf16
// activations (16 packed pairs in xp), unscaled. Products are exact in fp32.
__device__ __forceinline__ float block_dot_bf16(const u32x4 q, const uint32_t* xp) {
  float s = 0.0f;
#define K3_STEP(W, B) s = dot2_bf16(fp4x2_to_bf16<B>(q[W]), __builtin_bit_cast(bf16x2, xp[4 * (W) + (B)]), s)
  K3_STEP(0, 0); K3_STEP(0, 1); K3_STEP(0, 2); K3_STEP(0, 3);
  K3_STEP(1, 0); K3_STEP(1, 1); K3_STEP(1, 2); K3_STEP(1, 3);
  K3_STEP(2, 0); K3_STEP(2, 1); K3_STEP(2, 2); K3_STEP(2, 3);
  K3_STEP(3, 0); K3_STEP(3, 1); K3_STEP(3, 2); K3_STEP(3, 3);
#undef K3_STEP
  return s;
}

// Same block against 32 fp32 activations.
__device__ __forceinline__ float block_dot_f32(const u32x4 q, const float* xv) {
  float s = 0.0f;
#define K3_STEP(W, B)                                   \
  {                                                     \
    f32x2 v = fp4x2_to_f32<B>(q[W]);                    \
    s = fmaf(v.x, xv[8 * (W) + 2 * (B)], s);            \
    s = fmaf(v.y, xv[8 * (W) + 2 * (B) + 1], s);        \
  }
  K3_STEP(0, 0); K3_STEP(0, 1); K3_STEP(0, 2); K3_STEP(0, 3);
  K3_STEP(1, 0); K3_STEP(1, 1); K3_STEP(1, 2); K3_STEP(1, 3);
  K3_STEP(2, 0); K3_STEP(2, 1); K3_STEP(2, 2); K3_STEP(2, 3);
  K3_STEP(3, 0); K3_STEP(3, 1); K3_STEP(3, 2); K3_STEP(3, 3);
#undef K3_STEP
  return s;
}

__device__ __forceinline__ u32x4 load_u32x4(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load_u32x4_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// The value that lane (lane ^ M) of the wave holds, M in {1, 2, 4, 8, 16, 32}: DPP moves within
// rows of 16 lanes (quad permutations, the half-row mirror, a row rotation by 8) and the
// gfx950 permlane swaps across rows, all VALU operations, so a butterfly stage costs no LDS
// round trip (a bpermute does). lane = this thread's lane in the wave.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int lane) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "butterfly stage");
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    // lane ^ 7 within each half-row, then ^ 3 within each quad
    const uint32_t t = __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false);
    return __builtin_amdgcn_update_dpp(0u, t, 0x1B, 0xF, 0xF, false);
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (M == 16) {
    // rows 0,2 receive rows 1,3 in the second result, rows 1,3 rows 0,2 in the first
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    // lanes 0-31 receive lanes 32-63 in the second result, lanes 32-63 lanes 0-31 in the first
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}
template <int M>
__device__ __forceinline__ float lane_xor_f(float v, int lane) {
  return __uint_as_float(lane_xor<M>(__float_as_uint(v), lane));
}
template <int M>
__device__ __forceinline__ double lane_xor_d(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = lane_xor<M>((uint32_t)b, lane), hi = lane_xor<M>((uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(lo | (hi << 32)));
}
// Lane (lane ^ m) for a wave-uniform m that the caller's unrolled loop makes a constant.
__device__ __forceinline__ uint32_t lane_xor_rt(uint32_t v, int m, int lane) {
  switch (m) {
    case 1: return lane_xor<1>(v, lane);
    case 2: return lane_xor<2>(v, lane);
    case 4: return lane_xor<4>(v, lane);
    case 8: return lane_xor<8>(v, lane);
    case 16: return lane_xor<16>(v, lane);
    default: return lane_xor<32>(v, lane);
  }
}

// Sum over aligned groups of `G` lanes (G a power of two <= 64); every lane of a
// group ends with the group's total. The reduction tree is fixed, so results are
// identical from run to run.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  const int lane = (int)(threadIdx.x & (kWave - 1));
  if (G > 1) v += lane_xor_f<1>(v, lane);
  if (G > 2) v += lane_xor_f<2>(v, lane);
  if (G > 4) v += lane_xor_f<4>(v, lane);
  if (G > 8) v += lane_xor_f<8>(v, lane);
  if (G > 16) v += lane_xor_f<16>(v, lane);
  if (G > 32) v += lane_xor_f<32>(v, lane);
  return v;
}
__device__ __forceinline__ float group_sum_rt(float v, int G) {
  const int lane = (int)(threadIdx.x & (kWave - 1));
  if (G > 1) v += lane_xor_f<1>(v, lane);
  if (G > 2) v += lane_xor_f<2>(v, lane);
  if (G > 4) v += lane_xor_f<4>(v, lane);
  if (G > 8) v += lane_xor_f<8>(v, lane);
  if (G > 16) v += lane_xor_f<16>(v, lane);
  if (G > 32) v += lane_xor_f<32>(v, lane);
  return v;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Largest power of two (<= 64) dividing nb: lanes that share one row.
__host__ __device__ inline int lanes_per_row(int nb) {
  int l = 1;
  while (l < 64 && (nb % (2 * l)) == 0) l *= 2;
  return l;
}

}  // namespace k3moe
