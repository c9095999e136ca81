// Device helpers shared by the HIP kernels of the FP8 MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 128;          // activation group and weight block edge
constexpr float kFp8Max = 448.0f;    // largest finite e4m3fn magnitude
constexpr float kAmaxEps = 1e-8f;    // lower clamp of a group amax

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Correctly rounded float32 quotient x / s (s > 0) given r = RN(1 / s), from
// one product and two fused multiply-adds (Markstein's correction step: with
// r the correctly rounded reciprocal and q0 within an ulp of x / s, the
// remainder x - q0*s is exact and q0 + rem*r rounds to RN(x / s)).  The
// correction of an exact zero gives +0 whatever the sign of x, so the sign
// is taken from x, as in the IEEE quotient.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  float q0 = x * r;
  float rem = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(rem, r, q0), x);
}

__device__ __forceinline__ float clamp_fp8(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -kFp8Max), kFp8Max);
}

// Four float32 values (already within +-448) -> four e4m3fn codes, RNE, the
// first value in the lowest byte.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Scale of a group from its amax: max(amax, 1e-8) / 448 with an IEEE
// (correctly rounded) float32 division, and its correctly rounded reciprocal.
__device__ __forceinline__ void group_scale(float amax, float& s, float& r) {
  s = __builtin_fmaxf(amax, kAmaxEps) / kFp8Max;
  r = 1.0f / s;
}

// float32 s > 0 (normal) -> the smallest power of two >= s, as its bits.
__device__ __forceinline__ uint32_t ceil_pow2_bits(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x7FFFFFu) ? (b & 0x7F800000u) + 0x00800000u : b;
}

// Four e4m3fn codes (one dword) -> four f16 values, exactly (every e4m3fn
// value is an f16 value; the hardware conversion scales by 1.0).
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, _Float16* out) {
  const v2h lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const v2h hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

__device__ __forceinline__ float wave_max_xor(float v, int first_mask, int last_mask) {
  for (int m = first_mask; m >= last_mask; m >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Lane exchanges inside rows of 16 lanes by DPP (register reads, no LDS
// round trip as a shuffle takes): the gfx9 data-parallel-primitive controls
// for lane ^ 1 and lane ^ 2 (quad permutations), and the mirrors of each
// half row (lane i <-> 7 - i) and of each row (lane i <-> 15 - i).  After the
// two quad steps a quad holds one value, so the half-row mirror then pairs
// whole quads and the row mirror whole half rows: the four steps reduce a
// row as a butterfly over 16 lanes would.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ int dpp_int(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_float(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Maximum over aligned groups of LPG lanes (2, 4, 8 or 16), in every lane
// of the group; max is exact, so the order of the steps does not matter.
template <int LPG>
__device__ __forceinline__ float group_max(float v) {
  static_assert(LPG == 2 || LPG == 4 || LPG == 8 || LPG == 16, "lanes per group");
  v = __builtin_fmaxf(v, dpp_float<kDppXor1>(v));
  if (LPG >= 4) v = __builtin_fmaxf(v, dpp_float<kDppXor2>(v));
  if (LPG >= 8) v = __builtin_fmaxf(v, dpp_float<kDppHalfMirror>(v));
  if (LPG >= 16) v = __builtin_fmaxf(v, dpp_float<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Hardware dispatches consecutive workgroup ids round-robin over the eight
// XCDs.  Renumber them so that each XCD receives a contiguous range of
// logical ids: tiles that share a weight panel then run on one XCD and meet
// in its L2.  A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_contiguous_id(int bid, int n) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int q = n >> 3, rem = n & 7;
  return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace moe
