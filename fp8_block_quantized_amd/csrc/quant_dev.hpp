// The group quantiser's per-lane work, shared by the quant kernels and the
// decode front-end kernel; the operation is described in quant.hip.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

// Slots base, base + 256, ... (SLOTS of them) of the flat sequence of 16-byte
// input slots (8 bf16 each); the G / 8 lanes of a group are consecutive lanes
// of one wave, so base must be (a multiple of 256 * SLOTS) + the lane's index
// in a 256-thread group.
template <int G, int FMT, int SLOTS>
__device__ __forceinline__ void quant_slots(const uint4* __restrict__ x, uint2* __restrict__ q,
                                            void* __restrict__ scales, long long nslots,
                                            long long base) {
  constexpr int LPG = G / 8;   // lanes per group
  uint4 v[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    long long slot = base + (long long)u * 256;
    v[u] = slot < nslots ? x[slot] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    long long slot = base + (long long)u * 256;
    float f[8];
    f[0] = bf16_lo(v[u].x); f[1] = bf16_hi(v[u].x);
    f[2] = bf16_lo(v[u].y); f[3] = bf16_hi(v[u].y);
    f[4] = bf16_lo(v[u].z); f[5] = bf16_hi(v[u].z);
    f[6] = bf16_lo(v[u].w); f[7] = bf16_hi(v[u].w);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
    amax = group_max<LPG>(amax);             // the lanes of this group
    float s, r;
    group_scale(amax, s, r);
    float d[8];
    if (FMT == kScaleFloat32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = clamp_fp8(div_by_scale(f[i], s, r));
    } else {
      const uint32_t sb = ceil_pow2_bits(s);
      s = __uint_as_float(sb);
      r = __uint_as_float((254u - (sb >> 23)) << 23);   // exactly 1 / s
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = clamp_fp8(f[i] * r);
    }
    uint2 out;
    out.x = pack4_e4m3(d[0], d[1], d[2], d[3]);
    out.y = pack4_e4m3(d[4], d[5], d[6], d[7]);
    if (slot < nslots) {
      q[slot] = out;
      if ((threadIdx.x & (LPG - 1)) == 0) {
        if (FMT == kScaleUe8m0)
          ((uint8_t*)scales)[slot / LPG] = (uint8_t)(__float_as_uint(s) >> 23);
        else
          ((float*)scales)[slot / LPG] = s;
      }
    }
  }
}

}  // namespace moe
