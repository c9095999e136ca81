// Per-token softmax top-k selection, shared by the router kernel and the
// decode front-end kernel (one wave per token; see router.hip for the
// operation and the grouped variant).
#pragma once

#include <float.h>

#include "device_common.hpp"

namespace moe {

// Butterfly arg-max over the wave of (value, index), ties to the lower index;
// lanes with index 0x7FFFFFFF hold no candidate.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oi = __shfl_xor(bi, m);
    if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi))) {
      bv = ov;
      bi = oi;
    }
  }
}

// Token t of T (the calling wave's; t >= T: nothing is written).  srow: this
// wave's LDS row of at least E floats (the grouped variant stages its logits
// there; only this wave touches it).  ids_lds (optional): the ids also go to
// LDS at the same [t * top_k + j] positions.
template <int VPL>  // logits per lane: ceil(E / 64)
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int T, int E,
                                            int top_k, int renormalize, int num_group,
                                            int topk_group, float* srow, int32_t* __restrict__ ids,
                                            float* __restrict__ weights, int32_t* ids_lds) {
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -FLT_MAX;
  }
  // slots outside the kept groups start out as used
  uint32_t used = 0;
  if (num_group > 1) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) srow[lane + 64 * i] = v[i];
    // the row is this wave's alone: its LDS writes land before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int gs = E / num_group;
    float gm = -FLT_MAX;
    if (lane < num_group)
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) gm = __builtin_fmaxf(gm, srow[e]);
    unsigned long long keep = 0;
    bool taken = false;
    for (int r = 0; r < topk_group; ++r) {
      float bv = gm;
      int bi = lane < num_group && !taken ? lane : 0x7FFFFFFF;
      wave_argmax(bv, bi);
      keep |= 1ull << bi;
      if (lane == bi) taken = true;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((keep >> (e / gs)) & 1ull)) used |= 1u << i;
    }
  }
  int my_id = 0;
  float my_v = 0.0f, top_v = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      const bool ok = e < E && !((used >> i) & 1u);
      if (ok && (bi == 0x7FFFFFFF || v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if (j == 0) top_v = bv;
    if (lane == j) { my_id = bi; my_v = bv; }
    if ((bi & 63) == lane) used |= 1u << (bi >> 6);
  }
  float denom;
  if (renormalize) {
    float z = lane < top_k ? expf(my_v - top_v) : 0.0f;
    for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m);
    denom = z;
  } else {
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) z += expf(v[i] - top_v);
    for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m);
    denom = z;
  }
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    weights[(size_t)t * top_k + lane] = expf(my_v - top_v) / denom;
    if (ids_lds) ids_lds[t * top_k + lane] = my_id;
  }
}

}  // namespace moe
