// Per-token softmax top-k selection, shared by the router kernel and the
// decode front-end kernel (one wave per token; see router.hip for the
// operation and the grouped variant).
#pragma once

#include <float.h>

#include "device_common.hpp"

namespace moe {

constexpr int kNoIndex = 0x7FFFFFFF;

// (value, index) order of the selection: the larger value, ties to the
// lower index; index kNoIndex holds no candidate.  A strict total order on
// non-NaN values (-0 and +0 compare equal), so any reduction order picks
// the same winner.
__device__ __forceinline__ void take_better(float& bv, int& bi, float ov, int oi) {
  if (oi != kNoIndex && (bi == kNoIndex || ov > bv || (ov == bv && oi < bi))) {
    bv = ov;
    bi = oi;
  }
}

// Arg-max over the wave, the result in every lane: four DPP steps reduce
// each row of 16 lanes, then the four row winners are read out in row order.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  take_better(bv, bi, dpp_float<kDppXor1>(bv), dpp_int<kDppXor1>(bi));
  take_better(bv, bi, dpp_float<kDppXor2>(bv), dpp_int<kDppXor2>(bi));
  take_better(bv, bi, dpp_float<kDppHalfMirror>(bv), dpp_int<kDppHalfMirror>(bi));
  take_better(bv, bi, dpp_float<kDppMirror>(bv), dpp_int<kDppMirror>(bi));
  float v = read_lane(bv, 0);
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) take_better(v, i, read_lane(bv, r), __builtin_amdgcn_readlane(bi, r));
  bv = v;
  bi = i;
}

// Sum over the wave, the same bits in every lane: pairwise within each row
// of 16 lanes (both lanes of a pair add the same two values), then the row
// sums in row order.
__device__ __forceinline__ float wave_sum(float z) {
  z += dpp_float<kDppXor1>(z);
  z += dpp_float<kDppXor2>(z);
  z += dpp_float<kDppHalfMirror>(z);
  z += dpp_float<kDppMirror>(z);
  return ((read_lane(z, 0) + read_lane(z, 16)) + read_lane(z, 32)) + read_lane(z, 48);
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
      int bi = lane < num_group && !taken ? lane : kNoIndex;
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
    int bi = kNoIndex;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((used >> i) & 1u)) take_better(bv, bi, v[i], e);
    }
    wave_argmax(bv, bi);
    if (j == 0) top_v = bv;
    if (lane == j) { my_id = bi; my_v = bv; }
    if ((bi & 63) == lane) used |= 1u << (bi >> 6);
  }
  float denom;
  if (renormalize) {
    denom = wave_sum(lane < top_k ? expf(my_v - top_v) : 0.0f);
  } else {
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) z += expf(v[i] - top_v);
    denom = wave_sum(z);
  }
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    weights[(size_t)t * top_k + lane] = expf(my_v - top_v) / denom;
    if (ids_lds) ids_lds[t * top_k + lane] = my_id;
  }
}

}  // namespace moe
