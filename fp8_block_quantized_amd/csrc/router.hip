// Softmax top-k router: one wave per token.
//
// Operation (overview page, "FusedMoE Class": the top-K router in front of
// the experts): softmax over the E logits of a token, the top_k experts in
// descending order, weights optionally renormalised over the chosen slots.
// Selection compares the float32 logits themselves (softmax is monotone),
// ties going to the lower expert index, so the chosen ids are an exact
// integer result.  Each lane holds the logits of experts lane, lane+64, ...;
// a selection round is a lane-local scan and a 6-step butterfly over
// (value, index).  With renormalisation the full-softmax denominator cancels
// and only the chosen logits enter the weights.
//
// Grouped variant (num_group > 1; the overview page's environment table
// names a fused grouped top-K routing switch without defining it, and the
// reading taken is the plainest one): experts form num_group equal groups of
// consecutive ids, a group's score is its best logit, the topk_group best
// groups are kept (ties to the lower group), and the selection above runs on
// the kept groups' experts only; the weights are unchanged (full softmax,
// optional renormalisation).  The wave stages its logits in LDS, lanes below
// num_group scan their group for its best logit, and topk_group butterfly
// rounds pick the groups.
#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRouterMaxE = 512;

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

template <int VPL>  // logits per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int renormalize, int num_group,
    int topk_group, int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ float stage[4][kRouterMaxE];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool active = t < T;   // no early exit: the grouped path has a barrier
  const float* row = logits + (size_t)(active ? t : 0) * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -FLT_MAX;
  }
  // slots outside the kept groups start out as used
  uint32_t used = 0;
  if (num_group > 1) {
    float* srow = stage[threadIdx.x >> 6];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) srow[lane + 64 * i] = v[i];
    __syncthreads();
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
  if (!active) return;
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
  }
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int top_k, int renormalize,
                               int num_group, int topk_group, int32_t* ids, float* w,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + 63) / 64;
#define MOE_ROUTER_LAUNCH(V)                                                                      \
  hipLaunchKernelGGL(topk_softmax_kernel<V>, grid, block, 0, stream, logits, T, E, top_k,         \
                     renormalize, num_group, topk_group, ids, w)
  if (vpl <= 1) MOE_ROUTER_LAUNCH(1);
  else if (vpl <= 2) MOE_ROUTER_LAUNCH(2);
  else if (vpl <= 4) MOE_ROUTER_LAUNCH(4);
  else MOE_ROUTER_LAUNCH(8);
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
