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
#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

template <int VPL>  // logits per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int renormalize,
    int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together
  const float* row = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -FLT_MAX;
  }
  uint32_t used = 0;
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
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
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
                               int32_t* ids, float* w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(topk_softmax_kernel<1>, grid, block, 0, stream, logits, T, E, top_k, renormalize, ids, w);
  else if (vpl <= 2)
    hipLaunchKernelGGL(topk_softmax_kernel<2>, grid, block, 0, stream, logits, T, E, top_k, renormalize, ids, w);
  else if (vpl <= 4)
    hipLaunchKernelGGL(topk_softmax_kernel<4>, grid, block, 0, stream, logits, T, E, top_k, renormalize, ids, w);
  else
    hipLaunchKernelGGL(topk_softmax_kernel<8>, grid, block, 0, stream, logits, T, E, top_k, renormalize, ids, w);
  return hipGetLastError();
}

}  // namespace moe
