// Softmax top-k router: one wave per token.
//
// Operation (overview page, "FusedMoE Class": the top-K router in front of
// the experts): softmax over the E logits of a token, the top_k experts in
// descending order, weights optionally renormalised over the chosen slots.
// Selection compares the float32 logits themselves (softmax is monotone),
// ties going to the lower expert index, so the chosen ids are an exact
// integer result.  Each lane holds the logits of experts lane, lane+64, ...;
// a selection round is a lane-local scan and a wave arg-max over (value,
// index): four DPP steps within each row of 16 lanes, then the four row
// winners read out in order.  With renormalisation the full-softmax denominator cancels
// and only the chosen logits enter the weights.
//
// Grouped variant (num_group > 1; the overview page's environment table
// names a fused grouped top-K routing switch without defining it, and the
// reading taken is the plainest one): experts form num_group equal groups of
// consecutive ids, a group's score is its best logit, the topk_group best
// groups are kept (ties to the lower group), and the selection above runs on
// the kept groups' experts only; the weights are unchanged (full softmax,
// optional renormalisation).  The wave stages its logits in LDS, lanes below
// num_group scan their group for its best logit, and topk_group arg-max
// rounds pick the groups.
#include "device_common.hpp"
#include "launch.hpp"
#include "route_dev.hpp"

namespace moe {

constexpr int kRouterMaxE = 512;

template <int VPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int renormalize, int num_group,
    int topk_group, int32_t* __restrict__ ids, float* __restrict__ weights) {
  __shared__ float stage[4][kRouterMaxE];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  route_token<VPL>(logits, t, T, E, top_k, renormalize, num_group, topk_group,
                   stage[threadIdx.x >> 6], ids, weights, nullptr);
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
