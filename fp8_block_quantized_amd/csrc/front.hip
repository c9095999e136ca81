// Decode front end: the router, the sort-and-pad and the activation quant of
// a small batch in one launch.
//
// The three steps are those of router.hip, align.hip and quant.hip (overview
// page, "FusedMoE Class" and "Triton Fused MoE Kernel"; fp8 oracle API page,
// the group-128 dynamic activation quant), with the same arithmetic and so
// the same results.  At decode sizes each of them is a few microseconds of
// launch and drain around almost no work, and the quant does not depend on
// the routing, so:
//   - workgroup 0 (16 waves) routes the T tokens, wave w taking token w;
//     the ids also go to LDS, and after a barrier the same workgroup runs
//     the single-workgroup sort-and-pad on them;
//   - workgroups 1.. quantise x, each as four 256-thread groups of the
//     quant kernel.
// Limits: T <= 16 tokens (one per wave: the routing of a token is a chain of
// dependent wave operations, so more tokens per wave lengthen workgroup 0
// past the launches saved; measured, DeepSeek-shaped T = 64 took 48 us
// against 27 for the three separate kernels, Qwen3-shaped T = 1 48 against
// 52 for the whole forward), P = T * top_k <= 1024 pairs, E <= 512.
#include "align_dev.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "quant_dev.hpp"
#include "route_dev.hpp"

namespace moe {

struct FrontArgs {
  const float* logits;
  int T, E, top_k, renormalize, num_group, topk_group;
  const int32_t* emap;
  int n_map, EL, BM, ebits;
  const uint4* x;
  long long nslots;          // T * H / 8
  int32_t* ids;
  float* tw;
  int32_t *sorted_ids, *expert_ids, *ntpp, *eoff, *pair_pos;
  uint2* xq;
  float* xs;
};

constexpr int kFrontWaves = 16;
constexpr int kFrontSlots = 2;              // the quant kernel's slots per thread

template <int VPL>
__global__ __launch_bounds__(1024) void decode_front_kernel(FrontArgs a) {
  __shared__ float stage[kFrontWaves][kMaxE];
  __shared__ int32_t ids_lds[kChunk];
  __shared__ AlignSingleLds lds;
  if (blockIdx.x > 0) {
    const long long vb = (long long)(blockIdx.x - 1) * 4 + (threadIdx.x >> 8);
    quant_slots<128, kScaleFloat32, kFrontSlots>(a.x, a.xq, a.xs, a.nslots,
                                                 vb * 256 * kFrontSlots + (threadIdx.x & 255));
    return;
  }
  const int wave = threadIdx.x >> 6;
  route_token<VPL>(a.logits, wave, a.T, a.E, a.top_k, a.renormalize, a.num_group, a.topk_group,
                   stage[wave], a.ids, a.tw, ids_lds);
  __syncthreads();
  align_single(lds, ids_lds, a.emap, a.n_map, a.T * a.top_k, a.EL, a.BM, a.ebits, a.sorted_ids,
               a.expert_ids, a.ntpp, a.eoff, a.pair_pos);
}

bool decode_front_fits(int T, int E, int top_k) {
  return T >= 1 && T <= kFrontWaves && (long long)T * top_k <= kChunk && E <= kMaxE;
}

hipError_t launch_decode_front(const float* logits, int T, int E, int top_k, int renormalize,
                               int num_group, int topk_group, const int32_t* emap, int n_map,
                               int EL, int BM, const void* x, int H, int32_t* ids, float* tw,
                               int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                               int32_t* eoff, int32_t* pair_pos, uint8_t* xq, float* xs,
                               hipStream_t stream) {
  if (!decode_front_fits(T, E, top_k) || EL > kMaxE) return hipErrorInvalidValue;
  FrontArgs a;
  a.logits = logits; a.T = T; a.E = E; a.top_k = top_k; a.renormalize = renormalize;
  a.num_group = num_group; a.topk_group = topk_group;
  a.emap = emap; a.n_map = n_map; a.EL = EL; a.BM = BM;
  a.ebits = 0;
  while ((1 << a.ebits) < EL) ++a.ebits;
  a.x = (const uint4*)x; a.nslots = (long long)T * (H / 8);
  a.ids = ids; a.tw = tw;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.ntpp = ntpp; a.eoff = eoff;
  a.pair_pos = pair_pos;
  a.xq = (uint2*)xq; a.xs = xs;
  const long long per_block = 4LL * 256 * kFrontSlots;
  const dim3 grid((unsigned)(1 + (a.nslots + per_block - 1) / per_block)), block(kChunk);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) hipLaunchKernelGGL(decode_front_kernel<1>, grid, block, 0, stream, a);
  else if (vpl <= 2) hipLaunchKernelGGL(decode_front_kernel<2>, grid, block, 0, stream, a);
  else if (vpl <= 4) hipLaunchKernelGGL(decode_front_kernel<4>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(decode_front_kernel<8>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
