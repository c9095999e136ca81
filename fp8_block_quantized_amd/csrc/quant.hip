// Per-token, per-group dynamic FP8 (e4m3fn) activation quantisation.
//
// Operation (fp8 oracle API page, activation quant key kFp8Dynamic128Sym;
// overview page, "Weight Scale Granularities", GROUP = one scale per 128
// consecutive elements): for each row and group of 128 columns,
//   s = max(amax, 1e-8) / 448,  q = e4m3fn_RNE_saturate(x / s).
// Power-of-two variants (overview page, "DeepGEMM Scale Formats": float32
// scales rounded up to UE8M0, or the UE8M0 exponent bytes themselves; fp8
// oracle API page, the MXFP8 [1, 32] activation quant with uint8 UE8M0
// scales): the same float32 s rounded up to the next power of two, for
// groups of 32 or 128.  A power-of-two scale makes x / s an exact scaling,
// and rounding up keeps |x / s| <= 448.
//
// The row-major [M, K] input with K a multiple of the group is a flat
// sequence of M*K/G groups of G bf16 values.  G/8 lanes own one group, each
// lane 8 consecutive values (one 16-byte load), so a wave covers 1 KiB of
// contiguous input per step and every access is a full, aligned vector load
// or store.  The group amax is a DPP reduction over its lanes (quad swaps,
// then the half-row and row mirrors); the scale and its
// reciprocal are computed once per lane, and every element costs one
// multiply and two FMAs for the correctly rounded quotient (one multiply for
// a power-of-two scale).  HBM bound: 2 bytes in, 1 byte + 4/G (or 1/G)
// bytes out per element.
#include "device_common.hpp"
#include "launch.hpp"
#include "quant_dev.hpp"

namespace moe {

// kMasked: the rows form E blocks of M rows (blockIdx.y = block e) of which
// only the first counts[e] are quantised (the batched expert format); the
// others are neither read nor written.
template <int G, int FMT, int SLOTS, bool kMasked = false>
__global__ __launch_bounds__(256) void group_quant_bf16_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, void* __restrict__ scales,
    long long nslots, const int32_t* __restrict__ counts = nullptr, int M = 0,
    int slots_per_row = 0) {
  constexpr int LPG = G / 8;   // lanes per group
  if (kMasked) {   // this block's expert: its rows start at e * M
    int c = counts[blockIdx.y];
    c = c < 0 ? 0 : (c > M ? M : c);
    const long long first = (long long)blockIdx.y * M * slots_per_row;
    x += first;
    q += first;
    scales = (uint8_t*)scales + first / LPG * (FMT == kScaleUe8m0 ? 1 : 4);
    nslots = (long long)c * slots_per_row;
  }
  quant_slots<G, FMT, SLOTS>(x, q, scales, nslots, (long long)blockIdx.x * 256 * SLOTS + threadIdx.x);
}

template <int G, int FMT>
static hipError_t launch_quant_t(const void* x, long long nslots, uint8_t* q, void* s,
                                 hipStream_t stream) {
  constexpr int SLOTS = 2;
  const long long per_block = 256LL * SLOTS;
  const long long nblk = (nslots + per_block - 1) / per_block;
  hipLaunchKernelGGL((group_quant_bf16_kernel<G, FMT, SLOTS>), dim3((unsigned)nblk), dim3(256), 0,
                     stream, (const uint4*)x, (uint2*)q, s, nslots);
  return hipGetLastError();
}

hipError_t launch_group_quant_fmt(const void* x, long long M, int K, int group, int fmt,
                                  uint8_t* q, void* s, hipStream_t stream) {
  const long long nslots = M * (long long)(K / 8);
  if (nslots == 0) return hipSuccess;
  if (group == 128) {
    if (fmt == kScaleFloat32) return launch_quant_t<128, kScaleFloat32>(x, nslots, q, s, stream);
    if (fmt == kScaleFloat32CeilUe8m0)
      return launch_quant_t<128, kScaleFloat32CeilUe8m0>(x, nslots, q, s, stream);
    return launch_quant_t<128, kScaleUe8m0>(x, nslots, q, s, stream);
  }
  if (fmt == kScaleFloat32) return launch_quant_t<32, kScaleFloat32>(x, nslots, q, s, stream);
  if (fmt == kScaleFloat32CeilUe8m0)
    return launch_quant_t<32, kScaleFloat32CeilUe8m0>(x, nslots, q, s, stream);
  return launch_quant_t<32, kScaleUe8m0>(x, nslots, q, s, stream);
}

hipError_t launch_group_quant(const void* x, long long M, int K, uint8_t* q, float* s,
                              hipStream_t stream) {
  return launch_group_quant_fmt(x, M, K, 128, kScaleFloat32, q, s, stream);
}

hipError_t launch_group_quant_masked(const void* x, const int32_t* counts, int E, int M, int K,
                                     uint8_t* q, float* s, hipStream_t stream) {
  constexpr int SLOTS = 2;
  const long long per = (long long)M * (K / 8);
  if (per == 0 || E == 0) return hipSuccess;
  const unsigned nbx = (unsigned)((per + 256LL * SLOTS - 1) / (256LL * SLOTS));
  hipLaunchKernelGGL((group_quant_bf16_kernel<128, kScaleFloat32, SLOTS, true>), dim3(nbx, E),
                     dim3(256), 0, stream, (const uint4*)x, (uint2*)q, (void*)s, per, counts, M,
                     K / 8);
  return hipGetLastError();
}

}  // namespace moe
