// Per-token, per-128-group dynamic FP8 (e4m3fn) activation quantisation.
//
// Operation (fp8 oracle API page, activation quant key kFp8Dynamic128Sym;
// overview page, "Weight Scale Granularities", GROUP = one scale per 128
// consecutive elements): for each row and group of 128 columns,
//   s = max(amax, 1e-8) / 448,  q = e4m3fn_RNE_saturate(x / s).
//
// The row-major [M, K] input with K a multiple of 128 is a flat sequence of
// M*K/128 groups of 128 bf16 (256 bytes).  Sixteen lanes own one group, each
// lane 8 consecutive values (one 16-byte load), so a wave covers four groups
// (1 KiB of contiguous input) per step and every access is a full, aligned
// vector load or store.  The group amax is a 16-lane butterfly; the scale and
// its reciprocal are computed once per lane, and every element costs one
// multiply and two FMAs for the correctly rounded quotient.  HBM bound: 2
// bytes in, 1 byte + 4/128 bytes out per element.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

template <int SLOTS>
__global__ __launch_bounds__(256) void group_quant_bf16_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, float* __restrict__ scales,
    long long nslots) {
  // slot = one lane's 8 elements; 16 slots per group
  const long long base = ((long long)blockIdx.x * 256 * SLOTS) + threadIdx.x;
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
    amax = wave_max_xor(amax, 8, 1);   // the 16 lanes of this group
    float s, r;
    group_scale(amax, s, r);
    uint2 out;
    out.x = pack4_e4m3(clamp_fp8(div_by_scale(f[0], s, r)), clamp_fp8(div_by_scale(f[1], s, r)),
                       clamp_fp8(div_by_scale(f[2], s, r)), clamp_fp8(div_by_scale(f[3], s, r)));
    out.y = pack4_e4m3(clamp_fp8(div_by_scale(f[4], s, r)), clamp_fp8(div_by_scale(f[5], s, r)),
                       clamp_fp8(div_by_scale(f[6], s, r)), clamp_fp8(div_by_scale(f[7], s, r)));
    if (slot < nslots) {
      q[slot] = out;
      if ((threadIdx.x & 15) == 0) scales[slot >> 4] = s;
    }
  }
}

hipError_t launch_group_quant(const void* x, long long M, int K, uint8_t* q, float* s,
                              hipStream_t stream) {
  const long long nslots = M * (long long)(K / 8);
  if (nslots == 0) return hipSuccess;
  constexpr int SLOTS = 2;
  const long long per_block = 256LL * SLOTS;
  const long long nblk = (nslots + per_block - 1) / per_block;
  hipLaunchKernelGGL(group_quant_bf16_kernel<SLOTS>, dim3((unsigned)nblk), dim3(256), 0, stream,
                     (const uint4*)x, (uint2*)q, s, nslots);
  return hipGetLastError();
}

}  // namespace moe
