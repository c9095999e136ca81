// Weighted combine of the per-pair expert outputs.
//
// Operation (overview page, "Modular Kernel Architecture": the finalize step
// gathers the expert results; "Triton Fused MoE Kernel": the router weight is
// applied to the dequantised GEMM output, which the second GEMM's epilogue
// already did): out[t, :] = bf16( sum over slots j in order of y[t*k + j, :] ),
// summed in float32.  The k rows of a token are contiguous in pair order, so
// each thread reads k 16-byte vectors and writes one.  HBM bound.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y, int T, int H8,
                                                      int top_k, uint4* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * H8) return;
  const long long t = idx / H8, c = idx - t * H8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint4* src = y + (t * top_k) * H8 + c;
  for (int jj = 0; jj < top_k; ++jj) {
    const uint4 v = src[(long long)jj * H8];
    acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
    acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
    acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
    acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  out[idx] = o;
}

hipError_t launch_combine(const uint16_t* y, int T, int H, int top_k, uint16_t* out,
                          hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const uint4*)y, T, H / 8, top_k, (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
