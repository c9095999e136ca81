// Matrix-core rate probe: a measurement aid beside the layer's kernels.
//
// Each wave runs `iters` rounds of eight independent MFMA chains of one of
// the two instruction types the GEMMs use, with operands held in registers:
//   kind 0: v_mfma_f32_16x16x32_f16 (the first GEMM's exact-f16 products),
//           16384 flops per instruction;
//   kind 1: v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 operands, unit scales
//           (the second GEMM's FP8 products), 65536 flops per instruction.
// No memory is touched until the end, when every lane stores the sum of its
// accumulators to sink[global thread id] (so the chains stay live).  Timing a
// launch gives the achieved dense MFMA rate of the part, against which the
// GEMMs' roofline fractions can be read.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  v4f acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  if (KIND == 0) {
    v8h a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(0.0078125f * (float)((threadIdx.x + i) & 7));
      b[i] = (_Float16)(0.0078125f * (float)((threadIdx.x * 3 + i) & 7));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
  } else {
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x30303030 + ((threadIdx.x + i) & 7);       // e4m3 values near 0.5
      b[i] = 0x28282828 + ((threadIdx.x * 3 + i) & 7);   // near 0.25
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[tid] = s;
}

hipError_t launch_mfma_probe(int kind, int iters, int nblocks, float* sink, hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3((unsigned)nblocks), dim3(256), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3((unsigned)nblocks), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
