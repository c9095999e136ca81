// Rate probes: measurement aids beside the layer's kernels.
//
// Matrix-core rate probe.
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

// HBM read-stream probe.  The buffer is read as 16-byte words in chunks of
// 8 x 256 words (32 KB): a workgroup takes chunks in a grid-stride loop and
// each of its threads issues its eight loads of a chunk at once (eight
// independent 16-byte loads in flight, each instruction coalesced over the
// workgroup), then a ragged tail word by word.  Every thread XORs what it
// read and stores the XOR to sink[global thread id]: the XOR of all sink
// words is the XOR of all 32-bit words of src, so no load can be dropped.
// Over a buffer larger than the 256 MB last-level cache, a launch's time
// gives the rate at which HBM delivers a read-only stream (the bound of the
// weight-streaming decode GEMMs, which write almost nothing).
__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  constexpr int kLoads = 8;
  const size_t chunk = (size_t)kLoads * 256, nchunk = n16 / chunk;
  uint32_t x = 0;
  for (size_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
    const v4u* p = (const v4u*)src + c * chunk + threadIdx.x;
    v4u v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) v[i] = __builtin_nontemporal_load(p + i * 256);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  for (size_t i = nchunk * chunk + (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

hipError_t launch_hbm_read_probe(const void* src, size_t bytes, int nblocks, uint32_t* sink,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream,
                     (const uint4*)src, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
