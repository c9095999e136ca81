// Weighted combine of the per-pair expert outputs.
//
// Operation (overview page, "Modular Kernel Architecture": the finalize step
// gathers the expert results back to token order; "Triton Fused MoE Kernel":
// the router weight multiplies the dequantised GEMM output):
//   out[t, :] = bf16( sum over slots j in order of w[t, j] * y[row(t*k + j), :] )
// accumulated in float32 with one fused multiply-add per term, where row(p)
// is the sorted row that the second GEMM wrote pair p to; a pair left out of
// the layout (its expert held elsewhere, row -1) contributes zero, the
// expert map's zero output.  Each thread
// produces 8 outputs: k gathered 16-byte reads (consecutive threads read
// consecutive bytes of one row) and one 16-byte write.  HBM bound.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y, int ys,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int H8, int top_k, uint4* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * H8) return;
  const long long t = idx / H8, c = idx - t * H8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int jj = 0; jj < top_k; ++jj) {
    const long long p = t * top_k + jj;
    const int row = pair_pos[p];
    if (row < 0) continue;
    const float w = topk_w ? topk_w[p] : 1.0f;     // no weights: copy (1 * y is exact)
    const uint4 v = *(const uint4*)(y + (size_t)row * ys + c * 8);
    acc[0] = __builtin_fmaf(w, bf16_lo(v.x), acc[0]); acc[1] = __builtin_fmaf(w, bf16_hi(v.x), acc[1]);
    acc[2] = __builtin_fmaf(w, bf16_lo(v.y), acc[2]); acc[3] = __builtin_fmaf(w, bf16_hi(v.y), acc[3]);
    acc[4] = __builtin_fmaf(w, bf16_lo(v.z), acc[4]); acc[5] = __builtin_fmaf(w, bf16_hi(v.z), acc[5]);
    acc[6] = __builtin_fmaf(w, bf16_lo(v.w), acc[6]); acc[7] = __builtin_fmaf(w, bf16_hi(v.w), acc[7]);
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  out[idx] = o;
}

// The same combine over float32 K-slice partials of the second GEMM, stored
// by pair: y(p) = sum over slices s in order of part[s][p][:], then the
// weighted sum over the slots as above.  Each thread produces 8 outputs from
// two 16-byte reads per slice and slot.
constexpr int kMaxSlices = 8;

__global__ __launch_bounds__(256) void combine_slices_kernel(const float* __restrict__ part, int ys,
                                                             int nslice, int P,
                                                             const int32_t* __restrict__ pair_pos,
                                                             const float* __restrict__ topk_w, int T,
                                                             int H8, int top_k, uint4* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)T * H8) return;
  const long long t = idx / H8, c = idx - t * H8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int jj = 0; jj < top_k; ++jj) {
    const long long p = t * top_k + jj;
    if (pair_pos[p] < 0) continue;
    const float w = topk_w[p];
    // every slice's loads of this slot in flight together (nslice <= kMaxSlices)
    float4 u[kMaxSlices], v[kMaxSlices];
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s) {
      if (s < nslice) {
        const float4* src = (const float4*)(part + ((size_t)s * P + p) * ys + c * 8);
        u[s] = src[0];
        v[s] = src[1];
      }
    }
    float yv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSlices; ++s) {
      if (s < nslice) {
        yv[0] += u[s].x; yv[1] += u[s].y; yv[2] += u[s].z; yv[3] += u[s].w;
        yv[4] += v[s].x; yv[5] += v[s].y; yv[6] += v[s].z; yv[7] += v[s].w;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w, yv[i], acc[i]);
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  out[idx] = o;
}

hipError_t launch_combine_slices(const float* part, int y_stride, int nslice, int P,
                                 const int32_t* pair_pos, const float* topk_w, int T, int H,
                                 int top_k, uint16_t* out, hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  if (n == 0) return hipSuccess;
  if (nslice < 1 || nslice > kMaxSlices) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_slices_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     part, y_stride, nslice, P, pair_pos, topk_w, T, H / 8, top_k, (uint4*)out);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, int y_stride, const int32_t* pair_pos,
                          const float* topk_w, int T, int H, int top_k, uint16_t* out,
                          hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, y,
                     y_stride, pair_pos, topk_w, T, H / 8, top_k, (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
