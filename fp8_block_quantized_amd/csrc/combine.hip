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

// Small batches: the kernels above give each thread one token's 8 outputs
// and walk the top_k slots in turn, a chain of top_k dependent load
// latencies per thread with few threads in flight.  Here a workgroup takes
// one token and G = 256 / KP groups of 8 outputs (KP = top_k rounded up to a
// power of two): thread (slot j, group c) loads slot j's row piece (every
// K slice of it at once), sums the slices in order, and leaves the 8 values
// in LDS; then the G threads of slot 0 form the weighted sum over the slots
// in order, with the same float32 operations as combine_kernel /
// combine_slices_kernel, so the outputs are the same bits.
template <bool kSlices>
__global__ __launch_bounds__(256) void combine_slotpar_kernel(
    const void* __restrict__ src, int ys, int nslice, int P, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ topk_w, int H8, int top_k, int kp_log2, uint4* __restrict__ out) {
  __shared__ float4 yv_lds[256][2];
  const int G = 256 >> kp_log2;
  const int j = threadIdx.x / G, cg = threadIdx.x - j * G;
  const int per_tok = (H8 + G - 1) / G;
  const int t = blockIdx.x / per_tok;
  const int c = (blockIdx.x - t * per_tok) * G + cg;       // group of 8 outputs
  float yv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < H8 && j < top_k) {
    const long long p = (long long)t * top_k + j;
    const int row = pair_pos[p];
    if (row >= 0) {
      if (kSlices) {
        const float* part = (const float*)src;
        float4 u[kMaxSlices], v[kMaxSlices];
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s) {
          if (s < nslice) {
            const float4* q = (const float4*)(part + ((size_t)s * P + p) * ys + (size_t)c * 8);
            u[s] = q[0];
            v[s] = q[1];
          }
        }
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s) {
          if (s < nslice) {
            yv[0] += u[s].x; yv[1] += u[s].y; yv[2] += u[s].z; yv[3] += u[s].w;
            yv[4] += v[s].x; yv[5] += v[s].y; yv[6] += v[s].z; yv[7] += v[s].w;
          }
        }
      } else {
        const uint4 q = *(const uint4*)((const uint16_t*)src + (size_t)row * ys + (size_t)c * 8);
        yv[0] = bf16_lo(q.x); yv[1] = bf16_hi(q.x); yv[2] = bf16_lo(q.y); yv[3] = bf16_hi(q.y);
        yv[4] = bf16_lo(q.z); yv[5] = bf16_hi(q.z); yv[6] = bf16_lo(q.w); yv[7] = bf16_hi(q.w);
      }
    }
  }
  yv_lds[threadIdx.x][0] = make_float4(yv[0], yv[1], yv[2], yv[3]);
  yv_lds[threadIdx.x][1] = make_float4(yv[4], yv[5], yv[6], yv[7]);
  __syncthreads();
  if (j != 0 || c >= H8) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int jj = 0; jj < top_k; ++jj) {
    const long long p = (long long)t * top_k + jj;
    if (pair_pos[p] < 0) continue;
    const float w = topk_w ? topk_w[p] : 1.0f;
    const float4 a = yv_lds[jj * G + cg][0], b = yv_lds[jj * G + cg][1];
    acc[0] = __builtin_fmaf(w, a.x, acc[0]); acc[1] = __builtin_fmaf(w, a.y, acc[1]);
    acc[2] = __builtin_fmaf(w, a.z, acc[2]); acc[3] = __builtin_fmaf(w, a.w, acc[3]);
    acc[4] = __builtin_fmaf(w, b.x, acc[4]); acc[5] = __builtin_fmaf(w, b.y, acc[5]);
    acc[6] = __builtin_fmaf(w, b.z, acc[6]); acc[7] = __builtin_fmaf(w, b.w, acc[7]);
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  out[(size_t)t * H8 + c] = o;
}

// the slot-parallel form pays off while the one-thread-per-8-outputs grid is
// small: at most this many threads
constexpr long long kSlotParMaxThreads = 256LL * 256;

static bool use_slotpar(int T, int H, int top_k) {
  return (long long)T * (H / 8) <= kSlotParMaxThreads && top_k <= 32;
}

static int log2_ceil(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <bool kSlices>
static hipError_t launch_slotpar(const void* src, int ys, int nslice, int P, const int32_t* pair_pos,
                                 const float* topk_w, int T, int H, int top_k, uint16_t* out,
                                 hipStream_t stream) {
  const int kp = log2_ceil(top_k), G = 256 >> kp, H8 = H / 8;
  const long long blocks = (long long)T * ((H8 + G - 1) / G);
  hipLaunchKernelGGL(combine_slotpar_kernel<kSlices>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     src, ys, nslice, P, pair_pos, topk_w, H8, top_k, kp, (uint4*)out);
  return hipGetLastError();
}

hipError_t launch_combine_slices(const float* part, int y_stride, int nslice, int P,
                                 const int32_t* pair_pos, const float* topk_w, int T, int H,
                                 int top_k, uint16_t* out, hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  if (n == 0) return hipSuccess;
  if (nslice < 1 || nslice > kMaxSlices) return hipErrorInvalidValue;
  if (use_slotpar(T, H, top_k))
    return launch_slotpar<true>(part, y_stride, nslice, P, pair_pos, topk_w, T, H, top_k, out, stream);
  hipLaunchKernelGGL(combine_slices_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     part, y_stride, nslice, P, pair_pos, topk_w, T, H / 8, top_k, (uint4*)out);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y, int y_stride, const int32_t* pair_pos,
                          const float* topk_w, int T, int H, int top_k, uint16_t* out,
                          hipStream_t stream) {
  const long long n = (long long)T * (H / 8);
  if (n == 0) return hipSuccess;
  if (use_slotpar(T, H, top_k))
    return launch_slotpar<false>(y, y_stride, 1, T * top_k, pair_pos, topk_w, T, H, top_k, out,
                                 stream);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, y,
                     y_stride, pair_pos, topk_w, T, H / 8, top_k, (uint4*)out);
  return hipGetLastError();
}

}  // namespace moe
