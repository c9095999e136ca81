// Kernel launchers of the FP8 MoE library (internal; enqueue only, no checks).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Scale formats of the group quantiser (values of the public format enum).
enum { kScaleFloat32 = 0, kScaleFloat32CeilUe8m0 = 1, kScaleUe8m0 = 2 };
hipError_t launch_group_quant(const void* x, long long M, int K, uint8_t* q, float* s,
                              hipStream_t stream);
// group 32 or 128, fmt one of the kScale* values; s is float32 or uint8 per group
hipError_t launch_group_quant_fmt(const void* x, long long M, int K, int group, int fmt,
                                  uint8_t* q, void* s, hipStream_t stream);
// num_group > 1: grouped top-k (topk_group of num_group equal expert groups)
hipError_t launch_topk_softmax(const float* logits, int T, int E, int top_k, int renormalize,
                               int num_group, int topk_group, int32_t* ids, float* w,
                               hipStream_t stream);
size_t align_scratch_bytes(int P, int E);
const int32_t* align_expert_offsets(const void* scratch, int P, int E);
// emap (optional, n_map entries): global expert -> local index or -1; pairs whose
// expert falls outside [0, E) are left out and get pair_pos -1
hipError_t launch_align(const int32_t* ids, const int32_t* emap, int n_map, int P, int E, int BM,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* pair_pos,
                        void* scratch, hipStream_t stream);
// The router, the single-workgroup sort-and-pad and the group-128 quant of a
// decode batch in one launch (decode_front_fits: T <= 16, T * top_k <= 1024,
// E <= 512), with the same outputs as launch_topk_softmax + launch_align +
// launch_group_quant.
bool decode_front_fits(int T, int E, int top_k);
hipError_t launch_decode_front(const float* logits, int T, int E, int top_k, int renormalize,
                               int num_group, int topk_group, const int32_t* emap, int n_map,
                               int EL, int BM, const void* x, int H, int32_t* ids, float* tw,
                               int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                               int32_t* eoff, int32_t* pair_pos, uint8_t* xq, float* xs,
                               hipStream_t stream);
hipError_t launch_identity_layout(int M, int BM, int nblk, int32_t* sorted_ids,
                                  int32_t* expert_ids, int32_t* eoff, int32_t* ntpp,
                                  hipStream_t stream);
// kslices > 1 (block_m <= 64, at most H/128 slices): the workgroups of a tile
// split K and store float64 partials of h by pair, h_slices [kslices, P, 2I];
// a second kernel sums them and writes aq / as at each pair's sorted row
// (pair_pos; padding rows of aq are then left unwritten, and nothing reads
// their results)
hipError_t launch_gemm1(const uint8_t* xq, const float* xs, const uint8_t* w13, const float* w13s,
                        const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntpp,
                        const int32_t* eoff, int E, int H, int I, int P, int top_k, int BM, int nblk,
                        uint8_t* aq, float* as, int kslices, double* h_slices,
                        const int32_t* pair_pos, hipStream_t stream);
// kslices > 1 (block_m <= 64, at most I/128 slices): the workgroups of a tile
// split K and store float32 partials by pair, y_slices [kslices, P, y_stride],
// for launch_combine_slices; otherwise bf16 y by sorted row
hipError_t launch_gemm2(const uint8_t* aq, const float* as, const uint8_t* w2, const float* w2s,
                        const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntpp,
                        const int32_t* eoff, int E, int H, int I, int P, int BM, int nblk,
                        uint16_t* y, int y_stride, uint16_t* y_dump, int kslices, float* y_slices,
                        hipStream_t stream);
// The MXFP8 layer's GEMMs (block_m 16 to 128): exponent bytes [rows, K/32]
// for the activations, [E, N, K/32] for the weights; GEMM1 writes the
// requantised activation's exponent bytes [cap, I/32] into ae
hipError_t launch_gemm1_mx(const uint8_t* xq, const uint8_t* xe, const uint8_t* w13,
                           const uint8_t* w13e, const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* ntpp, const int32_t* eoff, int E, int H, int I, int P,
                           int top_k, int BM, int nblk, uint8_t* aq, uint8_t* ae, hipStream_t stream);
hipError_t launch_gemm2_mx(const uint8_t* aq, const uint8_t* ae, const uint8_t* w2, const uint8_t* w2e,
                           const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntpp,
                           const int32_t* eoff, int E, int H, int I, int P, int BM, int nblk,
                           uint16_t* y, int y_stride, uint16_t* y_dump, hipStream_t stream);
// GEMM2 with an output bounded to rows [0, y_rows) and columns [0, y_cols):
// stores outside go to a 1024-byte dump; with ksplit > 1, K slices go to
// float32 partials [ksplit, y_rows, y_cols] and are summed into y (the dense linear).
// mx: act_scale / w_scale point at UE8M0 exponent bytes, one per row and 32 K
// elements (BM must be 128 and every K slice at least two 128-blocks)
hipError_t launch_gemm2_bounded(const uint8_t* act, const float* act_scale, const uint8_t* w,
                                const float* w_scale, const int32_t* sorted_ids,
                                const int32_t* expert_ids, const int32_t* ntpp, const int32_t* eoff,
                                int N, int K, int P, int BM, int nblk, uint16_t* y, int y_stride,
                                int y_rows, int y_cols, uint16_t* y_dump, int ksplit, float* part,
                                bool mx, hipStream_t stream);
// quantise rows [e*M, e*M + counts[e]) of x [E*M, K] (group 128, float32 scales)
hipError_t launch_group_quant_masked(const void* x, const int32_t* counts, int E, int M, int K,
                                     uint8_t* q, float* s, hipStream_t stream);
// sorted layout of the batched format (token e*M + r = row r of expert e, counts[e] real rows)
hipError_t launch_batched_layout(const int32_t* counts, int E, int M, int BM, int32_t* sorted_ids,
                                 int32_t* expert_ids, int32_t* ntpp, int32_t* eoff,
                                 int32_t* pair_pos, hipStream_t stream);
// topk_w NULL: unit weights (a gather of the rows, zeros for row -1)
hipError_t launch_combine(const uint16_t* y, int y_stride, const int32_t* pair_pos,
                          const float* topk_w, int T, int H, int top_k, uint16_t* out,
                          hipStream_t stream);
// the combine over launch_gemm2's float32 K-slice partials (pairs with
// pair_pos -1 contribute zero)
hipError_t launch_combine_slices(const float* part, int y_stride, int nslice, int P,
                                 const int32_t* pair_pos, const float* topk_w, int T, int H,
                                 int top_k, uint16_t* out, hipStream_t stream);

// matrix-core rate probe (kind 0: f16 16x16x32, 1: FP8 16x16x128), nblocks x 256
// threads, one float per thread stored to sink
hipError_t launch_mfma_probe(int kind, int iters, int nblocks, float* sink, hipStream_t stream);
// HBM read-stream probe: nblocks x 256 threads XOR src (bytes, a multiple of
// 16) into one word per thread of sink
hipError_t launch_hbm_read_probe(const void* src, size_t bytes, int nblocks, uint32_t* sink,
                                 hipStream_t stream);

}  // namespace moe
