// Sort-and-pad of routed pairs by expert ("moe_align").
//
// Operation (overview page, "Triton Fused MoE Kernel": each program block
// takes BLOCK_SIZE_M sorted tokens of one expert): the P = T*top_k pairs
// p = t*top_k + j are grouped by expert in ascending p, each expert's run is
// padded with the sentinel P to a multiple of block_m, and every block of
// block_m rows records its expert.
//
// A deterministic three-kernel counting sort, no host synchronisation and no
// global atomics:
//   1. count:   each 1024-pair chunk builds its per-expert histogram in LDS.
//   2. scan:    one workgroup turns the chunk histograms into padded expert
//               offsets, the base of every (chunk, expert) run, the block ->
//               expert table, the sentinels and the padded total.
//   3. scatter: each chunk ranks its pairs stably inside their expert (a
//               ballot match inside each wave plus per-wave counts in LDS)
//               and writes them to base + rank; the forward also keeps the
//               inverse map (pair -> sorted row) for the combine.
#include "align_dev.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(1024) void align_count_kernel(const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ emap,
                                                           int n_map, int P, int E,
                                                           int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kChunk) hist[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * kChunk + threadIdx.x;
  if (p < P) {
    const int e = pair_expert(ids, emap, n_map, p);
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);   // ids outside [0, E) are dropped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) counts[(size_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(1024) void align_scan_kernel(
    const int32_t* __restrict__ counts, int nchunk, int E, int BM, int P,
    int32_t* __restrict__ base, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntpp, int32_t* __restrict__ eoff) {
  __shared__ int scan[kChunk];
  __shared__ int wsum[kChunk / 64];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
#pragma unroll 8
    for (int b = 0; b < nchunk; ++b) total += counts[(size_t)b * E + e];
  }
  const int pad = (total + BM - 1) / BM * BM;
  const int incl = block_inclusive_scan(pad, scan, wsum);
  const int excl = incl - pad;
  const int padded_total = scan[kChunk - 1];
  if (e == 0) ntpp[0] = padded_total;
  // first block of every expert, and the number of blocks in use after them
  if (e < E) eoff[e] = excl / BM;
  if (e == 0) eoff[E] = padded_total / BM;
  if (e < E) {
    int run = excl;
#pragma unroll 8
    for (int b = 0; b < nchunk; ++b) {
      base[(size_t)b * E + e] = run;
      run += counts[(size_t)b * E + e];
    }
    for (int r = total; r < pad; ++r) sorted_ids[excl + r] = P;
  }
  // block -> expert: the expert whose padded run [excl, incl) holds the block
  const int nblocks = padded_total / BM;
  for (int blk = threadIdx.x; blk < nblocks; blk += kChunk) {
    const int row = blk * BM;
    int lo = 0, hi = E - 1;  // first expert with inclusive end > row
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (scan[mid] > row) hi = mid; else lo = mid + 1;
    }
    expert_ids[blk] = lo;
  }
}

__global__ __launch_bounds__(1024) void align_scatter_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ emap, int n_map, int P, int E,
    int ebits, const int32_t* __restrict__ base, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ pair_pos) {
  __shared__ int wcnt[kChunk / 64][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (kChunk / 64) * E; i += kChunk) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int p = blockIdx.x * kChunk + threadIdx.x;
  const int e0 = p < P ? pair_expert(ids, emap, n_map, p) : -1;
  const bool valid = (unsigned)e0 < (unsigned)E;
  const int e = valid ? e0 : 0;
  unsigned long long peers = __ballot(valid);
  for (int bit = 0; bit < ebits; ++bit) {
    const bool b = (e >> bit) & 1;
    const unsigned long long m = __ballot(b);
    peers &= b ? m : ~m;
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  const int rank_in_wave = __popcll(peers & below);
  if (valid && rank_in_wave == 0) wcnt[wave][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w][e];
    const int pos = base[(size_t)blockIdx.x * E + e] + before + rank_in_wave;
    sorted_ids[pos] = p;
    if (pair_pos) pair_pos[p] = pos;
  } else if (pair_pos && p < P) {
    pair_pos[p] = -1;            // not in the layout: the combine skips it
  }
}

// The three steps in one workgroup, for at most kChunk pairs (decode
// batches): align_single in align_dev.hpp, from one launch instead of three.
__global__ __launch_bounds__(1024) void align_single_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ emap, int n_map, int P, int E,
    int BM, int ebits, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ ntpp, int32_t* __restrict__ eoff, int32_t* __restrict__ pair_pos) {
  __shared__ AlignSingleLds lds;
  align_single(lds, ids, emap, n_map, P, E, BM, ebits, sorted_ids, expert_ids, ntpp, eoff, pair_pos);
}

// The layout of one expert owning every row (the dense linear): sorted row r
// holds row r of the input (the sentinel M past its end), every block belongs
// to expert 0, eoff = {0, nblk} and the padded row count is nblk * BM.
__global__ __launch_bounds__(256) void identity_layout_kernel(int M, int BM, int nblk,
                                                              int32_t* __restrict__ sorted_ids,
                                                              int32_t* __restrict__ expert_ids,
                                                              int32_t* __restrict__ eoff,
                                                              int32_t* __restrict__ ntpp) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nblk * BM) sorted_ids[i] = i < M ? i : M;
  if (i < nblk) expert_ids[i] = 0;
  if (i == 0) {
    eoff[0] = 0;
    eoff[1] = nblk;
    ntpp[0] = nblk * BM;
  }
}

hipError_t launch_identity_layout(int M, int BM, int nblk, int32_t* sorted_ids,
                                  int32_t* expert_ids, int32_t* eoff, int32_t* ntpp,
                                  hipStream_t stream) {
  const long long n = (long long)nblk * BM;
  hipLaunchKernelGGL(identity_layout_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     M, BM, nblk, sorted_ids, expert_ids, eoff, ntpp);
  return hipGetLastError();
}

// The layout of the batched activation format: token t = e * M + r is row r
// of expert e, and expert e's first counts[e] rows (clamped to [0, M]) are
// real.  One workgroup: the padded expert offsets are a scan over E, then
// the sorted rows (t for real rows, the sentinel E * M for padding), the
// block -> expert table and the token -> row map (-1 for rows past a count,
// which the combine writes as zeros) are filled by all threads.
__global__ __launch_bounds__(1024) void batched_layout_kernel(
    const int32_t* __restrict__ counts, int E, int M, int BM, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntpp, int32_t* __restrict__ eoff,
    int32_t* __restrict__ pair_pos) {
  __shared__ int scan[kChunk];
  __shared__ int wsum[kChunk / 64];
  __shared__ int cnt[kMaxE], off[kMaxE];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E) {
    c = counts[e];
    c = c < 0 ? 0 : (c > M ? M : c);
    cnt[e] = c;
  }
  const int pad = (c + BM - 1) / BM * BM;
  block_inclusive_scan(pad, scan, wsum);
  const int total = scan[kChunk - 1];
  if (e < E) {
    off[e] = scan[e] - pad;
    eoff[e] = (scan[e] - pad) / BM;
  }
  if (e == 0) {
    eoff[E] = total / BM;
    ntpp[0] = total;
  }
  __syncthreads();
  const int P = E * M;
  for (int blk = threadIdx.x; blk < total / BM; blk += kChunk) {
    int lo = 0, hi = E - 1;  // first expert with inclusive end > row
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (scan[mid] > blk * BM) hi = mid; else lo = mid + 1;
    }
    expert_ids[blk] = lo;
  }
  for (int t = threadIdx.x; t < P; t += kChunk) {
    const int te = t / M, r = t - te * M;
    const bool real = r < cnt[te];
    if (real) sorted_ids[off[te] + r] = t;
    pair_pos[t] = real ? off[te] + r : -1;
  }
  for (int i = threadIdx.x; i < E * BM; i += kChunk) {   // padding after each expert's rows
    const int pe = i / BM, r = cnt[pe] + (i - pe * BM);
    if (r < (cnt[pe] + BM - 1) / BM * BM) sorted_ids[off[pe] + r] = P;
  }
}

hipError_t launch_batched_layout(const int32_t* counts, int E, int M, int BM, int32_t* sorted_ids,
                                 int32_t* expert_ids, int32_t* ntpp, int32_t* eoff,
                                 int32_t* pair_pos, hipStream_t stream) {
  hipLaunchKernelGGL(batched_layout_kernel, dim3(1), dim3(kChunk), 0, stream, counts, E, M, BM,
                     sorted_ids, expert_ids, ntpp, eoff, pair_pos);
  return hipGetLastError();
}

// scratch: per-chunk counts and bases [nchunk, E] each, then the expert
// block offsets [E + 1] that the GEMMs use to order their tiles
size_t align_scratch_bytes(int P, int E) {
  const size_t nchunk = ((size_t)P + kChunk - 1) / kChunk;
  return (2 * nchunk * (size_t)E + (size_t)E + 1) * sizeof(int32_t);
}

const int32_t* align_expert_offsets(const void* scratch, int P, int E) {
  const size_t nchunk = ((size_t)P + kChunk - 1) / kChunk;
  return (const int32_t*)scratch + 2 * nchunk * (size_t)E;
}

hipError_t launch_align(const int32_t* ids, const int32_t* emap, int n_map, int P, int E, int BM,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* pair_pos,
                        void* scratch, hipStream_t stream) {
  const int nchunk = (P + kChunk - 1) / kChunk;
  int32_t* counts = (int32_t*)scratch;
  int32_t* base = counts + (size_t)nchunk * E;
  int32_t* eoff = base + (size_t)nchunk * E;
  int ebits = 0;
  while ((1 << ebits) < E) ++ebits;
  if (nchunk == 1) {
    hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(kChunk), 0, stream, ids, emap, n_map, P,
                       E, BM, ebits, sorted_ids, expert_ids, ntpp, eoff, pair_pos);
    return hipGetLastError();
  }
  if (nchunk > 0)
    hipLaunchKernelGGL(align_count_kernel, dim3(nchunk), dim3(kChunk), 0, stream, ids, emap, n_map,
                       P, E, counts);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kChunk), 0, stream, counts, nchunk, E, BM, P,
                     base, sorted_ids, expert_ids, ntpp, eoff);
  if (nchunk > 0)
    hipLaunchKernelGGL(align_scatter_kernel, dim3(nchunk), dim3(kChunk), 0, stream, ids, emap,
                       n_map, P, E, ebits, base, sorted_ids, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
