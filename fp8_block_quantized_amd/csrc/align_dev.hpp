// The single-workgroup sort-and-pad (at most 1024 pairs), shared by the align
// kernel and the decode front-end kernel; the operation and the multi-chunk
// version are in align.hip.
#pragma once

#include "device_common.hpp"

namespace moe {

constexpr int kChunk = 1024;
constexpr int kMaxE = 512;

// Expert of pair p: ids[p], or through the expert map (global -> local, -1
// for experts held elsewhere) when one is given.  Anything outside [0, E)
// leaves the pair out of the layout.
__device__ __forceinline__ int pair_expert(const int32_t* ids, const int32_t* emap, int n_map, int p) {
  int e = ids[p];
  if (emap) e = (unsigned)e < (unsigned)n_map ? emap[e] : -1;
  return e;
}

struct AlignSingleLds {
  int hist[kMaxE];
  int scan[kChunk];
  int wcnt[kChunk / 64][kMaxE];
  int wsum[kChunk / 64];
};

// Inclusive prefix sum of v over the kChunk threads of the workgroup, also
// stored to scan[t]: a shuffle scan inside each wave, the 16 wave totals
// scanned by wave 0, then each wave's offset added (three barriers).
__device__ __forceinline__ int block_inclusive_scan(int v, int* scan, int* wsum) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kChunk / 64 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kChunk / 64; off <<= 1) {
      const int o = __shfl_up(w, off);
      if (lane >= off) w += o;
    }
    if (lane < kChunk / 64) wsum[lane] = w;
  }
  __syncthreads();
  if (wave > 0) v += wsum[wave - 1];
  scan[t] = v;
  __syncthreads();
  return v;
}

// Count, scan and scatter of P <= kChunk pairs by one workgroup of kChunk
// threads: the histogram, the padded offsets and the ranks stay in LDS, and
// only the expert block offsets (eoff) leave it for the GEMMs.  ids may
// point at global memory or at LDS that the workgroup has filled.
__device__ __forceinline__ void align_single(AlignSingleLds& s, const int32_t* ids,
                                             const int32_t* __restrict__ emap, int n_map, int P,
                                             int E, int BM, int ebits,
                                             int32_t* __restrict__ sorted_ids,
                                             int32_t* __restrict__ expert_ids,
                                             int32_t* __restrict__ ntpp, int32_t* __restrict__ eoff,
                                             int32_t* __restrict__ pair_pos) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int e = t; e < E; e += kChunk) s.hist[e] = 0;
  for (int i = t; i < (kChunk / 64) * E; i += kChunk) s.wcnt[i / E][i % E] = 0;
  __syncthreads();
  // 1. per-expert counts
  const int p = t;
  const int e0 = p < P ? pair_expert(ids, emap, n_map, p) : -1;
  const bool valid = (unsigned)e0 < (unsigned)E;
  if (valid) atomicAdd(&s.hist[e0], 1);
  __syncthreads();
  // 2. padded offsets, sentinels, block -> expert table
  const int total = t < E ? s.hist[t] : 0;
  const int pad = (total + BM - 1) / BM * BM;
  const int excl = block_inclusive_scan(pad, s.scan, s.wsum) - pad;
  const int padded_total = s.scan[kChunk - 1];
  if (t == 0) {
    ntpp[0] = padded_total;
    eoff[E] = padded_total / BM;
  }
  if (t < E) {
    eoff[t] = excl / BM;
    s.hist[t] = excl;                        // from here on: the expert's first row
    for (int r = total; r < pad; ++r) sorted_ids[excl + r] = P;
  }
  const int nblocks = padded_total / BM;
  for (int blk = t; blk < nblocks; blk += kChunk) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s.scan[mid] > blk * BM) hi = mid; else lo = mid + 1;
    }
    expert_ids[blk] = lo;
  }
  // 3. stable ranks: ballot match inside each wave, counts of earlier waves
  const int e = valid ? e0 : 0;
  unsigned long long peers = __ballot(valid);
  for (int bit = 0; bit < ebits; ++bit) {
    const bool b = (e >> bit) & 1;
    const unsigned long long m = __ballot(b);
    peers &= b ? m : ~m;
  }
  const int rank_in_wave = __popcll(peers & ((1ull << lane) - 1ull));
  if (valid && rank_in_wave == 0) s.wcnt[wave][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += s.wcnt[w][e];
    const int pos = s.hist[e] + before + rank_in_wave;
    sorted_ids[pos] = p;
    if (pair_pos) pair_pos[p] = pos;
  } else if (pair_pos && p < P) {
    pair_pos[p] = -1;
  }
}

}  // namespace moe
