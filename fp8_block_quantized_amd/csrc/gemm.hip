// Block-scaled FP8 grouped GEMMs over sorted tokens, with fused epilogues.
//
// Operation (overview page, "Triton Fused MoE Kernel": every block of
// BLOCK_SIZE_M sorted rows belongs to one expert; the quantized accumulation
// is dequantised in float32; "FusedMoE Class": w13 = gate+up and w2 = down,
// both [E, N, K]; fp8 oracle API page: static 128x128 weight blocks,
// dynamic 128-group activations, or the MXFP8 [1, 32] blocks):
//
//   GEMM1: h[r, n] = sum_kb xs[t, kb] * w13s[e, n/128, kb]
//                      * sum_{k in kb} dec(xq[t, k]) * dec(w13[e, n, k])
//          a = silu(h[:, :I]) * h[:, I:]  ->  per-row 128-group requant to
//          (aq, as) in sorted order
//   GEMM2: y[r, n] = sum_kb as[r, kb] * w2s[e, n/128, kb]
//                      * sum_{k in kb} dec(aq[r, k]) * dec(w2[e, n, k])
//          (bf16, sorted rows; the routing weight is the combine's)
//
// Common mapping onto gfx950.  A K step is one 128-wide scale block, so the
// product of a block is a fresh MFMA result and its two scales are applied
// once per output when it is folded into the accumulator: no partial sum
// spans scale blocks (with MXFP8 the MFMA applies the per-32 exponents and
// the accumulator runs through it).  Weights sit on the MFMA's M side (16
// weight rows per fragment) and tokens on its N side: decode-sized token
// counts still fill an MFMA, and every lane ends up with four consecutive
// output features of one token, which the epilogues store as packed words.
//
// Two families:
//   * decode (BM <= 64): each wave streams its private weight rows from HBM
//     straight into MFMA fragments one K block ahead; the token tile of a K
//     block is shared by the workgroup's waves through an XOR-swizzled,
//     double-buffered LDS tile (the MXFP8 decode kernels instead load the
//     token fragments per wave too, with no LDS);
//   * prefill (BM = 128): 128 rows x 256 weight rows per tile, 8 waves of
//     64 x 64, operands staged through a three-stage LDS ring filled by
//     direct global->LDS loads with hand-placed vmcnt waits; GEMM2 and the
//     dense linears run persistent (one workgroup per CU).
// GEMM2 uses v_mfma_f32_16x16x128_f8f6f4.  GEMM1 needs partial sums far
// more exact than the FP8 MFMA gives (see moe_gemm1_kernel) and runs on f16
// MFMAs of exactly converted operands, folded in float64 (decode) or float32
// (prefill); the MXFP8 layer's GEMM1 runs on the scaled FP8 MFMA instead.
//
// Work order: tiles are expert-major (the align scan publishes each expert's
// first block), and the XCD renumbering gives every XCD a contiguous range,
// so tiles sharing a token tile or an expert's weight panel run on one XCD
// and meet in its L2.  Tiles past the padded row count (read on the device)
// leave at once, so the grid is sized from the row capacity and the host
// never waits.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

struct GemmArgs {
  const uint8_t* act;        // GEMM1: xq [T, H]        GEMM2: aq [cap, I]
  const float* act_scale;    // GEMM1: xs [T, H/128]    GEMM2: as [cap, I/128]
  const uint8_t* w;          // GEMM1: w13 [E, 2I, H]   GEMM2: w2 [E, H, I]
  const float* w_scale;      // [E, N/128, K/128]
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* ntpp;
  uint8_t* aq_out;           // GEMM1: [cap, I]
  float* as_out;             // GEMM1: [cap, I/128]
  uint16_t* y_out;           // GEMM2: bf16 [cap, y_stride], sorted rows, before the routing weight
  int K;                     // reduction length (H or I)
  int N;                     // weight rows per expert (2I or H)
  int I;
  int H;
  int P;                     // pair count = padding sentinel
  int top_k;
  int n_tiles;               // I/128 (GEMM1) or ceil(H/256) (GEMM2)
  int nblk;                  // m blocks in the grid (row capacity / BM)
  const int32_t* eoff;       // [E + 1] first block of each expert, blocks in use
  int E;
  int split;                 // workgroups per row block (BM / rows per workgroup)
  int y_stride;              // GEMM2: row stride of y_out (H rounded up to 256)
  int y_rows, y_cols;        // GEMM2: stored region of y_out; other stores go to y_dump
  uint16_t* y_dump;          // GEMM2: 1024 bytes
  int ksplit;                // GEMM2 prefill: K slices per tile (1: bf16 y_out)
  float* part;               // GEMM2, ksplit > 1: float32 partials [ksplit, y_rows, y_stride]
  double* h_slices;          // GEMM1 decode with K slices: float64 partials of h [slices, P, 2I]
  int mx;                    // GEMM2 prefill: act_scale and w_scale hold UE8M0 exponent bytes,
                             // one per row and 32 K elements ([rows, K/32] and [E, N, K/32])
};

// M0 is written only inside these statements, each right before its load;
// the compiler uses M0 nowhere else in this file.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// The same loads with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (the saddr form): no 64-bit address arithmetic per lane.
__device__ __forceinline__ void dma16s(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4s(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_raw() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// a compile-time int for generic lambdas (loops instantiated per count)
template <int N>
struct IntC {
  static constexpr int value = N;
};

template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Tile order.  Workgroups are numbered expert by expert, then by weight
// tile, then over the expert's row blocks (split into `split` workgroups
// each), so the workgroups that read one expert's weight panel run at the same
// time and, with the XCD renumbering over the tiles in use, on one XCD: the
// panel comes from HBM once and from L2 for the other row blocks, and the
// token tiles they read meet in L2 and the MALL across weight tiles.  The
// grid is sized from the row capacity; workgroups past the tiles in use leave.
struct TileCoord {
  int b, half, j;
  bool valid;
};

__device__ __forceinline__ TileCoord tile_of(int bid, const GemmArgs& a) {
  const int per_block = a.split * a.n_tiles;
  const int n_real = load_uniform(a.eoff + a.E) * per_block;
  if (bid >= n_real) return {0, 0, 0, false};
  const int L = xcd_contiguous_id(bid, n_real);
  int lo = 0, hi = a.E - 1;           // the last expert whose first tile is <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (load_uniform(a.eoff + mid) * per_block <= L) lo = mid; else hi = mid - 1;
  }
  const int b0 = load_uniform(a.eoff + lo), nsub = (load_uniform(a.eoff + lo + 1) - b0) * a.split;
  const int local = L - b0 * per_block;
  const int j = local / nsub, sub = local - j * nsub;
  return {b0 + sub / a.split, sub % a.split, j, true};
}


__device__ __forceinline__ v8i load_frag_global(const uint8_t* p) {
  // 32 bytes of one row: K chunk g and chunk g+4 of the 128-byte block
  const uint4 a = *(const uint4*)(p);
  const uint4 b = *(const uint4*)(p + 64);
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// kSlices: the workgroups of a tile (TileCoord::half, args.split of them)
// each reduce one contiguous range of K blocks and store float32 partials by
// pair, part[slice][p][:] (the combine sums the slices in order); without it
// one workgroup covers all of K and stores the bf16 y row.
template <int BM, bool kSlices>
__global__ __launch_bounds__(256) void moe_gemm2_kernel(GemmArgs args) {
  constexpr int NQ = BM / 16;                  // token sub-tiles
  constexpr int CHUNKS = BM * 8;               // 16-byte chunks of a token tile
  constexpr int CPT = (CHUNKS + 255) / 256;    // chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][BM * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const TileCoord tc = tile_of(blockIdx.x, args);
  if (!tc.valid) return;
  const int b = tc.b, j = tc.j;
  const int e = load_uniform(args.expert_ids + b);
  const int K = args.K, nkb_all = K >> 7;
  // this workgroup's K blocks [kb0, kb0 + nkb)
  const int kb0 = kSlices ? (int)((long long)tc.half * nkb_all / args.split) : 0;
  const int nkb = kSlices ? (int)((long long)(tc.half + 1) * nkb_all / args.split) - kb0 : nkb_all;
  const int row0 = b * BM;

  // ---- weight side: 4 fragments of 16 rows per wave ----
  // (the last tile of an H that is not a multiple of 256 has two idle waves)
  const bool wave_on = 256 * j + 64 * wave < args.N;
  int prow[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) prow[pp] = 256 * j + 64 * wave + 16 * pp;
  const uint8_t* wbase = args.w + (size_t)e * args.N * K + (size_t)kb0 * 128;
  const uint8_t* wptr[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
    wptr[pp] = wbase + (size_t)(wave_on ? prow[pp] + l16 : l16) * K + g * 16;
  const int nblk_n = args.N >> 7;
  const float* ws0 =
      args.w_scale + ((size_t)e * nblk_n + (wave_on ? (256 * j + 64 * wave) >> 7 : 0)) * nkb_all + kb0;

  // ---- token side: BM x 128 tile per K block, staged in LDS ----
  const uint8_t* aptr[CPT];
  int soff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    aptr[i] = nullptr;
    soff[i] = -1;
    if (c < CHUNKS) {
      const int r = c >> 3, ch = c & 7;
      soff[i] = r * 128 + ((ch ^ (r & 7)) << 4);
      aptr[i] = args.act + (size_t)(row0 + r) * K + (size_t)kb0 * 128 + ch * 16;
    }
  }
  const float* sptr[NQ];
  int qoff0[NQ], qoff1[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int rq = 16 * q + l16;
    sptr[q] = args.act_scale + (size_t)(row0 + rq) * nkb_all + kb0;
    qoff0[q] = rq * 128 + ((g ^ (rq & 7)) << 4);
    qoff1[q] = rq * 128 + (((g + 4) ^ (rq & 7)) << 4);
  }

  // ---- prologue: K block 0 ----
  uint4 areg[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) areg[i] = aptr[i] ? *(const uint4*)aptr[i] : make_uint4(0, 0, 0, 0);
  v8i wcur[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) wcur[pp] = load_frag_global(wptr[pp]);
  float sa[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) sa[q] = sptr[q][0];
  float sw0 = ws0[0];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    if (soff[i] >= 0) *(uint4*)(&smem[0][soff[i]]) = areg[i];
  __syncthreads();

  v4f acc[4][NQ];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[pp][q] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int kn = kb + 1 < nkb ? kb + 1 : kb;     // the last prefetch re-reads
    const size_t koff = (size_t)kn * 128;
    // prefetch K block kn
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      areg[i] = aptr[i] ? *(const uint4*)(aptr[i] + koff) : make_uint4(0, 0, 0, 0);
    v8i wnext[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) wnext[pp] = load_frag_global(wptr[pp] + koff);
    float sa_n[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) sa_n[q] = sptr[q][kn];
    const float sw0_n = ws0[kn];

    // MFMAs on K block kb
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint4 t0 = *(const uint4*)(&smem[buf][qoff0[q]]);
      const uint4 t1 = *(const uint4*)(&smem[buf][qoff1[q]]);
      v8i bq;
      bq[0] = t0.x; bq[1] = t0.y; bq[2] = t0.z; bq[3] = t0.w;
      bq[4] = t1.x; bq[5] = t1.y; bq[6] = t1.z; bq[7] = t1.w;
      const float sc = sa[q] * sw0;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const v4f part =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wcur[pp], bq, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[pp][q][r] = __builtin_fmaf(part[r], sc, acc[pp][q][r]);
      }
    }
    if (kb + 1 < nkb) {
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        if (soff[i] >= 0) *(uint4*)(&smem[buf ^ 1][soff[i]]) = areg[i];
    }
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) wcur[pp] = wnext[pp];
#pragma unroll
    for (int q = 0; q < NQ; ++q) sa[q] = sa_n[q];
    sw0 = sw0_n;
  }

  // y of each sorted row of a real pair, bf16 (the combine applies the
  // routing weight); with K slices the float32 partial of the pair's row
  if (!wave_on) return;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int rq = 16 * q + l16;
    const int p = args.sorted_ids[row0 + rq];
    if (p >= args.P) continue;
    if (kSlices) {
      float* prow_out = args.part + ((size_t)tc.half * args.P + p) * args.y_stride;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int h0 = 256 * j + 64 * wave + 16 * pp + 4 * g;
        *(float4*)(prow_out + h0) = make_float4(acc[pp][q][0], acc[pp][q][1], acc[pp][q][2], acc[pp][q][3]);
      }
      continue;
    }
    uint16_t* yrow = args.y_out + (size_t)(row0 + rq) * args.y_stride;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int h0 = 256 * j + 64 * wave + 16 * pp + 4 * g;
      uint2 v;
      v.x = f32_to_bf16_bits(acc[pp][q][0]) | (f32_to_bf16_bits(acc[pp][q][1]) << 16);
      v.y = f32_to_bf16_bits(acc[pp][q][2]) | (f32_to_bf16_bits(acc[pp][q][3]) << 16);
      *(uint2*)(yrow + h0) = v;
    }
  }
}

// GEMM1 with partial sums exact to about 1e-9 of their size.
//
// The requantisation after SiLU*mul is a step function: a code that moves
// to the neighbouring e4m3 grid point shifts the whole output row by about
// |w2| * (one grid step), so the intermediate a must round to the same
// float32 as the exact product would.  The FP8 MFMA sums its products
// below float32 precision (about 1.4e-6 of sum |p| per 128 products on
// gfx950), which moved 0.16-0.5% of those codes on the Mixtral-, Qwen3- and
// DeepSeek-shaped layers and took outputs past the layer's bar; so this GEMM
// converts both e4m3 operands exactly to f16 (v_cvt_scalef32_pk_f16_fp8 with
// scale 1) and runs v_mfma_f32_16x16x32_f16 (four per 128-wide K block,
// chained), whose float32
// accumulation of the exact 8-bit products is accurate to ~1e-10 of sum |p|.
// Each block partial is scaled by xs * ws in float64 (exact) and summed in
// float64, and SiLU*mul is evaluated in float64 before the one rounding of
// a to float32.
//
// Workgroup = 4 waves, RM sorted rows x 256 weight rows (32 gate + 32 up per
// wave); a block of BM rows is covered by BM / RM workgroups.  Token tiles
// are staged in LDS already converted to f16 (RM x 128 x 2 bytes, XOR
// swizzled on 16-byte chunks, double buffered); weight fragments stream
// from HBM into registers one K block ahead and are converted there.
//
// kSlices (decode shapes whose tiles in use would leave CUs idle): the
// kslices workgroups of a tile each reduce one contiguous range of K blocks
// and store their float64 partials of h by pair, h_slices[slice][p][0, 2I);
// gemm1_slices_finish_kernel sums them in slice order and applies SiLU*mul
// and the requant exactly as the epilogue below does.
template <int RM, bool kSlices>
__global__ __launch_bounds__(256) void moe_gemm1_kernel(GemmArgs args, int BM, int split,
                                                        int kslices) {
  constexpr int NQ = RM / 16;
  constexpr int CHUNKS = RM * 8;               // 16-byte fp8 chunks of a token tile
  constexpr int CPT = (CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][RM * 256];
  __shared__ float red[4][RM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const TileCoord tc = tile_of(blockIdx.x, args);
  if (!tc.valid) return;
  const int b = tc.b, j = tc.j;
  // tc.half runs over the row parts of the block (split) times the K slices
  const int half = kSlices ? tc.half / kslices : tc.half;
  const int ks = kSlices ? tc.half - half * kslices : 0;
  const int row0 = b * BM + half * RM;
  if (split > 1 && load_uniform(args.sorted_ids + row0) >= args.P) return;   // padding only
  const int e = load_uniform(args.expert_ids + b);
  const int K = args.K, nkb_all = K >> 7;
  // this workgroup's K blocks [kb0, kb0 + nkb)
  const int kb0 = kSlices ? (int)((long long)ks * nkb_all / kslices) : 0;
  const int nkb = kSlices ? (int)((long long)(ks + 1) * nkb_all / kslices) - kb0 : nkb_all;

  int prow[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) prow[pp] = (pp < 2 ? 0 : args.I) + 128 * j + 32 * wave + 16 * (pp & 1);
  const uint8_t* wbase = args.w + (size_t)e * args.N * K + (size_t)kb0 * 128;
  const uint8_t* wptr[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) wptr[pp] = wbase + (size_t)(prow[pp] + l16) * K + g * 16;
  const int nblk_n = args.N >> 7;
  const float* ws0 = args.w_scale + ((size_t)e * nblk_n + j) * nkb_all + kb0;
  const float* ws1 = args.w_scale + ((size_t)e * nblk_n + (args.I >> 7) + j) * nkb_all + kb0;

  const uint8_t* aptr[CPT];
  int soff0[CPT], soff1[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    aptr[i] = nullptr;
    soff0[i] = soff1[i] = -1;
    if (c < CHUNKS) {
      const int r = c >> 3, ch = c & 7;
      soff0[i] = r * 256 + (((2 * ch) ^ (r & 15)) << 4);
      soff1[i] = r * 256 + (((2 * ch + 1) ^ (r & 15)) << 4);
      const int p = args.sorted_ids[row0 + r];
      if (p < args.P) aptr[i] = args.act + (size_t)(p / args.top_k) * K + (size_t)kb0 * 128 + ch * 16;
    }
  }
  const float* sptr[NQ];
  int qoff[NQ][4];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int rq = 16 * q + l16;
    const int p = args.sorted_ids[row0 + rq];
    sptr[q] = p < args.P ? args.act_scale + (size_t)(p / args.top_k) * nkb_all + kb0 : nullptr;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = 2 * g + (c & 1) + 8 * (c >> 1);
      qoff[q][c] = rq * 256 + ((idx ^ (rq & 15)) << 4);
    }
  }

  auto stage_tokens = [&](const uint4* regs, int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if (soff0[i] < 0) continue;
      _Float16 h[16];
      e4m3x4_to_f16(regs[i].x, h);
      e4m3x4_to_f16(regs[i].y, h + 4);
      e4m3x4_to_f16(regs[i].z, h + 8);
      e4m3x4_to_f16(regs[i].w, h + 12);
      *(uint4*)(&smem[buf][soff0[i]]) = *(const uint4*)(h);
      *(uint4*)(&smem[buf][soff1[i]]) = *(const uint4*)(h + 8);
    }
  };

  uint4 areg[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) areg[i] = aptr[i] ? *(const uint4*)aptr[i] : make_uint4(0, 0, 0, 0);
  v8i wcur[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) wcur[pp] = load_frag_global(wptr[pp]);
  float sa[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) sa[q] = sptr[q] ? sptr[q][0] : 0.0f;
  float sw0 = ws0[0], sw1 = ws1[0];
  stage_tokens(areg, 0);
  __syncthreads();

  double acc[4][NQ][4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[pp][q][r] = 0.0;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int kn = kb + 1 < nkb ? kb + 1 : kb;
    const size_t koff = (size_t)kn * 128;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      areg[i] = aptr[i] ? *(const uint4*)(aptr[i] + koff) : make_uint4(0, 0, 0, 0);
    v8i wnext[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) wnext[pp] = load_frag_global(wptr[pp] + koff);
    float sa_n[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) sa_n[q] = sptr[q] ? sptr[q][kn] : 0.0f;
    const float sw0_n = ws0[kn], sw1_n = ws1[kn];

    v8h wf[4][4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        _Float16 h[8];
        e4m3x4_to_f16((uint32_t)wcur[pp][2 * c], h);
        e4m3x4_to_f16((uint32_t)wcur[pp][2 * c + 1], h + 4);
        wf[pp][c] = *(const v8h*)h;
      }
    const double sw0d = (double)sw0, sw1d = (double)sw1;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      v8h tq[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) tq[c] = *(const v8h*)(&smem[buf][qoff[q][c]]);
      const double sad = (double)sa[q];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        v4f part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[pp][0], tq[0], zero, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[pp][1], tq[1], part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[pp][2], tq[2], part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[pp][3], tq[3], part, 0, 0, 0);
        const double sc = sad * (pp < 2 ? sw0d : sw1d);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[pp][q][r] = __builtin_fma((double)part[r], sc, acc[pp][q][r]);
      }
    }
    if (kb + 1 < nkb) stage_tokens(areg, buf ^ 1);
    __syncthreads();
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) wcur[pp] = wnext[pp];
#pragma unroll
    for (int q = 0; q < NQ; ++q) sa[q] = sa_n[q];
    sw0 = sw0_n;
    sw1 = sw1_n;
  }

  if (kSlices) {
    // float64 partials of the pair's gate and up features of this wave
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int p = args.sorted_ids[row0 + 16 * q + l16];
      if (p >= args.P) continue;
      double* hrow = args.h_slices + ((size_t)ks * args.P + p) * (2 * (size_t)args.I);
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        const int i = 128 * j + 32 * wave + 16 * pg + 4 * g;
        *(double2*)(hrow + i) = make_double2(acc[pg][q][0], acc[pg][q][1]);
        *(double2*)(hrow + i + 2) = make_double2(acc[pg][q][2], acc[pg][q][3]);
        *(double2*)(hrow + args.I + i) = make_double2(acc[pg + 2][q][0], acc[pg + 2][q][1]);
        *(double2*)(hrow + args.I + i + 2) = make_double2(acc[pg + 2][q][2], acc[pg + 2][q][3]);
      }
    }
    return;
  }

  // a = silu(gate) * up in float64, rounded once to float32, then requantised
  // per row over the 128 features of tile j
  float av[NQ][2][4];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float m = 0.0f;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double gt = acc[pg][q][r], up = acc[pg + 2][q][r];
        const float a = (float)(gt / (1.0 + exp(-gt)) * up);
        av[q][pg][r] = a;
        m = __builtin_fmaxf(m, __builtin_fabsf(a));
      }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    if (lane < 16) red[wave][16 * q + l16] = m;
  }
  __syncthreads();
  const int Iq = args.I;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int rq = 16 * q + l16;
    const float amax = __builtin_fmaxf(__builtin_fmaxf(red[0][rq], red[1][rq]),
                                       __builtin_fmaxf(red[2][rq], red[3][rq]));
    float s, rcp;
    group_scale(amax, s, rcp);
    const size_t grow = (size_t)(row0 + rq);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int i = 128 * j + 32 * wave + 16 * pg + 4 * g;
      const uint32_t word = pack4_e4m3(clamp_fp8(div_by_scale(av[q][pg][0], s, rcp)),
                                       clamp_fp8(div_by_scale(av[q][pg][1], s, rcp)),
                                       clamp_fp8(div_by_scale(av[q][pg][2], s, rcp)),
                                       clamp_fp8(div_by_scale(av[q][pg][3], s, rcp)));
      *(uint32_t*)(args.aq_out + grow * Iq + i) = word;
    }
    if (wave == 0 && lane < 16) args.as_out[grow * (Iq >> 7) + j] = s;
  }
}

constexpr int kMaxGemm1Slices = 8;

// The end of moe_gemm1_kernel<RM, true>: per pair p (at sorted row pair_pos[p])
// and 128-feature group j, h = the float64 sum of the slices' partials in
// slice order, then a = float32(silu(gate) * up) evaluated in float64, the
// group's amax, scale and e4m3 codes, exactly as that kernel's own epilogue.
// Half a wave per (p, j): lane l holds features 128 j + 4 l .. 4 l + 3.
__global__ __launch_bounds__(256) void gemm1_slices_finish_kernel(const double* __restrict__ hs,
                                                                  int kslices, int P, int I,
                                                                  const int32_t* __restrict__ pair_pos,
                                                                  uint8_t* __restrict__ aq,
                                                                  float* __restrict__ as) {
  const int nj = I >> 7;
  const long long hw = ((long long)blockIdx.x * 256 + threadIdx.x) >> 5;   // half-wave index
  const int l = threadIdx.x & 31;
  const bool on = hw < (long long)P * nj;
  const int p = on ? (int)(hw / nj) : 0, j = on ? (int)(hw - (long long)p * nj) : 0;
  const int row = on ? pair_pos[p] : -1;
  const int i = 128 * j + 4 * l;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  float m = 0.0f;
  if (row >= 0) {
    // every slice's loads in flight together (kslices <= kMaxGemm1Slices), then
    // the sums in slice order
    double2 g0[kMaxGemm1Slices], g1[kMaxGemm1Slices], u0[kMaxGemm1Slices], u1[kMaxGemm1Slices];
#pragma unroll
    for (int s = 0; s < kMaxGemm1Slices; ++s) {
      if (s < kslices) {
        const double* h = hs + ((size_t)s * P + p) * (2 * (size_t)I);
        g0[s] = *(const double2*)(h + i);
        g1[s] = *(const double2*)(h + i + 2);
        u0[s] = *(const double2*)(h + I + i);
        u1[s] = *(const double2*)(h + I + i + 2);
      }
    }
    double gt[4] = {0.0, 0.0, 0.0, 0.0}, up[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < kMaxGemm1Slices; ++s) {
      if (s < kslices) {
        gt[0] += g0[s].x; gt[1] += g0[s].y; gt[2] += g1[s].x; gt[3] += g1[s].y;
        up[0] += u0[s].x; up[1] += u0[s].y; up[2] += u1[s].x; up[3] += u1[s].y;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = (float)(gt[r] / (1.0 + exp(-gt[r])) * up[r]);
      m = __builtin_fmaxf(m, __builtin_fabsf(a[r]));
    }
  }
  m = wave_max_xor(m, 16, 1);             // within the half-wave
  if (row < 0) return;
  float s, rcp;
  group_scale(m, s, rcp);
  *(uint32_t*)(aq + (size_t)row * I + i) =
      pack4_e4m3(clamp_fp8(div_by_scale(a[0], s, rcp)), clamp_fp8(div_by_scale(a[1], s, rcp)),
                 clamp_fp8(div_by_scale(a[2], s, rcp)), clamp_fp8(div_by_scale(a[3], s, rcp)));
  if (l == 0) as[(size_t)row * nj + j] = s;
}

// ---------------------------------------------------------------------------
// Prefill kernels: a three-stage LDS ring filled by direct global->LDS loads.
//
// With 128-row blocks the GEMMs are compute- and L2-bandwidth-heavy, and a
// one-block register prefetch cannot cover the load latency.  These kernels
// keep two K blocks of weights and tokens in flight through LDS
// (global_load_lds_dwordx4 writes each lane's 16 bytes straight into LDS, no
// registers involved; the XOR swizzle is produced by permuting the source
// addresses).  The loads and their waits are inline asm: the compiler would
// otherwise wait for every outstanding LDS load before each LDS read, since
// it cannot tell the ring's stages apart, which serialises the pipeline.
// Per K block: wait until the oldest stage has landed (vmcnt), barrier, issue
// the stage two blocks ahead into the slot every wave finished reading one
// iteration ago, compute.  Everything the loop reads besides the ring comes
// through scalar loads, so no compiler-inserted vector-memory wait drains the
// ring.
// ---------------------------------------------------------------------------
constexpr int kRingStages = 3;
constexpr int kRingW = 256 * 128;      // 256 weight rows x one 128-byte K block

// GEMM2 prefill, persistent.  A tile is 128 sorted rows x 256 output
// features; eight waves (two per SIMD) own 64 tokens x 64 features each, with
// one FP8 MFMA per 16x16 tile and K block and a float32 accumulator.
//
// The grid is one workgroup per CU.  Each XCD takes a contiguous range of the
// tiles in use (expert-major order, so an expert's weight panel is read by
// row blocks running together on one XCD), and the XCD's workgroups walk it
// with a stride of their count.  A workgroup's tiles form one stream of
// K-block stages through a three-stage LDS ring: the first stages of the next
// tile load while the current tile finishes and stores its outputs, so no
// tile waits for its first operands and no workgroup start-up is exposed.
//
// Every wait is a hand-placed vmcnt: before computing stage s, the loads of
// stage s + 1 and the 16 output stores of a tile that ended one or two steps
// earlier may still be in flight (vector memory operations retire in order).
// The epilogue therefore stores unconditionally (the output has whole
// 256-feature tiles per row, padding rows included) and issues no loads.
// Needs at least two K blocks per tile.  A tile may cover one of ksplit equal
// K slices (for outputs with few tiles): it then stores float32 partials,
// which a reduction kernel sums in slice order.
//
// kMx: both operands carry a power-of-two scale per row and 32 K elements
// (MXFP8), applied by the MFMA itself (v_mfma_scale_f32_16x16x128_f8f6f4):
// the lane that holds 32 K values of a row in the instruction's K order
// (bytes 16g..16g+15 and 64+16g..64+16g+15 of the block for lane group g)
// passes the exponent byte of that row's 32-element block g, so the scale
// blocks of the instruction are exactly the 32-wide blocks of memory.  The
// accumulator then runs through the MFMAs across K blocks with no float
// fold.  The stage holds the exponent words of the 128 token rows (as the
// float scales would) and of the tile's 256 weight rows, loaded by waves 2-5
// in the slots the other waves leave unused.
//
// A wave whose 64 token rows of the tile are all padding (its first row is
// the sentinel) loads, waits and stores as usual but skips its MFMAs (the
// prefill GEMM1 skips per 16-row group; here that cost more than it saved).  The stores of a 16-row group that is all padding go to the 1 KB
// dump rather than to y: every wave still issues kPf2Stores per tile, which
// the ring's counted waits rely on, but the padding rows cost no HBM writes.
constexpr int kPf2Loads = 7;               // DMA instructions per wave per stage
constexpr int kPf2Stores = 16;             // output stores per wave per tile
constexpr int kPf2S = 2048;                // token scales, eight 256-byte wave slots

struct TileId {
  int e, b, j, ks;
  bool dead16;   // the 16 token rows this wave loads are all padding
};

// Logical tile L -> (expert, m block, n tile) in expert-major order, by a
// binary search over the expert block offsets.  Within an expert the row
// blocks go in groups of kRowGroup: group-major, then n tile, then the
// group's row blocks.  The 32 workgroups of an XCD that run together then
// cover 8 row blocks x 4 weight panels (256 KB of operands per K block from
// beyond L2) rather than 32 row blocks x 1 panel (544 KB); an expert with at
// most 8 row blocks is one group.  Scalar loads only: they stay out of the
// vector memory counter that the ring's waits rely on.
constexpr int kRowGroup = 8;

__device__ __forceinline__ TileId tile_id(int L, const GemmArgs& a, int ksplit) {
  const int ks = L % ksplit;
  L /= ksplit;
  const int nt = a.n_tiles;
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (load_uniform(a.eoff + mid) * nt <= L) lo = mid; else hi = mid - 1;
  }
  const int b0 = load_uniform(a.eoff + lo), nb = load_uniform(a.eoff + lo + 1) - b0;
  const int local = L - b0 * nt;
  const int grp = local / (kRowGroup * nt), rem = local - grp * kRowGroup * nt;
  const int left = nb - grp * kRowGroup, gb = left < kRowGroup ? left : kRowGroup;
  const int j = rem / gb, b = b0 + grp * kRowGroup + (rem - j * gb);
  // padding rows are a suffix of the block: wave w loads token rows 16 w .. 16 w + 15
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return {lo, b, j, ks, load_uniform(a.sorted_ids + b * 128 + 16 * w) >= a.P};
}

template <bool kSplitK, bool kMx>
__global__ __launch_bounds__(512) void moe_gemm2_pf_kernel(GemmArgs args) {
  constexpr int BM = 128;
  constexpr int kA = BM * 128, kStage = kRingW + kA + kPf2S;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingStages * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave >> 2, wf = wave & 3;
  const int g = lane >> 4, l16 = lane & 15;
  const int K = args.K, nkb = K >> 7, N = args.N;
  const int ksplit = kSplitK ? args.ksplit : 1;
  const int nkb_t = nkb / ksplit;         // K blocks of one tile's slice

  // this workgroup's tiles
  const int n_real = load_uniform(args.eoff + args.E) * args.n_tiles * ksplit;
  const int per_xcd = gridDim.x >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int q8 = n_real >> 3, r8 = n_real & 7;
  const int xbeg = xcd * q8 + (xcd < r8 ? xcd : r8), xcnt = q8 + (xcd < r8 ? 1 : 0);
  const int ntile = slot < xcnt ? (xcnt - 1 - slot) / per_xcd + 1 : 0;
  if (ntile == 0) return;
  const int G = ntile * nkb_t;
  auto tile_at = [&](int i) { return tile_id(xbeg + slot + i * per_xcd, args, ksplit); };

  // this lane's 16-byte pieces of a stage: weight rows (wave*4 + i)*8 + lr of
  // the tile's 256, token rows (wave*2 + i)*8 + lr of its 128, chunk lc under
  // the rows' XOR swizzle (rows 8 apart share it)
  const int lr = lane >> 3, lc = (lane & 7) ^ lr;
  auto w_offsets = [&](int j, uint32_t (&o)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 256 * j + (wave * 4 + i) * 8 + lr;
      o[i] = (uint32_t)((row < N ? row : 0) * K + lc * 16);    // rows past H: any valid row
    }
  };
  uint32_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) aoff[i] = (uint32_t)(((wave * 2 + i) * 8 + lr) * K + lc * 16);
  // a slice of padding rows loads row 0 of the block instead (an L2 hit; the
  // slots it fills feed only padding outputs)
  const uint32_t aoff_dead = (uint32_t)(lc * 16);
  const uint32_t soff = (uint32_t)(((wave & 1) * 64 + lane) * nkb * 4);
  auto issue = [&](int stage, const TileId& t, const uint32_t (&wo)[4], int kb) {
    const uint32_t base = lds_offset(ring + stage * kStage);
    const int kg = t.ks * nkb_t + kb;      // K block within the full reduction
    const uint8_t* wb = args.w + (size_t)t.e * N * K + (size_t)kg * 128;
    const uint8_t* ab = args.act + (size_t)t.b * BM * K + (size_t)kg * 128;
    const uint8_t* sb = (const uint8_t*)(args.act_scale + (size_t)t.b * BM * nkb + kg);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16s(wo[i], wb, base + (wave * 4 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      dma16s(t.dead16 ? aoff_dead : aoff[i], ab, base + kRingW + (wave * 2 + i) * 1024);
    if (kMx && wave >= 2 && wave < 6) {
      // exponent words of weight rows 256 j + 64 (wave - 2) + lane at K block kg
      const int row = 256 * t.j + 64 * (wave - 2) + lane;
      const uint8_t* eb = (const uint8_t*)args.w_scale + ((size_t)t.e * N * nkb + kg) * 4;
      dma4s((uint32_t)((row < N ? row : 0) * nkb * 4), eb, base + kRingW + kA + wave * 256);
    } else {
      dma4s(soff, sb, base + kRingW + kA + wave * 256);
    }
  };
  // LDS byte offsets of this lane's operand pieces: row, chunks g and g + 4;
  // rows 16 apart share the swizzle, so each fragment is a base + immediate
  int pbase[2], qbase[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pbase[h] = (64 * wf + l16) * 128 + (((g + 4 * h) ^ (l16 & 7)) << 4);
    qbase[h] = kRingW + (64 * wt + l16) * 128 + (((g + 4 * h) ^ (l16 & 7)) << 4);
  }
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  TileId cur = tile_at(0), nxt = cur;
  uint32_t cwo[4], nwo[4];
  w_offsets(cur.j, cwo);
  if (ntile > 1) {
    nxt = tile_at(1);
    w_offsets(nxt.j, nwo);
  }
  issue(0, cur, cwo, 0);
  issue(1, cur, cwo, 1);
  int s = 0;
  for (int ti = 0; ti < ntile; ++ti) {
    const int nf = 256 * cur.j + 64 * wf;
    const bool live = load_uniform(args.sorted_ids + cur.b * BM + 64 * wt) < args.P;
    const float* wsp = kMx ? nullptr
                           : args.w_scale + ((size_t)cur.e * (N >> 7) + ((nf < N ? nf : 0) >> 7)) * nkb;
    v4f acc[4][4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[pp][q] = zero;
    for (int kb = 0; kb < nkb_t; ++kb, ++s) {
      const bool more = s + 1 < G, stores = ti > 0 && kb < 2;
      if (more) {
        if (stores) wait_vmem<kPf2Loads + kPf2Stores>(); else wait_vmem<kPf2Loads>();
      } else {
        if (stores) wait_vmem<kPf2Stores>(); else wait_vmem<0>();
      }
      barrier_raw();
      if (s + 2 < G) {
        if (kb + 2 < nkb_t) issue((s + 2) % kRingStages, cur, cwo, kb + 2);
        else issue((s + 2) % kRingStages, nxt, nwo, kb + 2 - nkb_t);
      }
      if (!live) continue;
      const uint8_t* st = ring + (s % kRingStages) * kStage;
      v8i pf[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const uint4 a0 = *(const uint4*)(st + pbase[0] + pp * 2048);
        const uint4 a1 = *(const uint4*)(st + pbase[1] + pp * 2048);
        pf[pp] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      }
      if (kMx) {
        // exponent bytes: weight row 64 wf + 16 pp + l16 at stage byte 512 + 4 row + g,
        // token row 64 wt + 16 q + l16 at 4 row + g
        const uint8_t* se = st + kRingW + kA;
        int ew[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) ew[pp] = se[512 + (64 * wf + 16 * pp + l16) * 4 + g];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 b0 = *(const uint4*)(st + qbase[0] + q * 2048);
          const uint4 b1 = *(const uint4*)(st + qbase[1] + q * 2048);
          const v8i bq = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          const int ea = se[(64 * wt + 16 * q + l16) * 4 + g];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
            acc[pp][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf[pp], bq, acc[pp][q], 0, 0,
                                                                         0, ew[pp], 0, ea);
        }
      } else {
        const float sw = load_uniform(wsp + cur.ks * nkb_t + kb);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 b0 = *(const uint4*)(st + qbase[0] + q * 2048);
          const uint4 b1 = *(const uint4*)(st + qbase[1] + q * 2048);
          const v8i bq = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          const float sc = *(const float*)(st + kRingW + kA + (64 * wt + 16 * q + l16) * 4) * sw;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf[pp], bq, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[pp][q][r] = __builtin_fmaf(part[r], sc, acc[pp][q][r]);
          }
        }
      }
    }
    // y rows of the tile, bf16: kPf2Stores stores whatever the bounds, the
    // ones outside the stored region (a dense output's ragged edge) or in an
    // all-padding 16-row group into the dump
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = cur.b * BM + 64 * wt + 16 * q + l16;
      const bool pad = load_uniform(args.sorted_ids + cur.b * BM + 64 * wt + 16 * q) >= args.P;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int col = nf + 16 * pp + 4 * g;
        const bool in = !pad && row < args.y_rows && col < args.y_cols;
        if (!kSplitK) {
          uint16_t* dst = in ? args.y_out + (size_t)row * args.y_stride + col : args.y_dump + 4 * lane;
          uint2 v;
          v.x = f32_to_bf16_bits(acc[pp][q][0]) | (f32_to_bf16_bits(acc[pp][q][1]) << 16);
          v.y = f32_to_bf16_bits(acc[pp][q][2]) | (f32_to_bf16_bits(acc[pp][q][3]) << 16);
          *(uint2*)dst = v;
        } else {     // float32 partial of K slice ks
          float* dst = in ? args.part + ((size_t)cur.ks * args.y_rows + row) * args.y_stride + col
                          : (float*)args.y_dump + 4 * lane;
          *(float4*)dst = make_float4(acc[pp][q][0], acc[pp][q][1], acc[pp][q][2], acc[pp][q][3]);
        }
      }
    }
    if (ti + 1 < ntile) {
      cur = nxt;
#pragma unroll
      for (int i = 0; i < 4; ++i) cwo[i] = nwo[i];
      if (ti + 2 < ntile) {
        nxt = tile_at(ti + 2);
        w_offsets(nxt.j, nwo);
      }
    }
  }
}

// GEMM1 prefill.  A workgroup takes one 128-row block and 128 features: the
// 128 gate rows and 128 up rows of w13 that feed them, which is one whole
// requantisation group, so SiLU*mul and the requant run in the epilogue.
// Eight waves (two per SIMD: one wave's conversions and scale folds overlap
// the other's MFMAs) split the tile 2 x 4: 64 tokens x (32 gate + 32 up
// features).  Per 128-wide K block a wave converts 8 e4m3 fragments per
// 32-wide chunk to f16 and issues 16 chained v_mfma_f32_16x16x32_f16; its
// conversions grow with the wave tile's edges and its MFMAs with the area,
// and 64 x 64 is the largest tile whose float32 accumulators and block
// partials fit two waves per SIMD.  Each block partial (exact to ~1e-10 of
// sum |p|, as in moe_gemm1_kernel) is scaled by xs * ws and added into a
// float32 accumulator: the order of the oracle's kernel reading, with a
// relative error of a few 1e-7, far below one e4m3 step of a.  Operands stay
// e4m3 in a three-stage LDS ring filled by direct global->LDS loads (XOR
// swizzle on 16-byte chunks, no bank conflicts on the 16-byte reads).
// Padding rows sit at the end of an expert's last block, so the real rows of
// a wave's 64 form a prefix of its four 16-row groups.  The K loop is
// instantiated for 0-4 live groups: every wave loads its share of every
// stage and meets every barrier, but converts, multiplies and folds only the
// token fragments of its live groups (the other rows' outputs are never
// read); in the last block of an expert that drops the MFMAs of up to 48
// padding rows per wave.
constexpr int kPf1Stages = 3;
constexpr int kPf1W = 256 * 128, kPf1A = 128 * 128, kPf1S = 2048;
constexpr int kPf1Stage = kPf1W + kPf1A + kPf1S;
constexpr int kPf1Loads = 7;               // DMA instructions per wave per stage

__global__ __launch_bounds__(512) void moe_gemm1_pf_kernel(GemmArgs args) {
  constexpr int BM = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kPf1Stages * kPf1Stage];
  __shared__ float red[2][4][64];           // per-token amax of each wave's 32 features
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave >> 2, wr = wave & 3;
  const int g = lane >> 4, l16 = lane & 15;
  const TileCoord tc = tile_of(blockIdx.x, args);
  if (!tc.valid) return;
  const int b = tc.b, j = tc.j;
  const int e = load_uniform(args.expert_ids + b);
  const int K = args.K, nkb = K >> 7, I = args.I, i0 = 128 * j;
  const int row0 = b * BM;
  // live 16-row groups of this wave's rows: those whose first row is real
  int nlive = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) nlive += load_uniform(args.sorted_ids + row0 + 64 * wt + 16 * q) < args.P;

  // this lane's share of a stage: 4 x 16 bytes of weights, 2 x 16 of tokens
  const uint8_t* wsrc[4];
  const uint8_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = (wave * 4 + i) * 64 + lane, r = pos >> 3, lc = (pos & 7) ^ (r & 7);
    const int wrow = r < 128 ? i0 + r : I + i0 + (r - 128);
    wsrc[i] = args.w + ((size_t)e * args.N + wrow) * K + lc * 16;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pos = (wave * 2 + i) * 64 + lane, r = pos >> 3, lc = (pos & 7) ^ (r & 7);
    const int p = args.sorted_ids[row0 + r];
    asrc[i] = args.act + (size_t)(p < args.P ? p / args.top_k : 0) * K + lc * 16;
  }
  const float* ssrc;
  {
    const int p = args.sorted_ids[row0 + (wave & 1) * 64 + lane];
    ssrc = args.act_scale + (size_t)(p < args.P ? p / args.top_k : 0) * nkb;
  }
  // the token scales of rows 0..127 land in slots 0 and 1; the other waves'
  // copies fill unused slots and keep every wave's load count equal
  auto issue = [&](int stage, int kb) {
    const uint32_t base = lds_offset(ring + stage * kPf1Stage);
    const size_t ko = (size_t)kb * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(wsrc[i] + ko, base + (wave * 4 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(asrc[i] + ko, base + kPf1W + (wave * 2 + i) * 1024);
    dma4(ssrc + kb, base + kPf1W + kPf1A + wave * 256);
  };
  const int nbn = args.N >> 7;
  const float* wsg = args.w_scale + ((size_t)e * nbn + j) * nkb;
  const float* wsu = args.w_scale + ((size_t)e * nbn + ((I + i0) >> 7)) * nkb;
  // LDS byte offsets of this lane's 8-byte operand pieces: row, 16-byte chunk
  // (g + 4h) under the row's XOR swizzle; the chunk's second half is +8
  int pw[4][2], pa[4][2];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int r = (pp < 2 ? 32 * wr + 16 * pp : 128 + 32 * wr + 16 * (pp - 2)) + l16;
#pragma unroll
    for (int h = 0; h < 2; ++h) pw[pp][h] = r * 128 + (((g + 4 * h) ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 64 * wt + 16 * q + l16;
#pragma unroll
    for (int h = 0; h < 2; ++h) pa[q][h] = kPf1W + r * 128 + (((g + 4 * h) ^ (r & 7)) << 4);
  }
  v4f acc[4][4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[pp][q] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  auto frag = [](const uint8_t* p) {
    const uint2 d = *(const uint2*)p;
    _Float16 h[8];
    e4m3x4_to_f16(d.x, h);
    e4m3x4_to_f16(d.y, h + 4);
    return *(const v8h*)h;
  };

  // the K loop with NQ live token groups (the same loads, waits and barriers
  // for every NQ)
  auto kloop = [&](auto nq_c) {
    constexpr int NQ = decltype(nq_c)::value, NA = NQ > 0 ? NQ : 1;
    issue(0, 0);
    if (nkb > 1) issue(1, 1);
    for (int kb = 0; kb < nkb; ++kb) {
      // stage kb has landed once at most the next stage's loads are pending
      if (kb + 1 < nkb) wait_vmem<kPf1Loads>(); else wait_vmem<0>();
      barrier_raw();
      if (kb + 2 < nkb) issue((kb + 2) % kPf1Stages, kb + 2);
      if (NQ == 0) continue;
      const uint8_t* st = ring + (kb % kPf1Stages) * kPf1Stage;
      const float swg = load_uniform(wsg + kb), swu = load_uniform(wsu + kb);
      float sa[NA];
#pragma unroll
      for (int q = 0; q < NQ; ++q) sa[q] = *(const float*)(st + kPf1W + kPf1A + (64 * wt + 16 * q + l16) * 4);
      v4f part[4][NA];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v8h wf[4], tf[NA];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) wf[pp] = frag(st + pw[pp][c >> 1] + 8 * (c & 1));
#pragma unroll
        for (int q = 0; q < NQ; ++q) tf[q] = frag(st + pa[q][c >> 1] + 8 * (c & 1));
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            part[pp][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[pp], tf[q], c == 0 ? zero : part[pp][q], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const float sc = sa[q] * (pp < 2 ? swg : swu);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[pp][q][r] = __builtin_fmaf(part[pp][q][r], sc, acc[pp][q][r]);
        }
    }
  };
  switch (nlive) {
    case 0: kloop(IntC<0>{}); break;
    case 1: kloop(IntC<1>{}); break;
    case 2: kloop(IntC<2>{}); break;
    case 3: kloop(IntC<3>{}); break;
    default: kloop(IntC<4>{}); break;
  }

  // a = silu(gate) * up in float32, then the per-row requant over the 128
  // features of tile j: amax across the wave's lanes, then across its 4 waves
  float av[4][2][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float m = 0.0f;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gt = acc[pg][q][r], up = acc[pg + 2][q][r];
        const float a = gt / (1.0f + expf(-gt)) * up;
        av[q][pg][r] = a;
        m = __builtin_fmaxf(m, __builtin_fabsf(a));
      }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    if (lane < 16) red[wt][wr][16 * q + l16] = m;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rq = 16 * q + l16;
    const float amax = __builtin_fmaxf(__builtin_fmaxf(red[wt][0][rq], red[wt][1][rq]),
                                       __builtin_fmaxf(red[wt][2][rq], red[wt][3][rq]));
    float s, rcp;
    group_scale(amax, s, rcp);
    const size_t grow = (size_t)(row0 + 64 * wt + rq);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int i = i0 + 32 * wr + 16 * pg + 4 * g;
      const uint32_t word = pack4_e4m3(clamp_fp8(div_by_scale(av[q][pg][0], s, rcp)),
                                       clamp_fp8(div_by_scale(av[q][pg][1], s, rcp)),
                                       clamp_fp8(div_by_scale(av[q][pg][2], s, rcp)),
                                       clamp_fp8(div_by_scale(av[q][pg][3], s, rcp)));
      *(uint32_t*)(args.aq_out + grow * I + i) = word;
    }
    if (wr == 0 && lane < 16) args.as_out[grow * (I >> 7) + j] = s;
  }
}

// GEMM1 of the MXFP8 layer (fp8 oracle API page, block shape [1, 32] with
// UE8M0 scales): xq and w13 carry one power-of-two exponent per row and 32 K
// elements, which v_mfma_scale_f32_16x16x128_f8f6f4 applies itself, so the
// float32 accumulator runs through the MFMAs across K blocks (the lane that
// holds a row's 32 K values in the instruction's K order, chunks g and g + 4
// of the block, passes that row's exponent of block g).  The epilogue forms
// a = silu(gate) * up in float32 and requantises it in groups of 32 features
// with power-of-two scales: a wave holds the 32 gate and 32 up rows of one
// group (features 32 wf .. 32 wf + 31 of the tile), so the group maximum of
// a token is a two-step butterfly over its four lanes.  Tile, ring and row
// gather as in moe_gemm1_pf_kernel; the stage's exponent slots hold the 128
// token rows' words (waves 0, 1) and the 256 weight rows' words (waves 2-5).
// A wave whose 64 token rows are all padding skips its MFMAs (a per-16-row
// skip as in moe_gemm1_pf_kernel did not pay off here).
__global__ __launch_bounds__(512) void moe_gemm1_mx_kernel(GemmArgs args) {
  constexpr int BM = 128;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kPf1Stages * kPf1Stage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave >> 2, wf = wave & 3;
  const int g = lane >> 4, l16 = lane & 15;
  const TileCoord tc = tile_of(blockIdx.x, args);
  if (!tc.valid) return;
  const int b = tc.b, j = tc.j;
  const int e = load_uniform(args.expert_ids + b);
  const int K = args.K, nkb = K >> 7, I = args.I, i0 = 128 * j;
  const int row0 = b * BM;
  const bool live = load_uniform(args.sorted_ids + row0 + 64 * wt) < args.P;
  // w13 row of tile row r: gate rows i0 .. i0 + 127, then up rows I + i0 ..
  auto wrow_of = [&](int r) { return r < 128 ? i0 + r : I + i0 + (r - 128); };

  const uint8_t* wsrc[4];
  const uint8_t* asrc[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = (wave * 4 + i) * 64 + lane, r = pos >> 3, lc = (pos & 7) ^ (r & 7);
    wsrc[i] = args.w + ((size_t)e * args.N + wrow_of(r)) * K + lc * 16;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pos = (wave * 2 + i) * 64 + lane, r = pos >> 3, lc = (pos & 7) ^ (r & 7);
    const int p = args.sorted_ids[row0 + r];
    asrc[i] = args.act + (size_t)(p < args.P ? p / args.top_k : 0) * K + lc * 16;
  }
  // exponent words (4 blocks of 32 per K block): token rows for waves 0, 1 (6, 7
  // repeat them into unused slots), weight tile rows 64 (wave - 2) + lane for 2-5
  const uint32_t* esrc;
  if (wave >= 2 && wave < 6) {
    esrc = (const uint32_t*)args.w_scale + ((size_t)e * args.N + wrow_of(64 * (wave - 2) + lane)) * nkb;
  } else {
    const int p = args.sorted_ids[row0 + (wave & 1) * 64 + lane];
    esrc = (const uint32_t*)args.act_scale + (size_t)(p < args.P ? p / args.top_k : 0) * nkb;
  }
  auto issue = [&](int stage, int kb) {
    const uint32_t base = lds_offset(ring + stage * kPf1Stage);
    const size_t ko = (size_t)kb * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(wsrc[i] + ko, base + (wave * 4 + i) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(asrc[i] + ko, base + kPf1W + (wave * 2 + i) * 1024);
    dma4(esrc + kb, base + kPf1W + kPf1A + wave * 256);
  };
  // tile rows of this wave's weight fragments: gate 32 wf + 16 pp, up 128 + 32 wf + 16 (pp - 2)
  int prow[4], pw[4][2], pa[4][2];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    prow[pp] = (pp < 2 ? 32 * wf + 16 * pp : 128 + 32 * wf + 16 * (pp - 2)) + l16;
#pragma unroll
    for (int h = 0; h < 2; ++h) pw[pp][h] = prow[pp] * 128 + (((g + 4 * h) ^ (l16 & 7)) << 4);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 64 * wt + 16 * q + l16;
#pragma unroll
    for (int h = 0; h < 2; ++h) pa[q][h] = kPf1W + r * 128 + (((g + 4 * h) ^ (l16 & 7)) << 4);
  }
  v4f acc[4][4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[pp][q] = v4f{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (nkb > 1) issue(1, 1);
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) wait_vmem<kPf1Loads>(); else wait_vmem<0>();
    barrier_raw();
    if (kb + 2 < nkb) issue((kb + 2) % kPf1Stages, kb + 2);
    if (!live) continue;
    const uint8_t* st = ring + (kb % kPf1Stages) * kPf1Stage;
    const uint8_t* se = st + kPf1W + kPf1A;
    v8i pf[4];
    int ew[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const uint4 a0 = *(const uint4*)(st + pw[pp][0]);
      const uint4 a1 = *(const uint4*)(st + pw[pp][1]);
      pf[pp] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      ew[pp] = se[512 + prow[pp] * 4 + g];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 b0 = *(const uint4*)(st + pa[q][0]);
      const uint4 b1 = *(const uint4*)(st + pa[q][1]);
      const v8i bq = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      const int ea = se[(64 * wt + 16 * q + l16) * 4 + g];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp)
        acc[pp][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf[pp], bq, acc[pp][q], 0, 0, 0,
                                                                     ew[pp], 0, ea);
    }
  }

  // a = silu(gate) * up, requantised per token and group of 32 features:
  // lane (g, l16) holds features 32 wf + 16 pg + 4 g + r (pg, r < 2, 4) of token row
  // 64 wt + 16 q + l16; the group's other features sit in the lanes g' != g
  uint8_t* ae = (uint8_t*)args.as_out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float av[2][4];
    float m = 0.0f;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gt = acc[pg][q][r], up = acc[pg + 2][q][r];
        av[pg][r] = gt / (1.0f + expf(-gt)) * up;
        m = __builtin_fmaxf(m, __builtin_fabsf(av[pg][r]));
      }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    const uint32_t sb = ceil_pow2_bits(__builtin_fmaxf(m, kAmaxEps) / kFp8Max);
    const float rcp = __uint_as_float((254u - (sb >> 23)) << 23);   // exactly 1 / scale
    const size_t grow = (size_t)(row0 + 64 * wt + 16 * q + l16);
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const uint32_t word = pack4_e4m3(clamp_fp8(av[pg][0] * rcp), clamp_fp8(av[pg][1] * rcp),
                                       clamp_fp8(av[pg][2] * rcp), clamp_fp8(av[pg][3] * rcp));
      *(uint32_t*)(args.aq_out + grow * I + i0 + 32 * wf + 16 * pg + 4 * g) = word;
    }
    if (g == 0) ae[grow * (I >> 5) + ((i0 + 32 * wf) >> 5)] = (uint8_t)(sb >> 23);
  }
}

// Decode-sized MXFP8 GEMMs (block_m <= 64), register-streamed.
//
// At decode sizes the GEMMs read each weight byte once from HBM, and the
// token rows (a few KB per K block) come from L2.  A workgroup covers 16
// token rows (a block of BM rows is BM / 16 workgroups, which read the same
// weights, the later ones from L2), and each of its waves 64 weight rows.
// Both operands are loaded straight into MFMA fragments (lane (g, l16)
// takes bytes 16g..16g+15 and 64+16g..64+16g+15 of its row's 128-byte K
// block, the scaled MFMA's K order) together with the row's exponent byte
// of 32-element block g.  No LDS and no barrier: every wave runs on its own,
// and the K loop alternates between two register sets, so the loads of K
// block kb + 1 are in flight while block kb is multiplied (a single set
// copied at the end of each step would make the compiler wait for those
// loads first).  Token rows past the block's real pairs read the first real
// row instead; their results are never stored.
struct MxDecStream {
  const uint8_t* w;      // this wave's weight fragment rows: base of the expert's matrix
  const uint8_t* we;     // and of its exponent bytes
  uint32_t woff[4];      // per fragment: row * K + 16 g
  uint32_t weoff[4];     // per fragment: row * K / 32 + g
  uint32_t wqoff;        // row l16 of fragment g: row * K / 32 (the 16-byte exponent groups)
};

// Buffer descriptor word 3 for raw byte-addressed buffers on CDNA
// (32-bit data format, no swizzle, range checking on the byte offset).
constexpr int kBufferWord3 = 0x00020000;

template <int NQ>
struct MxDecRegs {
  v8i w[4];
  v8i t[NQ];
  int ew[4];
  int et[NQ];
};

template <int NQ>
__device__ __forceinline__ void mx_dec_load(MxDecRegs<NQ>& r, const MxDecStream& s,
                                            const uint8_t* const (&tptr)[NQ],
                                            const uint8_t* const (&tep)[NQ], int kb) {
  const uint32_t ko = (uint32_t)kb * 128;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) r.w[pp] = load_frag_global(s.w + s.woff[pp] + ko);
#pragma unroll
  for (int q = 0; q < NQ; ++q) r.t[q] = load_frag_global(tptr[q] + ko);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) r.ew[pp] = s.we[s.weoff[pp] + 4 * kb];
#pragma unroll
  for (int q = 0; q < NQ; ++q) r.et[q] = tep[q][4 * kb];
}

template <int NQ>
__device__ __forceinline__ void mx_dec_mma(v4f (&acc)[4][NQ], const MxDecRegs<NQ>& r) {
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
      acc[pp][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r.w[pp], r.t[q], acc[pp][q], 0, 0,
                                                                   0, r.ew[pp], 0, r.et[q]);
}

// acc[pp][q] += W[rows of fragment pp] . T[token rows of q] over all nkb K blocks
template <int NQ>
__device__ __forceinline__ void mx_dec_kloop(v4f (&acc)[4][NQ], const MxDecStream& s,
                                             const uint8_t* const (&tptr)[NQ],
                                             const uint8_t* const (&tep)[NQ], int nkb) {
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[pp][q] = v4f{0.f, 0.f, 0.f, 0.f};
  // the scheduling barriers keep each load group ahead of the MFMAs it
  // overlaps (the scheduler would otherwise sink the loads below them)
  MxDecRegs<NQ> ra, rb;
  mx_dec_load(ra, s, tptr, tep, 0);
  int kb = 0;
  for (; kb + 2 <= nkb; kb += 2) {
    mx_dec_load(rb, s, tptr, tep, kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_mma(acc, ra);
    __builtin_amdgcn_sched_barrier(0);
    // the last even step re-reads block nkb - 1 (an L2 hit) rather than branch
    mx_dec_load(ra, s, tptr, tep, kb + 2 < nkb ? kb + 2 : nkb - 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_mma(acc, rb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kb < nkb) mx_dec_mma(acc, ra);   // odd nkb: block nkb - 1, loaded into ra
}

// The same loop for K a multiple of 512 with 16-byte aligned weight
// exponents: the exponent bytes of a weight row for four K blocks are one
// aligned 16-byte group.  Lane (g, l16) loads the group of row l16 of
// fragment g once per four K blocks, two steps before the next group's first
// use (its last word is kept aside for the group's last step), and the lane
// that multiplies fragment pp takes word d of lane (pp, l16)'s group with
// ds_bpermute and its byte g.  The weight exponents then cost one load per
// four K blocks instead of four per block.  The weights and their exponents
// are read through buffer descriptors over the expert's matrices (a 32-bit
// lane offset and the K step as the scalar offset; reads past the matrix
// would return zeros), which with the above leaves few enough registers for
// four waves per SIMD.
template <int NQ>
struct MxDecRegs4 {
  v8i w[4];
  v8i t[NQ];
  int et[NQ];
};

struct MxDecBuf {
  __amdgpu_buffer_rsrc_t w, we;   // the expert's weights and weight exponents
  uint32_t woff[4];               // per fragment: row * K + 16 g
  uint32_t wqoff;                 // row l16 of fragment g: row * K / 32
};

__device__ __forceinline__ v8i load_frag_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  const v4u a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
  const v4u b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff + 64, 0);
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

template <int NQ>
__device__ __forceinline__ void mx_dec_load4(MxDecRegs4<NQ>& r, const MxDecBuf& s,
                                             const uint8_t* const (&tptr)[NQ],
                                             const uint8_t* const (&tep)[NQ], int kb) {
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) r.w[pp] = load_frag_buf(s.w, s.woff[pp], kb * 128);
#pragma unroll
  for (int q = 0; q < NQ; ++q) r.t[q] = load_frag_global(tptr[q] + (size_t)kb * 128);
#pragma unroll
  for (int q = 0; q < NQ; ++q) r.et[q] = tep[q][4 * kb];
}

// word: this K block's word of the exponent group held by this lane
template <int NQ>
__device__ __forceinline__ void mx_dec_mma4(v4f (&acc)[4][NQ], const MxDecRegs4<NQ>& r, int word) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  int ew[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
    ew[pp] = (__builtin_amdgcn_ds_bpermute((16 * pp + l16) << 2, word) >> (8 * g)) & 0xff;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
      acc[pp][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r.w[pp], r.t[q], acc[pp][q], 0, 0,
                                                                   0, ew[pp], 0, r.et[q]);
}

template <int NQ>
__device__ __forceinline__ void mx_dec_kloop4(v4f (&acc)[4][NQ], const MxDecBuf& s,
                                              const uint8_t* const (&tptr)[NQ],
                                              const uint8_t* const (&tep)[NQ], int nkb) {
#pragma unroll
  for (int pp = 0; pp < 4; ++pp)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[pp][q] = v4f{0.f, 0.f, 0.f, 0.f};
  v4u wq = __builtin_amdgcn_raw_buffer_load_b128(s.we, s.wqoff, 0, 0);
  MxDecRegs4<NQ> ra, rb;
  mx_dec_load4(ra, s, tptr, tep, 0);
  for (int kb = 0; kb < nkb; kb += 4) {
    mx_dec_load4(rb, s, tptr, tep, kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_mma4(acc, ra, (int)wq[0]);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_load4(ra, s, tptr, tep, kb + 2);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_mma4(acc, rb, (int)wq[1]);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_load4(rb, s, tptr, tep, kb + 3);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_mma4(acc, ra, (int)wq[2]);
    __builtin_amdgcn_sched_barrier(0);
    // the last group re-reads block nkb - 1 and its own exponents rather than branch
    const int w3 = (int)wq[3];
    const int kn = kb + 4 < nkb ? kb + 4 : kb;
    wq = __builtin_amdgcn_raw_buffer_load_b128(s.we, s.wqoff, 4 * kn, 0);
    mx_dec_load4(ra, s, tptr, tep, kb + 4 < nkb ? kb + 4 : nkb - 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_dec_mma4(acc, rb, w3);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GEMM1: wave w holds the gate and up rows of features 32 w .. 32 w + 31 of
// the workgroup's 128-feature tile j (fragments pp = 0, 1 gate, 2, 3 up), so
// SiLU*mul pairs in-lane and each token's 32-feature requant group is reduced
// over the wave's four lane groups.  A block of BM rows is covered by
// BM / 16 workgroups.
template <bool kQuad>
__global__ __launch_bounds__(256) void moe_gemm1_mx_dec_kernel(GemmArgs args, int BM) {
  constexpr int RM = 16, NQ = 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const TileCoord tc = tile_of(blockIdx.x, args);
  if (!tc.valid) return;
  const int row0 = tc.b * BM + tc.half * RM;
  const int p0 = load_uniform(args.sorted_ids + row0);
  if (p0 >= args.P) return;   // padding only
  const int e = load_uniform(args.expert_ids + tc.b);
  const int K = args.K, nkb = K >> 7, I = args.I, i0 = 128 * tc.j;

  MxDecStream s;
  s.w = args.w + (size_t)e * args.N * K;
  s.we = (const uint8_t*)args.w_scale + (size_t)e * args.N * (nkb * 4);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int row = (pp < 2 ? 0 : I) + i0 + 32 * wave + 16 * (pp & 1) + l16;
    s.woff[pp] = (uint32_t)row * K + 16 * g;
    s.weoff[pp] = (uint32_t)row * (nkb * 4) + g;
  }
  s.wqoff = (uint32_t)((g < 2 ? 0 : I) + i0 + 32 * wave + 16 * (g & 1) + l16) * (nkb * 4);
  const uint32_t wbytes = (uint32_t)args.N * K;
  const uint8_t* tptr[NQ];
  const uint8_t* tep[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int p = args.sorted_ids[row0 + 16 * q + l16];
    if (p >= args.P) p = p0;
    const size_t tok = (size_t)(p / args.top_k);
    tptr[q] = args.act + tok * K + 16 * g;
    tep[q] = (const uint8_t*)args.act_scale + tok * (nkb * 4) + g;
  }

  v4f acc[4][NQ];
  if (kQuad) {
    MxDecBuf b;
    b.w = __builtin_amdgcn_make_buffer_rsrc((void*)s.w, 0, (int)wbytes, kBufferWord3);
    b.we = __builtin_amdgcn_make_buffer_rsrc((void*)s.we, 0, (int)(wbytes / 32), kBufferWord3);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) b.woff[pp] = s.woff[pp];
    b.wqoff = s.wqoff;
    mx_dec_kloop4(acc, b, tptr, tep, nkb);
  } else {
    mx_dec_kloop(acc, s, tptr, tep, nkb);
  }

  // a = silu(gate) * up, requantised per token row and 32-feature group;
  // padding rows are not written (nothing reads them)
  uint8_t* ae = (uint8_t*)args.as_out;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float av[2][4];
    float m = 0.0f;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gt = acc[pg][q][r], up = acc[pg + 2][q][r];
        av[pg][r] = gt / (1.0f + expf(-gt)) * up;
        m = __builtin_fmaxf(m, __builtin_fabsf(av[pg][r]));
      }
    m = __builtin_fmaxf(m, __shfl_xor(m, 16));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32));
    const uint32_t sb = ceil_pow2_bits(__builtin_fmaxf(m, kAmaxEps) / kFp8Max);
    const float rcp = __uint_as_float((254u - (sb >> 23)) << 23);
    const int grow = row0 + 16 * q + l16;
    if (args.sorted_ids[grow] >= args.P) continue;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const uint32_t word = pack4_e4m3(clamp_fp8(av[pg][0] * rcp), clamp_fp8(av[pg][1] * rcp),
                                       clamp_fp8(av[pg][2] * rcp), clamp_fp8(av[pg][3] * rcp));
      *(uint32_t*)(args.aq_out + (size_t)grow * I + i0 + 32 * wave + 16 * pg + 4 * g) = word;
    }
    if (g == 0) ae[(size_t)grow * (I >> 5) + ((i0 + 32 * wave) >> 5)] = (uint8_t)(sb >> 23);
  }
}

// GEMM2: wave w holds output features 256 j + 64 w .. + 63 (fragments of 16
// rows), bf16 y for each sorted row of a real pair (the combine applies the
// routing weight).  The sorted activation rows are dense, so token rows are
// rows row0 .. row0 + RM - 1 of act.  The last tile of an H that is not a
// multiple of 256 has idle waves, which leave at once.
template <bool kQuad>
__global__ __launch_bounds__(256) void moe_gemm2_mx_dec_kernel(GemmArgs args, int BM) {
  constexpr int RM = 16, NQ = 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const TileCoord tc = tile_of(blockIdx.x, args);
  if (!tc.valid) return;
  const int row0 = tc.b * BM + tc.half * RM;
  if (load_uniform(args.sorted_ids + row0) >= args.P) return;   // padding only
  const int h0 = 256 * tc.j + 64 * wave;
  if (h0 >= args.N) return;
  const int e = load_uniform(args.expert_ids + tc.b);
  const int K = args.K, nkb = K >> 7;

  MxDecStream s;
  s.w = args.w + (size_t)e * args.N * K;
  s.we = (const uint8_t*)args.w_scale + (size_t)e * args.N * (nkb * 4);
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int row = h0 + 16 * pp + l16;
    s.woff[pp] = (uint32_t)row * K + 16 * g;
    s.weoff[pp] = (uint32_t)row * (nkb * 4) + g;
  }
  s.wqoff = (uint32_t)(h0 + 16 * g + l16) * (nkb * 4);
  const uint32_t wbytes = (uint32_t)args.N * K;
  const uint8_t* tptr[NQ];
  const uint8_t* tep[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int r = row0 + 16 * q + l16;
    if (args.sorted_ids[r] >= args.P) r = row0;
    tptr[q] = args.act + (size_t)r * K + 16 * g;
    tep[q] = (const uint8_t*)args.act_scale + (size_t)r * (nkb * 4) + g;
  }

  v4f acc[4][NQ];
  if (kQuad) {
    MxDecBuf b;
    b.w = __builtin_amdgcn_make_buffer_rsrc((void*)s.w, 0, (int)wbytes, kBufferWord3);
    b.we = __builtin_amdgcn_make_buffer_rsrc((void*)s.we, 0, (int)(wbytes / 32), kBufferWord3);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) b.woff[pp] = s.woff[pp];
    b.wqoff = s.wqoff;
    mx_dec_kloop4(acc, b, tptr, tep, nkb);
  } else {
    mx_dec_kloop(acc, s, tptr, tep, nkb);
  }

#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int r = row0 + 16 * q + l16;
    if (args.sorted_ids[r] >= args.P) continue;
    uint16_t* yrow = args.y_out + (size_t)r * args.y_stride;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      uint2 v;
      v.x = f32_to_bf16_bits(acc[pp][q][0]) | (f32_to_bf16_bits(acc[pp][q][1]) << 16);
      v.y = f32_to_bf16_bits(acc[pp][q][2]) | (f32_to_bf16_bits(acc[pp][q][3]) << 16);
      *(uint2*)(yrow + h0 + 16 * pp + 4 * g) = v;
    }
  }
}

// The decode MXFP8 kernels' 16-byte weight exponent groups: K a multiple of
// 512 and the exponent array 16-byte aligned.
static bool mx_quad_ok(const GemmArgs& a) {
  return (a.K >> 7) % 4 == 0 && (uintptr_t)a.w_scale % 16 == 0;
}

hipError_t launch_gemm1_mx(const uint8_t* xq, const uint8_t* xe, const uint8_t* w13,
                           const uint8_t* w13e, const int32_t* sorted_ids, const int32_t* expert_ids,
                           const int32_t* ntpp, const int32_t* eoff, int E, int H, int I, int P,
                           int top_k, int BM, int nblk, uint8_t* aq, uint8_t* ae, hipStream_t stream) {
  GemmArgs a{};
  a.eoff = eoff; a.E = E; a.split = 1;
  a.act = xq; a.act_scale = (const float*)xe; a.w = w13; a.w_scale = (const float*)w13e;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.ntpp = ntpp;
  a.aq_out = aq; a.as_out = (float*)ae;
  a.K = H; a.N = 2 * I; a.I = I; a.H = H; a.P = P; a.top_k = top_k;
  a.nblk = nblk; a.n_tiles = I / 128; a.mx = 1;
  if (BM == 128) {
    hipLaunchKernelGGL(moe_gemm1_mx_kernel, dim3((unsigned)(nblk * a.n_tiles)), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  if (BM < 16 || BM > 64) return hipErrorInvalidValue;
  a.split = BM / 16;
  const dim3 grid((unsigned)(nblk * a.split * a.n_tiles)), block(256);
  if (mx_quad_ok(a))
    hipLaunchKernelGGL(moe_gemm1_mx_dec_kernel<true>, grid, block, 0, stream, a, BM);
  else
    hipLaunchKernelGGL(moe_gemm1_mx_dec_kernel<false>, grid, block, 0, stream, a, BM);
  return hipGetLastError();
}

// Sum of the float32 K-slice partials in slice order, rounded once to bf16:
// out[r, c] = bf16( sum_s part[s, r, c] ) for r < rows, c < cols (cols % 8 == 0).
__global__ __launch_bounds__(256) void reduce_slices_kernel(const float4* __restrict__ part,
                                                            int ksplit, int rows, int cols8,
                                                            uint4* __restrict__ out) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;   // 8 outputs per thread
  const long long n = (long long)rows * cols8;
  if (i >= n) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ksplit; ++s) {
    const float4 a = part[2 * (s * n + i)], b = part[2 * (s * n + i) + 1];
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  uint4 o;
  o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
  o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
  out[i] = o;
}

static hipError_t launch_reduce_slices(const float* part, int ksplit, int rows, int cols,
                                       uint16_t* out, hipStream_t stream) {
  const long long n = (long long)rows * (cols / 8);
  hipLaunchKernelGGL(reduce_slices_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const float4*)part, ksplit, rows, cols / 8, (uint4*)out);
  return hipGetLastError();
}

static hipError_t launch_gemm2_bm(const GemmArgs& a, int BM, hipStream_t stream) {
  const dim3 grid((unsigned)(a.nblk * a.n_tiles)), block(256);
  if (a.split > 1) {               // K slices of the register-streaming kernel, float32 partials by pair
    if (a.mx || a.ksplit != 1) return hipErrorInvalidValue;
    const dim3 gs((unsigned)(a.nblk * a.split * a.n_tiles));
    switch (BM) {
      case 16: hipLaunchKernelGGL((moe_gemm2_kernel<16, true>), gs, block, 0, stream, a); break;
      case 32: hipLaunchKernelGGL((moe_gemm2_kernel<32, true>), gs, block, 0, stream, a); break;
      case 64: hipLaunchKernelGGL((moe_gemm2_kernel<64, true>), gs, block, 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const bool persistent = BM == 128 && (a.K >> 7) / a.ksplit >= 2;
  if (a.mx && !persistent) {       // exponent scales: the persistent kernel, or the decode ones
    if (BM > 64 || a.ksplit != 1) return hipErrorInvalidValue;
    GemmArgs d = a;
    d.split = BM / 16;
    const dim3 g2((unsigned)(d.nblk * d.split * d.n_tiles));
    if (mx_quad_ok(d))
      hipLaunchKernelGGL(moe_gemm2_mx_dec_kernel<true>, g2, block, 0, stream, d, BM);
    else
      hipLaunchKernelGGL(moe_gemm2_mx_dec_kernel<false>, g2, block, 0, stream, d, BM);
    return hipGetLastError();
  }
  if (persistent) {
    // one persistent workgroup per CU, a multiple of the 8 XCDs
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    const long long tiles = (long long)a.nblk * a.n_tiles * a.ksplit;
    long long wg = cus / 8 * 8;
    if (wg > (tiles + 7) / 8 * 8) wg = (tiles + 7) / 8 * 8;
    if (wg < 8) wg = 8;
    if (a.mx && a.ksplit > 1)
      hipLaunchKernelGGL((moe_gemm2_pf_kernel<true, true>), dim3((unsigned)wg), dim3(512), 0, stream, a);
    else if (a.mx)
      hipLaunchKernelGGL((moe_gemm2_pf_kernel<false, true>), dim3((unsigned)wg), dim3(512), 0, stream, a);
    else if (a.ksplit > 1)
      hipLaunchKernelGGL((moe_gemm2_pf_kernel<true, false>), dim3((unsigned)wg), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((moe_gemm2_pf_kernel<false, false>), dim3((unsigned)wg), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  switch (BM) {
    case 16: hipLaunchKernelGGL((moe_gemm2_kernel<16, false>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((moe_gemm2_kernel<32, false>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((moe_gemm2_kernel<64, false>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((moe_gemm2_kernel<128, false>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm1(const uint8_t* xq, const float* xs, const uint8_t* w13, const float* w13s,
                        const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntpp,
                        const int32_t* eoff, int E, int H, int I, int P, int top_k, int BM, int nblk,
                        uint8_t* aq, float* as, int kslices, double* h_slices,
                        const int32_t* pair_pos, hipStream_t stream) {
  if (kslices > 1 && (BM > 64 || !h_slices || !pair_pos || kslices > (H >> 7) ||
                      kslices > kMaxGemm1Slices))
    return hipErrorInvalidValue;
  GemmArgs a{};
  a.eoff = eoff; a.E = E;
  a.act = xq; a.act_scale = xs; a.w = w13; a.w_scale = w13s;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.ntpp = ntpp;
  a.aq_out = aq; a.as_out = as;
  a.K = H; a.N = 2 * I; a.I = I; a.H = H; a.P = P; a.top_k = top_k;
  a.nblk = nblk;
  a.n_tiles = I / 128;
  if (BM == 128) {
    a.split = 1;
    hipLaunchKernelGGL(moe_gemm1_pf_kernel, dim3((unsigned)(nblk * a.n_tiles)), dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  const int rm = BM < 32 ? BM : 32;
  const int split = BM / rm;
  if (kslices > 1) {
    a.split = split * kslices;
    a.h_slices = h_slices;
    const dim3 grid((unsigned)(nblk * a.split * a.n_tiles)), block(256);
    if (rm == 16)
      hipLaunchKernelGGL((moe_gemm1_kernel<16, true>), grid, block, 0, stream, a, BM, split, kslices);
    else if (rm == 32)
      hipLaunchKernelGGL((moe_gemm1_kernel<32, true>), grid, block, 0, stream, a, BM, split, kslices);
    else
      return hipErrorInvalidValue;
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long long threads = (long long)P * (I >> 7) * 32;
    hipLaunchKernelGGL(gemm1_slices_finish_kernel, dim3((unsigned)((threads + 255) / 256)), block, 0,
                       stream, h_slices, kslices, P, I, pair_pos, aq, as);
    return hipGetLastError();
  }
  a.split = split;
  const dim3 grid((unsigned)(nblk * split * a.n_tiles)), block(256);
  if (rm == 16)
    hipLaunchKernelGGL((moe_gemm1_kernel<16, false>), grid, block, 0, stream, a, BM, split, 1);
  else if (rm == 32)
    hipLaunchKernelGGL((moe_gemm1_kernel<32, false>), grid, block, 0, stream, a, BM, split, 1);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm2(const uint8_t* aq, const float* as, const uint8_t* w2, const float* w2s,
                        const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntpp,
                        const int32_t* eoff, int E, int H, int I, int P, int BM, int nblk,
                        uint16_t* y, int y_stride, uint16_t* y_dump, int kslices, float* y_slices,
                        hipStream_t stream) {
  if (kslices > 1 && (BM > 64 || !y_slices || kslices > (I >> 7))) return hipErrorInvalidValue;
  GemmArgs a{};
  a.eoff = eoff; a.E = E; a.split = kslices > 1 ? kslices : 1;
  a.part = y_slices;
  a.act = aq; a.act_scale = as; a.w = w2; a.w_scale = w2s;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.ntpp = ntpp;
  a.y_out = y; a.y_stride = y_stride;
  a.y_rows = nblk * BM; a.y_cols = y_stride; a.y_dump = y_dump; a.ksplit = 1;
  a.K = I; a.N = H; a.I = I; a.H = H; a.P = P; a.top_k = 1;
  a.n_tiles = (H + 255) / 256; a.nblk = nblk;
  return launch_gemm2_bm(a, BM, stream);
}

hipError_t launch_gemm2_mx(const uint8_t* aq, const uint8_t* ae, const uint8_t* w2, const uint8_t* w2e,
                           const int32_t* sorted_ids, const int32_t* expert_ids, const int32_t* ntpp,
                           const int32_t* eoff, int E, int H, int I, int P, int BM, int nblk,
                           uint16_t* y, int y_stride, uint16_t* y_dump, hipStream_t stream) {
  GemmArgs a{};
  a.eoff = eoff; a.E = E; a.split = 1; a.mx = 1;
  a.act = aq; a.act_scale = (const float*)ae; a.w = w2; a.w_scale = (const float*)w2e;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.ntpp = ntpp;
  a.y_out = y; a.y_stride = y_stride;
  a.y_rows = nblk * BM; a.y_cols = y_stride; a.y_dump = y_dump; a.ksplit = 1;
  a.K = I; a.N = H; a.I = I; a.H = H; a.P = P; a.top_k = 1;
  a.n_tiles = (H + 255) / 256; a.nblk = nblk;
  return launch_gemm2_bm(a, BM, stream);
}

hipError_t launch_gemm2_bounded(const uint8_t* act, const float* act_scale, const uint8_t* w,
                                const float* w_scale, const int32_t* sorted_ids,
                                const int32_t* expert_ids, const int32_t* ntpp, const int32_t* eoff,
                                int N, int K, int P, int BM, int nblk, uint16_t* y, int y_stride,
                                int y_rows, int y_cols, uint16_t* y_dump, int ksplit, float* part,
                                bool mx, hipStream_t stream) {
  GemmArgs a{};
  a.mx = mx ? 1 : 0;
  a.eoff = eoff; a.E = 1; a.split = 1;
  a.act = act; a.act_scale = act_scale; a.w = w; a.w_scale = w_scale;
  a.sorted_ids = sorted_ids; a.expert_ids = expert_ids; a.ntpp = ntpp;
  a.y_out = y; a.y_stride = y_stride;
  a.y_rows = y_rows; a.y_cols = y_cols; a.y_dump = y_dump;
  a.ksplit = ksplit; a.part = part;
  a.K = K; a.N = N; a.I = K; a.H = N; a.P = P; a.top_k = 1;
  a.n_tiles = (N + 255) / 256; a.nblk = nblk;
  hipError_t err = launch_gemm2_bm(a, BM, stream);
  if (err != hipSuccess || ksplit == 1) return err;
  return launch_reduce_slices(part, ksplit, y_rows, y_cols, y, stream);
}

}  // namespace moe
