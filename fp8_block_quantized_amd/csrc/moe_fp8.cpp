// C ABI of the FP8 MoE library: argument checks, workspace layout and the
// launch sequence of the fused forward.  Every check runs on the host before
// anything is enqueued; nothing here allocates or synchronises.
#include "../../include/moe_fp8.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kDumpBytes = 1024;   // after y: the second GEMM's stores of padding row groups

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// row stride of the per-pair outputs: whole 256-feature tiles, so that the
// GEMM2 epilogue stores unconditionally
size_t y_stride(int H) { return round_up((size_t)H, 256); }

int check_moe_shape(int T, int H, int I, int E, int top_k) {
  if (T < 1 || T > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
  if (H < 128 || H % 128 || I < 128 || I % 128) return MOE_ERR_SHAPE;
  if (H > (1 << 16) || I > (1 << 16)) return MOE_ERR_SHAPE;
  if (2LL * I * H >= (1LL << 31)) return MOE_ERR_SHAPE;   // 32-bit offsets inside one expert
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (top_k < 1 || top_k > E || top_k > MOE_MAX_TOP_K) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// Rows per expert block: the smallest power of two holding 1.5x the mean
// number of pairs per expert, within [16, 128].  Decode batches get small
// blocks (little padding, one block per expert); prefill batches get 128.
int pick_block_m(int T, int E, int top_k) {
  const long long P = (long long)T * top_k;
  const double want = 1.5 * (double)P / (double)E;
  int bm = 16;
  while (bm < 128 && bm < want) bm <<= 1;
  return bm;
}

// K slices of the decode GEMM2 (block_m <= 64): when the weight tiles in use
// (at most one block per expert plus ceil(P / block_m) more, times ceil(H / 256)
// tiles of output features) would not give every CU of a 256-CU part four
// workgroups, each tile's K is split over up to 8 workgroups (at most one per
// 128-wide K block) that store float32 partials.  A function of the shape
// alone, so the workspace size is known before anything runs.  (The same
// kernel at block_m 128, one wave per SIMD, ran slower with slices than the
// persistent prefill kernel without them.)
int pick_kslices(int T, int H, int I, int E, int top_k, int BM) {
  if (BM > 64) return 1;
  const long long P = (long long)T * top_k;
  const long long cap_blocks = (P + (long long)E * (BM - 1) + BM - 1) / BM;
  long long live = (P + BM - 1) / BM + (E < P ? E : P);
  if (live > cap_blocks) live = cap_blocks;
  const long long tiles = live * ((H + 255) / 256), want = 4 * 256;
  if (tiles >= want) return 1;
  long long s = (want + tiles - 1) / tiles;
  if (s > 8) s = 8;
  if (s > I / 128) s = I / 128;
  return (int)s;
}

// K slices of the decode GEMM1 (block_m <= 64), by the same rule over its
// tiles (blocks in use x the block's row parts x I/128 feature groups) with
// a target of two workgroups per CU; at most 8 slices and one per 128-wide
// K block of H.  The slices' float64 partials are summed before SiLU*mul by
// a second kernel, whose launch and partial traffic cost more than a third
// workgroup per CU gains (the Qwen3-shaped T=32 ran slower split in two).
int pick_kslices1(int T, int H, int I, int E, int top_k, int BM) {
  if (BM > 64) return 1;
  const long long P = (long long)T * top_k;
  const long long cap_blocks = (P + (long long)E * (BM - 1) + BM - 1) / BM;
  long long live = (P + BM - 1) / BM + (E < P ? E : P);
  if (live > cap_blocks) live = cap_blocks;
  const long long rows_split = BM / (BM < 32 ? BM : 32);
  const long long tiles = live * rows_split * (I / 128), want = 2 * 256;
  if (tiles >= want) return 1;
  long long s = (want + tiles - 1) / tiles;
  if (s > 8) s = 8;
  if (s > H / 128) s = H / 128;
  return (int)s;
}

struct Layout {
  int BM;
  int kslices1;      // K slices of GEMM1 (1: its own epilogue requantises)
  int kslices;       // K slices of GEMM2 (1: bf16 y by sorted row)
  size_t cap;
  size_t off[MOE_TAP_COUNT];
  size_t total;
};

// block_m 0: the forward's choice; the MXFP8 layer passes 128.  The
// activation scale regions hold float32 per 128 elements or, at the same
// size, exponent bytes per 32.  slices: room for GEMM2's K-slice partials
// (the forward's layout; the batched and MXFP8 paths do not split K).
void make_layout(int T, int H, int I, int E, int top_k, Layout& L, int block_m = 0,
                 bool slices = true) {
  const size_t P = (size_t)T * top_k;
  L.BM = block_m ? block_m : pick_block_m(T, E, top_k);
  L.kslices = slices ? pick_kslices(T, H, I, E, top_k, L.BM) : 1;
  L.kslices1 = slices ? pick_kslices1(T, H, I, E, top_k, L.BM) : 1;
  L.cap = round_up(P + (size_t)E * (L.BM - 1), L.BM);
  size_t sz[MOE_TAP_COUNT];
  sz[MOE_TAP_TOPK_IDS] = P * 4;
  sz[MOE_TAP_TOPK_WEIGHTS] = P * 4;
  sz[MOE_TAP_SORTED_IDS] = L.cap * 4;
  sz[MOE_TAP_EXPERT_IDS] = (L.cap / L.BM) * 4;
  sz[MOE_TAP_NTPP] = 4;
  sz[MOE_TAP_PAIR_POS] = P * 4;
  sz[MOE_TAP_XQ] = (size_t)T * H;
  sz[MOE_TAP_XS] = (size_t)T * (H / 128) * 4;
  sz[MOE_TAP_AQ] = L.cap * I;
  sz[MOE_TAP_AS] = L.cap * (I / 128) * 4;
  sz[MOE_TAP_Y] = L.cap * y_stride(H) * 2 + kDumpBytes;
  sz[MOE_TAP_ALIGN_SCRATCH] = moe::align_scratch_bytes((int)P, E);
  sz[MOE_TAP_Y_SLICES] = L.kslices > 1 ? (size_t)L.kslices * P * y_stride(H) * 4 : 0;
  sz[MOE_TAP_H_SLICES] = L.kslices1 > 1 ? (size_t)L.kslices1 * P * 2 * I * 8 : 0;
  size_t o = 0;
  for (int i = 0; i < MOE_TAP_COUNT; ++i) {
    L.off[i] = o;
    o = round_up(o + sz[i], kAlign);
  }
  L.total = o;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// Dense linear: one expert owning every row, in blocks of 128 rows (the
// persistent GEMM), the reduction split into ksplit equal K slices when the
// output has too few tiles to give each of the 256 workgroups work.
struct LinearLayout {
  int BM, nblk, ksplit;
  size_t cap, xq, xs, sorted, eids, meta, dump, part, total;
};

// The divisor of the K-block count that minimises the K blocks the busiest
// of 256 workgroups streams (at least two per slice); ties to fewer slices.
int pick_ksplit(int nblk, int N, int K) {
  constexpr long long kWorkgroups = 256;
  const long long tiles = (long long)nblk * ((N + 255) / 256);
  const int nkb = K / 128;
  int best = 1;
  long long best_cost = (tiles + kWorkgroups - 1) / kWorkgroups * nkb;
  for (int d = 2; d <= nkb / 2; ++d) {
    if (nkb % d) continue;
    const long long cost = (tiles * d + kWorkgroups - 1) / kWorkgroups * (nkb / d);
    if (cost < best_cost) {
      best = d;
      best_cost = cost;
    }
  }
  return best;
}

int check_linear_shape(int M, int N, int K) {
  if (M < 1 || M > (1 << 20)) return MOE_ERR_SHAPE;
  if (N < 128 || N % 128 || K < 128 || K % 128) return MOE_ERR_SHAPE;
  if (N > (1 << 16) || K > (1 << 16) || (long long)N * K >= (1LL << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

void make_linear_layout(int M, int N, int K, LinearLayout& L) {
  L.BM = 128;
  L.nblk = (M + L.BM - 1) / L.BM;
  L.ksplit = pick_ksplit(L.nblk, N, K);
  L.cap = (size_t)L.nblk * L.BM;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, kAlign);
    return at;
  };
  L.xq = take(L.cap * K);            // rows past M: never written, read as padding
  L.xs = take(L.cap * (K / 128) * 4);
  L.sorted = take(L.cap * 4);
  L.eids = take((size_t)L.nblk * 4);
  L.meta = take(16);                 // eoff[2], ntpp
  L.dump = take(1024);
  L.part = take(L.ksplit > 1 ? (size_t)L.ksplit * M * N * 4 : 0);
  L.total = o;
}

}  // namespace

// Scratch of the scratch-free sort-and-pad (moe_align_noalloc): a file-scope
// device array sized for the largest call the ABI accepts (MOE_MAX_TOKENS *
// MOE_MAX_TOP_K pairs in 1024-pair chunks, MOE_MAX_EXPERTS experts: per-chunk
// counts and bases, then the expert block offsets).  Every GPU the library
// runs on holds its own copy, created with the code object and kept until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): it asks the runtime for the
// current device's address of it once per device and uses that.
namespace moe_noalloc {
constexpr size_t kChunkPairs = 1024;
constexpr size_t kScratchInts =
    2 * ((size_t)MOE_MAX_TOKENS * MOE_MAX_TOP_K / kChunkPairs) * MOE_MAX_EXPERTS + MOE_MAX_EXPERTS + 1;
__device__ __attribute__((aligned(256))) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of scratch on each device, once looked up

// Address of `scratch` on the current device: looked up on the first call
// on that device (with that device current), then reused.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}
}  // namespace moe_noalloc

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a multiple of 128";
    case MOE_ERR_UNSUPPORTED: return "request not supported by this library";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP runtime error at launch";
    case MOE_ERR_ALIAS: return "an output overlaps an input or the workspace";
    case MOE_ERR_SCRATCH: return "request exceeds the fixed scratch of a scratch-free entry point";
    default: return "unknown status";
  }
}

int moe_fp8_block_m(int T, int H, int I, int E, int top_k) {
  const int st = check_moe_shape(T, H, I, E, top_k);
  if (st != MOE_OK) return st;
  return pick_block_m(T, E, top_k);
}

size_t moe_fp8_workspace_bytes(int T, int H, int I, int E, int top_k) {
  if (check_moe_shape(T, H, I, E, top_k) != MOE_OK) return 0;
  Layout L;
  make_layout(T, H, I, E, top_k, L);
  return L.total;
}

int moe_fp8_workspace_layout(int T, int H, int I, int E, int top_k,
                             size_t offsets[MOE_TAP_COUNT]) {
  if (!offsets) return MOE_ERR_NULL;
  const int st = check_moe_shape(T, H, I, E, top_k);
  if (st != MOE_OK) return st;
  Layout L;
  make_layout(T, H, I, E, top_k, L);
  for (int i = 0; i < MOE_TAP_COUNT; ++i) offsets[i] = L.off[i];
  return MOE_OK;
}

// Routing options of the forward: grouped top-k and an expert map.
struct Routing {
  int num_group = 1, topk_group = 1;   // num_group 1: plain top-k
  const int32_t* emap = nullptr;       // device int32 [E]: global -> local expert or -1
  int e_local = 0;                     // experts the weights hold (E without a map)
};

static int check_routing(int E, int top_k, const Routing& r) {
  if (r.num_group < 1 || r.num_group > 64 || E % r.num_group) return MOE_ERR_SHAPE;
  if (r.num_group == 1 ? r.topk_group != 1 : (r.topk_group < 1 || r.topk_group > r.num_group))
    return MOE_ERR_SHAPE;
  if (top_k > r.topk_group * (E / r.num_group)) return MOE_ERR_SHAPE;
  if (r.emap ? (r.e_local < 1 || r.e_local > E) : r.e_local != E) return MOE_ERR_SHAPE;
  if (r.emap && (uintptr_t)r.emap % 4) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static int forward_impl(const void* x, const float* router_logits, const uint8_t* w13,
                        const float* w13_scale, const uint8_t* w2, const float* w2_scale, int T,
                        int H, int I, int E, int top_k, int renormalize, const Routing& route,
                        void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        hipEvent_t* ev) {
  if (!x || !router_logits || !w13 || !w13_scale || !w2 || !w2_scale || !out || !workspace)
    return MOE_ERR_NULL;
  int st = check_moe_shape(T, H, I, E, top_k);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_SHAPE;
  if ((st = check_routing(E, top_k, route)) != MOE_OK) return st;
  const int EL = route.e_local;        // experts of the weights, the layout's experts
  Layout L;
  make_layout(T, H, I, E, top_k, L);
  if (workspace_bytes < L.total || ((uintptr_t)workspace % kAlign)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)x % 16 || (uintptr_t)out % 16 || (uintptr_t)w13 % 16 || (uintptr_t)w2 % 16 ||
      (uintptr_t)router_logits % 4 || (uintptr_t)w13_scale % 4 || (uintptr_t)w2_scale % 4)
    return MOE_ERR_UNSUPPORTED;
  const size_t out_bytes = (size_t)T * H * 2;
  const size_t w13_bytes = (size_t)EL * 2 * I * H, w2_bytes = (size_t)EL * H * I;
  const size_t w13s_bytes = (size_t)EL * (2 * I / 128) * (H / 128) * 4;
  const size_t w2s_bytes = (size_t)EL * (H / 128) * (I / 128) * 4;
  if (overlaps(out, out_bytes, x, out_bytes) ||
      overlaps(out, out_bytes, router_logits, (size_t)T * E * 4) ||
      overlaps(out, out_bytes, w13, w13_bytes) || overlaps(out, out_bytes, w2, w2_bytes) ||
      overlaps(out, out_bytes, w13_scale, w13s_bytes) ||
      overlaps(out, out_bytes, w2_scale, w2s_bytes) ||
      overlaps(out, out_bytes, workspace, L.total) ||
      (route.emap && overlaps(out, out_bytes, route.emap, (size_t)E * 4)))
    return MOE_ERR_ALIAS;

  char* ws = (char*)workspace;
  int32_t* ids = (int32_t*)(ws + L.off[MOE_TAP_TOPK_IDS]);
  float* tw = (float*)(ws + L.off[MOE_TAP_TOPK_WEIGHTS]);
  int32_t* sorted = (int32_t*)(ws + L.off[MOE_TAP_SORTED_IDS]);
  int32_t* eids = (int32_t*)(ws + L.off[MOE_TAP_EXPERT_IDS]);
  int32_t* ntpp = (int32_t*)(ws + L.off[MOE_TAP_NTPP]);
  uint8_t* xq = (uint8_t*)(ws + L.off[MOE_TAP_XQ]);
  float* xs = (float*)(ws + L.off[MOE_TAP_XS]);
  uint8_t* aq = (uint8_t*)(ws + L.off[MOE_TAP_AQ]);
  float* as = (float*)(ws + L.off[MOE_TAP_AS]);
  uint16_t* y = (uint16_t*)(ws + L.off[MOE_TAP_Y]);
  int32_t* ppos = (int32_t*)(ws + L.off[MOE_TAP_PAIR_POS]);
  void* scratch = ws + L.off[MOE_TAP_ALIGN_SCRATCH];
  const int P = T * top_k;
  // the layout covers the EL local experts: at most P + EL * (BM - 1) rows, within
  // the workspace sized for E
  const int nblk = (int)(round_up((size_t)P + (size_t)EL * (L.BM - 1), L.BM) / L.BM);

  hipError_t err;
  auto mark = [&](int i) { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if (mark(0)) return MOE_ERR_HIP;
  if (moe::decode_front_fits(T, E, top_k)) {
    // one launch for the three front stages (their events all mark its end)
    int32_t* eoffw = (int32_t*)moe::align_expert_offsets(scratch, P, EL);
    if ((err = moe::launch_decode_front(router_logits, T, E, top_k, renormalize, route.num_group,
                                        route.topk_group, route.emap, E, EL, L.BM, x, H, ids, tw,
                                        sorted, eids, ntpp, eoffw, ppos, xq, xs, stream)))
      return MOE_ERR_HIP;
    if (mark(1) || mark(2) || mark(3)) return MOE_ERR_HIP;
  } else {
    if ((err = moe::launch_topk_softmax(router_logits, T, E, top_k, renormalize, route.num_group,
                                        route.topk_group, ids, tw, stream)))
      return MOE_ERR_HIP;
    if (mark(1)) return MOE_ERR_HIP;
    if ((err = moe::launch_align(ids, route.emap, E, P, EL, L.BM, sorted, eids, ntpp, ppos, scratch,
                                 stream)))
      return MOE_ERR_HIP;
    if (mark(2)) return MOE_ERR_HIP;
    if ((err = moe::launch_group_quant(x, T, H, xq, xs, stream))) return MOE_ERR_HIP;
    if (mark(3)) return MOE_ERR_HIP;
  }
  const int32_t* eoff = moe::align_expert_offsets(scratch, P, EL);
  double* hslices = (double*)(ws + L.off[MOE_TAP_H_SLICES]);
  if ((err = moe::launch_gemm1(xq, xs, w13, w13_scale, sorted, eids, ntpp, eoff, EL, H, I, P,
                               top_k, L.BM, nblk, aq, as, L.kslices1, hslices, ppos, stream)))
    return MOE_ERR_HIP;
  if (mark(4)) return MOE_ERR_HIP;
  float* yslices = (float*)(ws + L.off[MOE_TAP_Y_SLICES]);
  uint16_t* ydump = y + L.cap * y_stride(H);
  if ((err = moe::launch_gemm2(aq, as, w2, w2_scale, sorted, eids, ntpp, eoff, EL, H, I, P, L.BM,
                               nblk, y, (int)y_stride(H), ydump, L.kslices, yslices, stream)))
    return MOE_ERR_HIP;
  if (mark(5)) return MOE_ERR_HIP;
  if (L.kslices > 1)
    err = moe::launch_combine_slices(yslices, (int)y_stride(H), L.kslices, P, ppos, tw, T, H, top_k,
                                     (uint16_t*)out, stream);
  else
    err = moe::launch_combine(y, (int)y_stride(H), ppos, tw, T, H, top_k, (uint16_t*)out, stream);
  if (err) return MOE_ERR_HIP;
  if (mark(6)) return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_fp8_forward(const void* x, const float* router_logits, const uint8_t* w13,
                    const float* w13_scale, const uint8_t* w2, const float* w2_scale, int T,
                    int H, int I, int E, int top_k, int renormalize, void* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Routing r;
  r.e_local = E;
  return forward_impl(x, router_logits, w13, w13_scale, w2, w2_scale, T, H, I, E, top_k,
                      renormalize, r, out, workspace, workspace_bytes, stream, nullptr);
}

int moe_fp8_forward_routed(const void* x, const float* router_logits, const uint8_t* w13,
                           const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                           int T, int H, int I, int E, int top_k, int renormalize,
                           int num_expert_group, int topk_group, const int32_t* expert_map,
                           int num_local_experts, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  Routing r;
  r.num_group = num_expert_group;
  r.topk_group = topk_group;
  r.emap = expert_map;
  r.e_local = num_local_experts;
  return forward_impl(x, router_logits, w13, w13_scale, w2, w2_scale, T, H, I, E, top_k,
                      renormalize, r, out, workspace, workspace_bytes, stream, nullptr);
}

int moe_fp8_forward_traced(const void* x, const float* router_logits, const uint8_t* w13,
                           const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                           int T, int H, int I, int E, int top_k, int renormalize, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           hipEvent_t events[MOE_STAGE_COUNT + 1]) {
  if (!events) return MOE_ERR_NULL;
  for (int i = 0; i <= MOE_STAGE_COUNT; ++i)
    if (!events[i]) return MOE_ERR_NULL;
  Routing r;
  r.e_local = E;
  return forward_impl(x, router_logits, w13, w13_scale, w2, w2_scale, T, H, I, E, top_k,
                      renormalize, r, out, workspace, workspace_bytes, stream, events);
}

// The batched expert format uses the forward's layout for T = E * max_tokens
// tokens routed to one slot each (token e * max_tokens + r is row r of expert e).
size_t moe_fp8_batched_workspace_bytes(int E, int max_tokens, int H, int I) {
  if (E < 1 || max_tokens < 1 || (long long)E * max_tokens > MOE_MAX_TOKENS) return 0;
  if (check_moe_shape(E * max_tokens, H, I, E, 1) != MOE_OK) return 0;
  Layout L;
  make_layout(E * max_tokens, H, I, E, 1, L, 0, false);
  return L.total;
}

int moe_fp8_batched_experts(const void* x, const int32_t* expert_num_tokens, const uint8_t* w13,
                            const float* w13_scale, const uint8_t* w2, const float* w2_scale,
                            int E, int max_tokens, int H, int I, void* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (E < 1 || max_tokens < 1 || (long long)E * max_tokens > MOE_MAX_TOKENS) return MOE_ERR_SHAPE;
  const int T = E * max_tokens;
  int st = check_moe_shape(T, H, I, E, 1);
  if (st != MOE_OK) return st;
  if (!x || !expert_num_tokens || !w13 || !w13_scale || !w2 || !w2_scale || !out || !workspace)
    return MOE_ERR_NULL;
  Layout L;
  make_layout(T, H, I, E, 1, L, 0, false);
  if (workspace_bytes < L.total || ((uintptr_t)workspace % kAlign)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)x % 16 || (uintptr_t)out % 16 || (uintptr_t)w13 % 16 || (uintptr_t)w2 % 16 ||
      (uintptr_t)expert_num_tokens % 4 || (uintptr_t)w13_scale % 4 || (uintptr_t)w2_scale % 4)
    return MOE_ERR_UNSUPPORTED;
  const size_t out_bytes = (size_t)T * H * 2;
  const size_t w13_bytes = (size_t)E * 2 * I * H, w2_bytes = (size_t)E * H * I;
  const size_t w13s_bytes = (size_t)E * (2 * I / 128) * (H / 128) * 4;
  const size_t w2s_bytes = (size_t)E * (H / 128) * (I / 128) * 4;
  if (overlaps(out, out_bytes, x, out_bytes) || overlaps(out, out_bytes, w13, w13_bytes) ||
      overlaps(out, out_bytes, w2, w2_bytes) || overlaps(out, out_bytes, w13_scale, w13s_bytes) ||
      overlaps(out, out_bytes, w2_scale, w2s_bytes) ||
      overlaps(out, out_bytes, expert_num_tokens, (size_t)E * 4) ||
      overlaps(out, out_bytes, workspace, L.total))
    return MOE_ERR_ALIAS;
  char* ws = (char*)workspace;
  int32_t* sorted = (int32_t*)(ws + L.off[MOE_TAP_SORTED_IDS]);
  int32_t* eids = (int32_t*)(ws + L.off[MOE_TAP_EXPERT_IDS]);
  int32_t* ntpp = (int32_t*)(ws + L.off[MOE_TAP_NTPP]);
  int32_t* ppos = (int32_t*)(ws + L.off[MOE_TAP_PAIR_POS]);
  uint8_t* xq = (uint8_t*)(ws + L.off[MOE_TAP_XQ]);
  float* xs = (float*)(ws + L.off[MOE_TAP_XS]);
  uint8_t* aq = (uint8_t*)(ws + L.off[MOE_TAP_AQ]);
  float* as = (float*)(ws + L.off[MOE_TAP_AS]);
  uint16_t* y = (uint16_t*)(ws + L.off[MOE_TAP_Y]);
  int32_t* eoff = (int32_t*)(ws + L.off[MOE_TAP_ALIGN_SCRATCH]);   // [E + 1]
  const int nblk = (int)(L.cap / L.BM);
  if (moe::launch_batched_layout(expert_num_tokens, E, max_tokens, L.BM, sorted, eids, ntpp, eoff,
                                 ppos, stream))
    return MOE_ERR_HIP;
  if (moe::launch_group_quant_masked(x, expert_num_tokens, E, max_tokens, H, xq, xs, stream))
    return MOE_ERR_HIP;
  if (moe::launch_gemm1(xq, xs, w13, w13_scale, sorted, eids, ntpp, eoff, E, H, I, T, 1, L.BM,
                        nblk, aq, as, 1, nullptr, nullptr, stream))
    return MOE_ERR_HIP;
  if (moe::launch_gemm2(aq, as, w2, w2_scale, sorted, eids, ntpp, eoff, E, H, I, T, L.BM, nblk, y,
                        (int)y_stride(H), y + L.cap * y_stride(H), 1, nullptr, stream))
    return MOE_ERR_HIP;
  if (moe::launch_combine(y, (int)y_stride(H), ppos, nullptr, T, H, 1, (uint16_t*)out, stream))
    return MOE_ERR_HIP;
  return MOE_OK;
}

size_t moe_fp8_mx_workspace_bytes(int T, int H, int I, int E, int top_k) {
  if (check_moe_shape(T, H, I, E, top_k) != MOE_OK || I < 256) return 0;
  Layout L;
  make_layout(T, H, I, E, top_k, L, 0, false);
  return L.total;
}

int moe_fp8_mx_workspace_layout(int T, int H, int I, int E, int top_k,
                                size_t offsets[MOE_TAP_COUNT]) {
  if (!offsets) return MOE_ERR_NULL;
  const int st = check_moe_shape(T, H, I, E, top_k);
  if (st != MOE_OK) return st;
  if (I < 256) return MOE_ERR_UNSUPPORTED;
  Layout L;
  make_layout(T, H, I, E, top_k, L, 0, false);
  for (int i = 0; i < MOE_TAP_COUNT; ++i) offsets[i] = L.off[i];
  return MOE_OK;
}

int moe_fp8_mx_forward(const void* x, const float* router_logits, const uint8_t* w13,
                       const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale, int T,
                       int H, int I, int E, int top_k, int renormalize, void* out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!x || !router_logits || !w13 || !w13_scale || !w2 || !w2_scale || !out || !workspace)
    return MOE_ERR_NULL;
  int st = check_moe_shape(T, H, I, E, top_k);
  if (st != MOE_OK) return st;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_SHAPE;
  if (I < 256) return MOE_ERR_UNSUPPORTED;
  Layout L;
  make_layout(T, H, I, E, top_k, L, 0, false);
  if (workspace_bytes < L.total || ((uintptr_t)workspace % kAlign)) return MOE_ERR_WORKSPACE;
  if ((uintptr_t)x % 16 || (uintptr_t)out % 16 || (uintptr_t)w13 % 16 || (uintptr_t)w2 % 16 ||
      (uintptr_t)router_logits % 4 || (uintptr_t)w13_scale % 4 || (uintptr_t)w2_scale % 4)
    return MOE_ERR_UNSUPPORTED;
  const size_t out_bytes = (size_t)T * H * 2;
  const size_t w13_bytes = (size_t)E * 2 * I * H, w2_bytes = (size_t)E * H * I;
  if (overlaps(out, out_bytes, x, out_bytes) ||
      overlaps(out, out_bytes, router_logits, (size_t)T * E * 4) ||
      overlaps(out, out_bytes, w13, w13_bytes) || overlaps(out, out_bytes, w2, w2_bytes) ||
      overlaps(out, out_bytes, w13_scale, w13_bytes / 32) ||
      overlaps(out, out_bytes, w2_scale, w2_bytes / 32) ||
      overlaps(out, out_bytes, workspace, L.total))
    return MOE_ERR_ALIAS;
  char* ws = (char*)workspace;
  int32_t* ids = (int32_t*)(ws + L.off[MOE_TAP_TOPK_IDS]);
  float* tw = (float*)(ws + L.off[MOE_TAP_TOPK_WEIGHTS]);
  int32_t* sorted = (int32_t*)(ws + L.off[MOE_TAP_SORTED_IDS]);
  int32_t* eids = (int32_t*)(ws + L.off[MOE_TAP_EXPERT_IDS]);
  int32_t* ntpp = (int32_t*)(ws + L.off[MOE_TAP_NTPP]);
  int32_t* ppos = (int32_t*)(ws + L.off[MOE_TAP_PAIR_POS]);
  uint8_t* xq = (uint8_t*)(ws + L.off[MOE_TAP_XQ]);
  uint8_t* xe = (uint8_t*)(ws + L.off[MOE_TAP_XS]);
  uint8_t* aq = (uint8_t*)(ws + L.off[MOE_TAP_AQ]);
  uint8_t* ae = (uint8_t*)(ws + L.off[MOE_TAP_AS]);
  uint16_t* y = (uint16_t*)(ws + L.off[MOE_TAP_Y]);
  void* scratch = ws + L.off[MOE_TAP_ALIGN_SCRATCH];
  const int P = T * top_k;
  const int nblk = (int)(L.cap / L.BM);
  if (moe::launch_topk_softmax(router_logits, T, E, top_k, renormalize, 1, 1, ids, tw, stream))
    return MOE_ERR_HIP;
  if (moe::launch_align(ids, nullptr, 0, P, E, L.BM, sorted, eids, ntpp, ppos, scratch, stream))
    return MOE_ERR_HIP;
  if (moe::launch_group_quant_fmt(x, T, H, 32, moe::kScaleUe8m0, xq, xe, stream)) return MOE_ERR_HIP;
  const int32_t* eoff = moe::align_expert_offsets(scratch, P, E);
  if (moe::launch_gemm1_mx(xq, xe, w13, w13_scale, sorted, eids, ntpp, eoff, E, H, I, P, top_k,
                           L.BM, nblk, aq, ae, stream))
    return MOE_ERR_HIP;
  if (moe::launch_gemm2_mx(aq, ae, w2, w2_scale, sorted, eids, ntpp, eoff, E, H, I, P, L.BM, nblk, y,
                           (int)y_stride(H), y + L.cap * y_stride(H), stream))
    return MOE_ERR_HIP;
  if (moe::launch_combine(y, (int)y_stride(H), ppos, tw, T, H, top_k, (uint16_t*)out, stream))
    return MOE_ERR_HIP;
  return MOE_OK;
}

int per_token_group_quant_fp8(const void* x, int M, int K, int group_size, uint8_t* q,
                              float* scales, hipStream_t stream) {
  if (group_size != MOE_QUANT_GROUP) return MOE_ERR_UNSUPPORTED;
  if (M < 0 || K < 128 || K % 128) return MOE_ERR_SHAPE;
  if ((long long)M * K > (1LL << 40)) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_NULL;
  if ((uintptr_t)x % 16 || (uintptr_t)q % 8 || (uintptr_t)scales % 4) return MOE_ERR_UNSUPPORTED;
  const size_t n = (size_t)M * K;
  if (overlaps(q, n, x, 2 * n) || overlaps(scales, n / 128 * 4, x, 2 * n) ||
      overlaps(q, n, scales, n / 128 * 4))
    return MOE_ERR_ALIAS;
  return moe::launch_group_quant(x, M, K, q, scales, stream) ? MOE_ERR_HIP : MOE_OK;
}

int per_token_group_quant_fp8_fmt(const void* x, int M, int K, int group_size, int scale_format,
                                  uint8_t* q, void* scales, hipStream_t stream) {
  if (group_size != 32 && group_size != 128) return MOE_ERR_UNSUPPORTED;
  if (scale_format < MOE_SCALE_FLOAT32 || scale_format > MOE_SCALE_UE8M0)
    return MOE_ERR_UNSUPPORTED;
  if (M < 0 || K < group_size || K % group_size) return MOE_ERR_SHAPE;
  if ((long long)M * K > (1LL << 40)) return MOE_ERR_SHAPE;
  if (M == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_NULL;
  const size_t sb = scale_format == MOE_SCALE_UE8M0 ? 1 : 4;
  if ((uintptr_t)x % 16 || (uintptr_t)q % 8 || (uintptr_t)scales % sb) return MOE_ERR_UNSUPPORTED;
  const size_t n = (size_t)M * K, ns = n / group_size * sb;
  if (overlaps(q, n, x, 2 * n) || overlaps(scales, ns, x, 2 * n) || overlaps(q, n, scales, ns))
    return MOE_ERR_ALIAS;
  return moe::launch_group_quant_fmt(x, M, K, group_size, scale_format, q, scales, stream)
             ? MOE_ERR_HIP
             : MOE_OK;
}

int moe_topk_softmax(const float* logits, int T, int E, int top_k, int renormalize,
                     int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || top_k < 1 || top_k > E || top_k > MOE_MAX_TOP_K)
    return MOE_ERR_SHAPE;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  return moe::launch_topk_softmax(logits, T, E, top_k, renormalize, 1, 1, topk_ids, topk_weights,
                                  stream)
             ? MOE_ERR_HIP
             : MOE_OK;
}

int moe_topk_softmax_grouped(const float* logits, int T, int E, int top_k, int num_expert_group,
                             int topk_group, int renormalize, int32_t* topk_ids,
                             float* topk_weights, hipStream_t stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || top_k < 1 || top_k > E || top_k > MOE_MAX_TOP_K)
    return MOE_ERR_SHAPE;
  if (renormalize != 0 && renormalize != 1) return MOE_ERR_SHAPE;
  Routing r;
  r.num_group = num_expert_group;
  r.topk_group = topk_group;
  r.e_local = E;
  const int st = check_routing(E, top_k, r);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  return moe::launch_topk_softmax(logits, T, E, top_k, renormalize, num_expert_group, topk_group,
                                  topk_ids, topk_weights, stream)
             ? MOE_ERR_HIP
             : MOE_OK;
}

size_t moe_align_scratch_bytes(int T, int top_k, int E) {
  if (T < 0 || top_k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  const long long P = (long long)T * top_k;
  if (P > (long long)MOE_MAX_TOKENS * MOE_MAX_TOP_K) return 0;
  return moe::align_scratch_bytes((int)P, E);
}

int moe_align(const int32_t* topk_ids, int T, int top_k, int E, int block_m, int32_t* sorted_ids,
              int32_t* expert_ids, int32_t* num_tokens_post_padded, void* scratch,
              size_t scratch_bytes, hipStream_t stream) {
  if (T < 0 || top_k < 1 || E < 1 || E > MOE_MAX_EXPERTS || top_k > E) return MOE_ERR_SHAPE;
  if ((long long)T * top_k > (long long)MOE_MAX_TOKENS * MOE_MAX_TOP_K) return MOE_ERR_SHAPE;
  if (block_m < 16 || block_m > 256 || (block_m & (block_m - 1))) return MOE_ERR_SHAPE;
  if (!sorted_ids || !expert_ids || !num_tokens_post_padded || !scratch) return MOE_ERR_NULL;
  if (T > 0 && !topk_ids) return MOE_ERR_NULL;
  const int P = T * top_k;
  if (scratch_bytes < moe::align_scratch_bytes(P, E) || ((uintptr_t)scratch % 4))
    return MOE_ERR_WORKSPACE;
  return moe::launch_align(topk_ids, nullptr, 0, P, E, block_m, sorted_ids, expert_ids,
                           num_tokens_post_padded, nullptr, scratch, stream)
             ? MOE_ERR_HIP
             : MOE_OK;
}

size_t moe_align_noalloc_max_scratch_bytes(void) {
  return sizeof(moe_noalloc::scratch);
}

int moe_align_noalloc(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                      hipStream_t stream) {
  if (T < 0 || top_k < 1 || E < 1 || E > MOE_MAX_EXPERTS || top_k > E) return MOE_ERR_SHAPE;
  if ((long long)T * top_k > (long long)MOE_MAX_TOKENS * MOE_MAX_TOP_K) return MOE_ERR_SHAPE;
  if (block_m < 16 || block_m > 256 || (block_m & (block_m - 1))) return MOE_ERR_SHAPE;
  if (!sorted_ids || !expert_ids || !num_tokens_post_padded) return MOE_ERR_NULL;
  if (T > 0 && !topk_ids) return MOE_ERR_NULL;
  const int P = T * top_k;
  if (moe::align_scratch_bytes(P, E) > sizeof(moe_noalloc::scratch)) return MOE_ERR_SCRATCH;
  if (stream) {            // the scratch looked up must be the stream's device's copy
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess)
      return MOE_ERR_HIP;
    if (cur != sdev) return MOE_ERR_UNSUPPORTED;
  }
  void* scratch = nullptr;
  const int st = moe_noalloc::scratch_on_current_device(&scratch);
  if (st != MOE_OK) return st;
  // the kernels write every scratch word they read (counts, then bases and
  // offsets), so nothing is cleared between calls
  return moe::launch_align(topk_ids, nullptr, 0, P, E, block_m, sorted_ids, expert_ids,
                           num_tokens_post_padded, nullptr, scratch, stream)
             ? MOE_ERR_HIP
             : MOE_OK;
}

size_t fp8_block_linear_workspace_bytes(int M, int N, int K) {
  if (check_linear_shape(M, N, K) != MOE_OK) return 0;
  LinearLayout L;
  make_linear_layout(M, N, K, L);
  return L.total;
}

int fp8_block_linear(const void* x, const uint8_t* w, const float* w_scale, int M, int N, int K,
                     void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_linear_shape(M, N, K);
  if (st != MOE_OK) return st;
  if (!x || !w || !w_scale || !out || !workspace) return MOE_ERR_NULL;
  if ((uintptr_t)x % 16 || (uintptr_t)w % 16 || (uintptr_t)w_scale % 4 || (uintptr_t)out % 16 ||
      (uintptr_t)workspace % kAlign)
    return MOE_ERR_UNSUPPORTED;
  LinearLayout L;
  make_linear_layout(M, N, K, L);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  const size_t xb = (size_t)M * K * 2, ob = (size_t)M * N * 2;
  const size_t wb = (size_t)N * K, sb = (size_t)(N / 128) * (K / 128) * 4;
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, w, wb) || overlaps(out, ob, w_scale, sb) ||
      overlaps(workspace, L.total, x, xb) || overlaps(workspace, L.total, w, wb) ||
      overlaps(workspace, L.total, w_scale, sb) || overlaps(workspace, L.total, out, ob))
    return MOE_ERR_ALIAS;
  char* ws = (char*)workspace;
  uint8_t* xq = (uint8_t*)(ws + L.xq);
  float* xs = (float*)(ws + L.xs);
  int32_t* sorted = (int32_t*)(ws + L.sorted);
  int32_t* eids = (int32_t*)(ws + L.eids);
  int32_t* eoff = (int32_t*)(ws + L.meta);
  int32_t* ntpp = eoff + 2;
  uint16_t* dump = (uint16_t*)(ws + L.dump);
  float* part = (float*)(ws + L.part);
  if (moe::launch_group_quant(x, M, K, xq, xs, stream)) return MOE_ERR_HIP;
  if (moe::launch_identity_layout(M, L.BM, L.nblk, sorted, eids, eoff, ntpp, stream)) return MOE_ERR_HIP;
  if (moe::launch_gemm2_bounded(xq, xs, w, w_scale, sorted, eids, ntpp, eoff, N, K, M, L.BM, L.nblk,
                                (uint16_t*)out, N, M, N, dump, L.ksplit, part, false, stream))
    return MOE_ERR_HIP;
  return MOE_OK;
}

// The MXFP8 linear reuses the dense layout: the activation scale region holds
// cap * K/128 floats, i.e. exactly the cap * K/32 exponent bytes.
size_t mxfp8_linear_workspace_bytes(int M, int N, int K) {
  if (check_linear_shape(M, N, K) != MOE_OK || K < 256) return 0;
  LinearLayout L;
  make_linear_layout(M, N, K, L);
  return L.total;
}

int mxfp8_linear(const void* x, const uint8_t* w, const uint8_t* w_scale, int M, int N, int K,
                 void* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_linear_shape(M, N, K);
  if (st != MOE_OK) return st;
  if (K < 256) return MOE_ERR_UNSUPPORTED;
  if (!x || !w || !w_scale || !out || !workspace) return MOE_ERR_NULL;
  if ((uintptr_t)x % 16 || (uintptr_t)w % 16 || (uintptr_t)w_scale % 4 || (uintptr_t)out % 16 ||
      (uintptr_t)workspace % kAlign)
    return MOE_ERR_UNSUPPORTED;
  LinearLayout L;
  make_linear_layout(M, N, K, L);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  const size_t xb = (size_t)M * K * 2, ob = (size_t)M * N * 2;
  const size_t wb = (size_t)N * K, sb = (size_t)N * (K / 32);
  if (overlaps(out, ob, x, xb) || overlaps(out, ob, w, wb) || overlaps(out, ob, w_scale, sb) ||
      overlaps(workspace, L.total, x, xb) || overlaps(workspace, L.total, w, wb) ||
      overlaps(workspace, L.total, w_scale, sb) || overlaps(workspace, L.total, out, ob))
    return MOE_ERR_ALIAS;
  char* ws = (char*)workspace;
  uint8_t* xq = (uint8_t*)(ws + L.xq);
  uint8_t* xe = (uint8_t*)(ws + L.xs);
  int32_t* sorted = (int32_t*)(ws + L.sorted);
  int32_t* eids = (int32_t*)(ws + L.eids);
  int32_t* eoff = (int32_t*)(ws + L.meta);
  int32_t* ntpp = eoff + 2;
  uint16_t* dump = (uint16_t*)(ws + L.dump);
  float* part = (float*)(ws + L.part);
  if (moe::launch_group_quant_fmt(x, M, K, 32, moe::kScaleUe8m0, xq, xe, stream)) return MOE_ERR_HIP;
  if (moe::launch_identity_layout(M, L.BM, L.nblk, sorted, eids, eoff, ntpp, stream)) return MOE_ERR_HIP;
  if (moe::launch_gemm2_bounded(xq, (const float*)xe, w, (const float*)w_scale, sorted, eids, ntpp,
                                eoff, N, K, M, L.BM, L.nblk, (uint16_t*)out, N, M, N, dump,
                                L.ksplit, part, true, stream))
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_mfma_rate_probe(int kind, int iters, int nblocks, float* sink, hipStream_t stream) {
  if (kind != 0 && kind != 1) return MOE_ERR_UNSUPPORTED;
  if (iters < 1 || nblocks < 1 || nblocks > (1 << 20)) return MOE_ERR_SHAPE;
  if (!sink) return MOE_ERR_NULL;
  if ((uintptr_t)sink % 4) return MOE_ERR_UNSUPPORTED;
  return moe::launch_mfma_probe(kind, iters, nblocks, sink, stream) ? MOE_ERR_HIP : MOE_OK;
}

int moe_hbm_read_probe(const void* src, size_t bytes, int nblocks, uint32_t* sink,
                       hipStream_t stream) {
  if (bytes == 0 || bytes % 16 || nblocks < 1 || nblocks > (1 << 20)) return MOE_ERR_SHAPE;
  if (!src || !sink) return MOE_ERR_NULL;
  if ((uintptr_t)src % 16 || (uintptr_t)sink % 4) return MOE_ERR_UNSUPPORTED;
  return moe::launch_hbm_read_probe(src, bytes, nblocks, sink, stream) ? MOE_ERR_HIP : MOE_OK;
}

}  // extern "C"
