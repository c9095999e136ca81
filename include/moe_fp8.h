/*
 * moe_fp8.h - C ABI of the MI355X (gfx950) fused FP8 block-quantized MoE
 * layer forward and its stages.
 *
 * The operation is the fused MoE layer of the vLLM pages on quantization and
 * MoE optimisations:
 *   - overview page, "FusedMoE Class": experts w13 (gate+up) and w2 (down)
 *     stored [num_experts, N, K], a top-K router in front;
 *   - overview page, "Modular Kernel Architecture": quantize the inputs,
 *     permute -> expert GEMMs -> unpermute, gather the results;
 *   - overview page, "Triton Fused MoE Kernel": blocks of BLOCK_SIZE_M
 *     sorted tokens that all belong to one expert; float32 dequantisation of
 *     the quantized accumulation, then the router-weight multiply;
 *   - fp8 oracle API page, make_fp8_moe_quant_config / quant keys: static
 *     128x128 block weight scales (block_shape [128, 128]) and dynamic
 *     per-token 128-group activation scales, symmetric, so no activation
 *     scale is an input.
 * The activation between the GEMMs is SiLU(gate) * up, requantised per token
 * and 128-group before the second GEMM; routing is softmax top-k with
 * optional renormalisation.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *     contiguous.  bf16 tensors are passed as const void* (raw 16-bit
 *     bfloat16 words).  FP8 tensors hold OCP e4m3fn codes, one byte each.
 *   - Scales are float32 dequant multipliers: value = dec(code) * scale.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without synchronising.  The library allocates no device memory
 *     and keeps no mutable global state (the one exception is the fixed
 *     per-GPU scratch of moe_align_noalloc, described there); calls on
 *     different streams with disjoint outputs and workspaces may run
 *     concurrently.
 *   - Arguments are validated on the host before anything is launched; a
 *     negative moe_status is returned on error and nothing is enqueued.  A
 *     launch failure reported by the HIP runtime returns MOE_ERR_HIP.  On any
 *     error the contents of the outputs are unspecified.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is out of range or not a multiple of 128 */
  MOE_ERR_UNSUPPORTED = -3, /* a valid request this library does not serve */
  MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_fp8_workspace_bytes() */
  MOE_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
  MOE_ERR_ALIAS = -6,       /* an output overlaps an input or the workspace */
  MOE_ERR_SCRATCH = -7      /* the request exceeds the fixed scratch of a scratch-free entry point */
} moe_status;

/* Limits.  H and I must be multiples of 128 (the weight block and activation
 * group), 1 <= top_k <= E <= MOE_MAX_EXPERTS, 1 <= T <= MOE_MAX_TOKENS (the
 * fused-MoE activation chunk of the overview page's environment-variable
 * table is 16384 tokens; one call covers one such chunk). */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOKENS 16384
#define MOE_MAX_TOP_K 32
#define MOE_QUANT_GROUP 128

/* Intermediate tensors inside the forward's workspace, for inspection by
 * tests (offsets from moe_fp8_workspace_layout, in bytes). */
enum {
  MOE_TAP_TOPK_IDS = 0,     /* int32 [T, top_k] expert id per slot, descending score */
  MOE_TAP_TOPK_WEIGHTS,     /* float32 [T, top_k] routing weight per slot */
  MOE_TAP_SORTED_IDS,       /* int32 [cap] pair index p = t*top_k + j, sentinel T*top_k */
  MOE_TAP_EXPERT_IDS,       /* int32 [cap / block_m] expert of each block */
  MOE_TAP_NTPP,             /* int32 [1] number of sorted rows after padding */
  MOE_TAP_PAIR_POS,         /* int32 [T*top_k] sorted row of each pair (inverse of sorted_ids) */
  MOE_TAP_XQ,               /* uint8 [T, H] e4m3fn codes of x */
  MOE_TAP_XS,               /* float32 [T, H/128] scales of x */
  MOE_TAP_AQ,               /* uint8 [cap, I] requantised activation, sorted order */
  MOE_TAP_AS,               /* float32 [cap, I/128] its scales */
  MOE_TAP_Y,                /* bf16 [cap, roundup(H, 256)] expert output per sorted row, before
                               the routing weight (rows of padding undefined); unused when
                               the second GEMM splits K (MOE_TAP_Y_SLICES) */
  MOE_TAP_ALIGN_SCRATCH,    /* int32 scratch of the sort-and-pad stage */
  MOE_TAP_Y_SLICES,         /* float32 [S, T*top_k, roundup(H, 256)] K-slice partials of the
                               expert output per pair, summed in slice order by the combine;
                               S > 1 only for decode shapes (block_m <= 64) whose weight
                               tiles in use would leave CUs idle, else empty */
  MOE_TAP_H_SLICES,         /* float64 [S1, T*top_k, 2I] K-slice partials of the first GEMM's
                               gate and up outputs per pair, summed in slice order before
                               SiLU*mul; S1 > 1 under the same condition, else empty (with
                               S1 > 1, MOE_TAP_AQ / MOE_TAP_AS rows of padding are unwritten) */
  MOE_TAP_COUNT
};

/* Block size (BLOCK_SIZE_M: sorted rows per expert block) the forward uses
 * for this shape.  Returns a positive power of two, or a negative moe_status
 * for an invalid shape. */
int moe_fp8_block_m(int T, int H, int I, int E, int top_k);

/* Bytes of device workspace moe_fp8_forward needs for this shape (0 for an
 * invalid shape).  The workspace must be 256-byte aligned. */
size_t moe_fp8_workspace_bytes(int T, int H, int I, int E, int top_k);

/* Byte offsets of the MOE_TAP_* tensors inside the workspace.  Writes
 * MOE_TAP_COUNT entries into offsets (host memory).  Returns MOE_OK or a
 * negative moe_status. */
int moe_fp8_workspace_layout(int T, int H, int I, int E, int top_k,
                             size_t offsets[MOE_TAP_COUNT]);

/*
 * Fused FP8 block-quantized MoE layer forward (FusedMoE.forward(hidden_states,
 * router_logits) of the overview page, with the fp8 block-quant config):
 *   (ids, w) = softmax top-k of router_logits (renormalised if asked)
 *   (xq, xs) = per-token 128-group FP8 quantisation of x
 *   h = block-scaled FP8 GEMM of xq with w13[e]        e = expert of the pair
 *   a = silu(h[:, :I]) * h[:, I:], requantised per token and 128-group
 *   y = block-scaled FP8 GEMM of a with w2[e]
 *   out[t] = bf16( sum over the top_k slots of w * y )
 *
 *   x             bf16    [T, H]
 *   router_logits float32 [T, E]
 *   w13           e4m3fn  [E, 2I, H]      rows [0, I) gate, [I, 2I) up
 *   w13_scale     float32 [E, 2I/128, H/128]
 *   w2            e4m3fn  [E, H, I]
 *   w2_scale      float32 [E, H/128, I/128]
 *   renormalize   0 or 1
 *   out           bf16    [T, H]; must not overlap any input or the workspace
 *   workspace     device memory of at least moe_fp8_workspace_bytes(), 256-byte
 *                 aligned, owned by the caller; its contents on return are the
 *                 MOE_TAP_* intermediates (needs no initialisation)
 */
int moe_fp8_forward(const void* x, const float* router_logits,
                    const uint8_t* w13, const float* w13_scale,
                    const uint8_t* w2, const float* w2_scale,
                    int T, int H, int I, int E, int top_k, int renormalize,
                    void* out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * moe_fp8_forward with the routing variants of the pages:
 *   - grouped top-k (num_expert_group > 1; the overview page's environment
 *     table names a fused grouped top-K routing switch without defining it,
 *     read here in the router's own terms): the E experts form
 *     num_expert_group equal groups of consecutive ids, a group's score is its
 *     best logit, the topk_group best groups are kept (ties to the lower
 *     group), and the top_k experts are chosen among the kept groups' experts
 *     as moe_topk_softmax chooses them; the weights are the same full softmax,
 *     renormalised over the chosen slots if asked.  num_expert_group == 1
 *     (with topk_group == 1) is the plain router.
 *   - an expert map (overview page, "Expert Parallelism and Expert Maps":
 *     global expert -> local index, -1 for experts on other ranks; "Triton
 *     Fused MoE Kernel": zeros are written for blocks of absent experts):
 *     expert_map is device int32 [E]; w13, w2 and their scales hold the
 *     num_local_experts local experts; a pair routed to an expert mapped
 *     outside [0, num_local_experts) contributes zero to out, so out is this
 *     rank's share of the layer, the sum over ranks being the full layer.
 *     Routing (ids and weights, MOE_TAP_TOPK_*) is over the E global logits;
 *     MOE_TAP_EXPERT_IDS and the sorted layout are over local experts, and
 *     MOE_TAP_PAIR_POS is -1 for the pairs left out.  expert_map NULL requires
 *     num_local_experts == E.
 * Constraints: those of moe_fp8_forward, plus 1 <= num_expert_group <= 64
 * dividing E, 1 <= topk_group <= num_expert_group, top_k <= topk_group * E /
 * num_expert_group, 1 <= num_local_experts <= E, expert_map 4-byte aligned and
 * not overlapping out.  The workspace is moe_fp8_workspace_bytes(T, H, I, E,
 * top_k) with the global E (it bounds the local layout).
 */
int moe_fp8_forward_routed(const void* x, const float* router_logits,
                           const uint8_t* w13, const float* w13_scale,
                           const uint8_t* w2, const float* w2_scale,
                           int T, int H, int I, int E, int top_k, int renormalize,
                           int num_expert_group, int topk_group,
                           const int32_t* expert_map, int num_local_experts,
                           void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * The expert computation in the batched activation format (overview page,
 * "FusedMoEPermuteExpertsUnpermute Implementations": BatchedDeepGemmExperts,
 * the masked grouped GEMM of the FP8 block scheme; fp8 oracle API page, the
 * BatchedExperts activation format): the tokens are already dispatched per
 * expert, and expert e's rows [0, expert_num_tokens[e]) of x[e] are real.
 *   for every e and r < expert_num_tokens[e] (clamped to [0, max_tokens]):
 *     out[e, r] = bf16( the layer's expert steps on x[e, r] with expert e:
 *                       128-group quant, GEMM1, SiLU*mul, requant, GEMM2 )
 *   out[e, r] = 0 for the rows past the count.
 * No routing weight is applied: in this format it belongs to the finalize
 * step.  The counts stay on the device (the host never reads them), so a
 * caller can replay the call with new counts; an expert with no row costs
 * no GEMM work.
 *
 *   x                 bf16    [E, max_tokens, H]  (rows past the counts are never read)
 *   expert_num_tokens int32   [E]                 device
 *   w13, w13_scale, w2, w2_scale as in moe_fp8_forward (E experts)
 *   out               bf16    [E, max_tokens, H]; must not overlap any input
 *   workspace         moe_fp8_batched_workspace_bytes(E, max_tokens, H, I) bytes,
 *                     256-byte aligned; its MOE_TAP_* tensors are those of
 *                     moe_fp8_workspace_layout(E * max_tokens, H, I, E, 1) with
 *                     token e * max_tokens + r (the router taps are unused,
 *                     MOE_TAP_ALIGN_SCRATCH holds the expert block offsets, and
 *                     the second GEMM does not split K: no MOE_TAP_Y_SLICES)
 * Constraints: E * max_tokens <= MOE_MAX_TOKENS, E <= MOE_MAX_EXPERTS, H and I
 * multiples of 128 as in moe_fp8_forward.
 */
size_t moe_fp8_batched_workspace_bytes(int E, int max_tokens, int H, int I);
int moe_fp8_batched_experts(const void* x, const int32_t* expert_num_tokens,
                            const uint8_t* w13, const float* w13_scale,
                            const uint8_t* w2, const float* w2_scale,
                            int E, int max_tokens, int H, int I,
                            void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * The MXFP8 MoE layer forward: the fp8 oracle API page's MXFP8 quant config,
 * block shape [1, 32] with uint8 UE8M0 scales, whose activations go through
 * the MXFP8 activation quant:
 *   (ids, w) = softmax top-k of router_logits (as moe_fp8_forward)
 *   (xq, xe) = per_token_group_quant_fp8_fmt(x, group 32, MOE_SCALE_UE8M0)
 *   h = sum_k dec(xq)*2^(xe-127) * dec(w13[e])*2^(w13_scale[e]-127)   per [1, 32] block
 *   a = silu(h[:, :I]) * h[:, I:], requantised per token and 32 features with
 *       power-of-two scales (UE8M0)
 *   y = the same block-scaled product of a with w2[e]
 *   out[t] = bf16( sum over the top_k slots of w * y )
 * Both GEMMs run on FP8 MFMAs that apply the exponents in hardware
 * (float32 accumulation); the block size is moe_fp8_block_m()'s.
 *
 *   x             bf16    [T, H]
 *   router_logits float32 [T, E]
 *   w13           e4m3fn  [E, 2I, H]      rows [0, I) gate, [I, 2I) up
 *   w13_scale     uint8   [E, 2I, H/32]   UE8M0 exponent bytes (4-byte aligned)
 *   w2            e4m3fn  [E, H, I]
 *   w2_scale      uint8   [E, H, I/32]
 *   out           bf16    [T, H]; must not overlap any input or the workspace
 *   workspace     moe_fp8_mx_workspace_bytes() bytes, 256-byte aligned; its
 *                 MOE_TAP_* tensors at moe_fp8_mx_workspace_layout()'s offsets
 *                 (MOE_TAP_XS and MOE_TAP_AS hold exponent bytes [rows, K/32];
 *                 MOE_TAP_Y_SLICES is empty)
 * Constraints: those of moe_fp8_forward, and I >= 256 (else
 * MOE_ERR_UNSUPPORTED; the workspace query returns 0).
 */
size_t moe_fp8_mx_workspace_bytes(int T, int H, int I, int E, int top_k);
int moe_fp8_mx_workspace_layout(int T, int H, int I, int E, int top_k,
                                size_t offsets[MOE_TAP_COUNT]);
int moe_fp8_mx_forward(const void* x, const float* router_logits,
                       const uint8_t* w13, const uint8_t* w13_scale,
                       const uint8_t* w2, const uint8_t* w2_scale,
                       int T, int H, int I, int E, int top_k, int renormalize,
                       void* out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Stages of the forward, in launch order (for moe_fp8_forward_traced). */
enum {
  MOE_STAGE_ROUTER = 0,     /* softmax top-k */
  MOE_STAGE_ALIGN,          /* sort and pad by expert (one kernel up to 1024 pairs, else three) */
  MOE_STAGE_QUANT,          /* activation quantisation of x */
  MOE_STAGE_GEMM1,          /* w13 GEMM + SiLU*mul + requantisation (with K slices: the
                               partials' kernel and the one that finishes them) */
  MOE_STAGE_GEMM2,          /* w2 GEMM (per sorted row, or per pair as K-slice partials,
                               before the routing weight) */
  MOE_STAGE_COMBINE,        /* weighted sum over the top_k slots */
  MOE_STAGE_COUNT
};

/*
 * moe_fp8_forward, plus tracing: records events[i] on `stream` just before
 * stage i is enqueued and events[MOE_STAGE_COUNT] after the last one, so that
 * hipEventElapsedTime(events[i], events[i+1]) is the GPU time of stage i.
 * The MOE_STAGE_COUNT + 1 events are created by the caller (with timing
 * enabled).  Same kernels and arguments as moe_fp8_forward.
 */
int moe_fp8_forward_traced(const void* x, const float* router_logits,
                           const uint8_t* w13, const float* w13_scale,
                           const uint8_t* w2, const float* w2_scale,
                           int T, int H, int I, int E, int top_k, int renormalize,
                           void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, hipEvent_t events[MOE_STAGE_COUNT + 1]);

/*
 * Per-token-group dynamic FP8 activation quantisation (quant key
 * kFp8Dynamic128Sym of the fp8 oracle API page; GROUP granularity of the
 * overview page's "Weight Scale Granularities"):
 *   s[m, g] = max(max_i |x[m, 128g + i]|, 1e-8) / 448     (float32, RNE)
 *   q[m, k] = e4m3fn_RNE_saturate(x[m, k] / s[m, k / 128]) (float32 quotient)
 *
 *   x       bf16    [M, K]
 *   q       e4m3fn  [M, K]
 *   scales  float32 [M, K / group_size]
 *   group_size must be 128; K must be a positive multiple of 128; M >= 0
 *   (M == 0 enqueues nothing).
 */
int per_token_group_quant_fp8(const void* x, int M, int K, int group_size,
                              uint8_t* q, float* scales, hipStream_t stream);

/* Scale formats of per_token_group_quant_fp8_fmt (overview page, "DeepGEMM
 * Scale Formats"). */
typedef enum {
  MOE_SCALE_FLOAT32 = 0,            /* float32 s = max(amax, 1e-8) / 448 */
  MOE_SCALE_FLOAT32_CEIL_UE8M0 = 1, /* float32, that s rounded up to a power of two */
  MOE_SCALE_UE8M0 = 2               /* uint8 exponent byte e of that power: s = 2^(e - 127) */
} moe_scale_format;

/*
 * Per-token-group FP8 quantisation with a choice of group size and scale
 * format: the float32 scales of per_token_group_quant_fp8, the same scales
 * rounded up to a power of two (FLOAT32_CEIL_UE8M0 of the overview page's
 * "DeepGEMM Scale Formats"), or their UE8M0 exponent bytes (UE8M0 there; with
 * group 32 the MXFP8 [1, 32] activation quant of the fp8 oracle API page,
 * whose scales are uint8 UE8M0 values laid out [num_tokens, hidden / 32]).
 *   s32[m, g]  = max(max_i |x[m, G*g + i]|, 1e-8) / 448           (float32, RNE)
 *   s[m, g]    = s32 (FLOAT32) or the smallest power of two >= s32 (the others)
 *   q[m, k]    = e4m3fn_RNE_saturate(x[m, k] / s[m, k / G])      (float32 quotient;
 *                exact for a power-of-two s, and then never saturating)
 *   scales     float32 [M, K / G] holding s, or for MOE_SCALE_UE8M0 uint8
 *              [M, K / G] holding log2(s) + 127.  Row-major bytes are the
 *              "four per int32" packing read as little-endian int32 words
 *              (group 4w + i in byte i of word w) when K / G is a multiple of 4.
 *
 *   x  bf16 [M, K] (16-byte aligned); q e4m3fn [M, K] (8-byte aligned)
 *   group_size G is 32 or 128 (else MOE_ERR_UNSUPPORTED); K a positive
 *   multiple of G; M >= 0 (M == 0 enqueues nothing); scale_format a
 *   moe_scale_format (else MOE_ERR_UNSUPPORTED).
 */
int per_token_group_quant_fp8_fmt(const void* x, int M, int K, int group_size, int scale_format,
                                  uint8_t* q, void* scales, hipStream_t stream);

/*
 * Router stage alone (the top-K router of the overview page's "FusedMoE
 * Class"): softmax over E logits, the top_k experts by logit (ties to the
 * lower index) in descending order, weights renormalised to sum 1 if
 * renormalize.  Same kernel as inside moe_fp8_forward.
 *   logits float32 [T, E]; topk_ids int32 [T, top_k]; topk_weights float32 [T, top_k]
 */
int moe_topk_softmax(const float* logits, int T, int E, int top_k, int renormalize,
                     int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Router stage alone with grouped top-k (the routing of moe_fp8_forward_routed;
 * same kernel).  Constraints as there. */
int moe_topk_softmax_grouped(const float* logits, int T, int E, int top_k, int num_expert_group,
                             int topk_group, int renormalize, int32_t* topk_ids,
                             float* topk_weights, hipStream_t stream);

/* Bytes of int32 scratch moe_align needs for P = T*top_k pairs and E experts. */
size_t moe_align_scratch_bytes(int T, int top_k, int E);

/*
 * Sort-and-pad stage alone (the sorted-token blocks of the overview page's
 * "Triton Fused MoE Kernel"): pairs p = t*top_k + j are grouped by expert in
 * ascending p; each expert's run is padded with the sentinel T*top_k to a
 * multiple of block_m; expert_ids[b] is the expert of rows
 * [b*block_m, (b+1)*block_m); num_tokens_post_padded[0] is the padded total.
 * Only the first num_tokens_post_padded rows are defined.  Same kernels as
 * inside moe_fp8_forward.
 *   topk_ids   int32 [T, top_k] values in [0, E) (pairs with other values are
 *              left out of the layout)
 *   sorted_ids int32 [T*top_k + E*(block_m-1)] (rounded up to block_m)
 *   expert_ids int32 [that / block_m]
 *   block_m    a power of two in [16, 256]
 *   scratch    device memory of moe_align_scratch_bytes(), 256-byte aligned
 */
int moe_align(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
              int32_t* sorted_ids, int32_t* expert_ids,
              int32_t* num_tokens_post_padded,
              void* scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * moe_align without a scratch argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and outputs as
 * moe_align; the scratch is a fixed device array inside the library (one per
 * GPU, created with the library's code object and held until the process
 * ends) of moe_align_noalloc_max_scratch_bytes() bytes, about 2.1 MB: enough
 * for every shape moe_align accepts (T*top_k <= MOE_MAX_TOKENS*MOE_MAX_TOP_K,
 * E <= MOE_MAX_EXPERTS).  A request that would need more returns
 * MOE_ERR_SCRATCH.  The call allocates nothing and enqueues no memset; the
 * first call on a device looks up that device's copy of the array (the device
 * must be current, and a non-NULL stream must belong to it, else
 * MOE_ERR_UNSUPPORTED).  All calls on one GPU share its one array: calls that
 * may overlap on a GPU (on different streams, or concurrently from several
 * host threads) race on it and must be serialised by the caller.
 */
size_t moe_align_noalloc_max_scratch_bytes(void);
int moe_align_noalloc(const int32_t* topk_ids, int T, int top_k, int E, int block_m,
                      int32_t* sorted_ids, int32_t* expert_ids,
                      int32_t* num_tokens_post_padded, hipStream_t stream);

/*
 * Dense block-FP8 linear layer (overview page, "W8A8BlockFp8LinearOp - Block
 * FP8 GEMM Dispatch": the block-wise FP8 GEMM of DeepSeek-V3-style dense
 * layers, with the weights on the MFMA's M side for small token counts as the
 * section's swapAB path does; scales as in "Weight Scale Granularities": a
 * dynamic 128-group scale per token row, a static scale per 128x128 weight
 * block):
 *   (xq, xs) = per_token_group_quant_fp8(x)
 *   out[m, n] = bf16_RNE( sum_kb xs[m, kb] * w_scale[n/128, kb]
 *                          * sum_{k in kb} dec(xq[m, k]) * dec(w[n, k]) )
 * accumulated in float32 on FP8 MFMAs (the E = 1 case of the second grouped
 * GEMM).
 *
 *   x        bf16    [M, K]          device, 16-byte aligned
 *   w        e4m3fn  [N, K]          device, row-major (one output per row)
 *   w_scale  float32 [N/128, K/128]  device, dequantisation multipliers
 *   out      bf16    [M, N]          device, must not overlap any input
 *   workspace: fp8_block_linear_workspace_bytes(M, N, K) bytes, 256-byte
 *   aligned, caller-owned, contents undefined on return.
 * Constraints: 1 <= M <= 2^20; N and K positive multiples of 128, each
 * <= 65536, N*K < 2^31.  Returns MOE_OK or a negative moe_status (checked
 * before anything is enqueued); out is undefined on error.
 */
size_t fp8_block_linear_workspace_bytes(int M, int N, int K);
int fp8_block_linear(const void* x, const uint8_t* w, const float* w_scale, int M, int N, int K,
                     void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MXFP8 dense linear layer: the block shape [1, 32] of the fp8 oracle API
 * page (activations quantised by the MXFP8 activation quant, uint8 UE8M0
 * scales [num_tokens, hidden / 32]), with the weight in the same format (an
 * MXFP8 checkpoint: e4m3fn codes and one UE8M0 exponent byte per row and 32
 * K elements; overview page, "DeepGEMM Scale Formats", UE8M0):
 *   (xq, xe) = per_token_group_quant_fp8_fmt(x, group 32, MOE_SCALE_UE8M0)
 *   out[m, n] = bf16_RNE( sum_k dec(xq[m, k]) * 2^(xe[m, k/32] - 127)
 *                               * dec(w[n, k]) * 2^(w_scale[n, k/32] - 127) )
 * accumulated in float32 by FP8 MFMAs that apply both exponents in hardware.
 *
 *   x        bf16    [M, K]          device, 16-byte aligned
 *   w        e4m3fn  [N, K]          device, 16-byte aligned, one output per row
 *   w_scale  uint8   [N, K/32]       device, 4-byte aligned, UE8M0 bytes (255 is NaN)
 *   out      bf16    [M, N]          device, must not overlap any input
 *   workspace: mxfp8_linear_workspace_bytes(M, N, K) bytes, 256-byte aligned,
 *   caller-owned, contents undefined on return.
 * Constraints: those of fp8_block_linear, and K >= 256 (K == 128 returns
 * MOE_ERR_UNSUPPORTED; the workspace query returns 0).  Returns MOE_OK or a
 * negative moe_status (checked before anything is enqueued).
 */
size_t mxfp8_linear_workspace_bytes(int M, int N, int K);
int mxfp8_linear(const void* x, const uint8_t* w, const uint8_t* w_scale, int M, int N, int K,
                 void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Matrix-core rate probe, a measurement aid (not a step of the layer): the
 * roofline fractions of the GEMMs are quoted against MI355X's published
 * dense peaks, and this gives the rate the part actually sustains for the
 * two MFMA types the GEMMs issue.  nblocks workgroups of 4 waves each run
 * iters rounds of 8 independent accumulator chains of one instruction:
 *   kind 0: v_mfma_f32_16x16x32_f16 (first GEMM), 16384 flops each;
 *   kind 1: v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 x e4m3 with unit scales
 *           (second GEMM), 65536 flops each.
 * So one call performs nblocks * 4 * iters * 8 instructions.  Operands live
 * in registers; the only memory access is one float32 store per thread to
 * sink [nblocks * 256] (device, 4-byte aligned, caller-owned; contents
 * meaningless).  Returns MOE_OK, MOE_ERR_UNSUPPORTED for another kind,
 * MOE_ERR_SHAPE unless iters >= 1 and 1 <= nblocks <= 2^20, MOE_ERR_NULL
 * for a null sink, MOE_ERR_HIP if the launch fails.
 */
int moe_mfma_rate_probe(int kind, int iters, int nblocks, float* sink, hipStream_t stream);

/*
 * HBM read-stream probe, a measurement aid (not a step of the layer): the
 * decode-sized GEMMs stream their weights and write almost nothing, so the
 * rate HBM delivers to a pure read stream is the ceiling they are measured
 * against beside the published 8 TB/s.  nblocks workgroups of 256 threads
 * read src (bytes, a multiple of 16; 16-byte aligned) once in a grid-stride
 * loop of 16-byte loads and store the XOR of each thread's 32-bit words to
 * sink[thread] (uint32 [nblocks * 256], device, 4-byte aligned, caller-owned):
 * the XOR of all of sink equals the XOR of all 32-bit words of src.
 * Returns MOE_OK, MOE_ERR_SHAPE (bytes 0 or not a multiple of 16, nblocks
 * outside [1, 2^20]), MOE_ERR_NULL, MOE_ERR_UNSUPPORTED (misaligned) or
 * MOE_ERR_HIP.
 */
int moe_hbm_read_probe(const void* src, size_t bytes, int nblocks, uint32_t* sink,
                       hipStream_t stream);

/* Static description of a moe_status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
