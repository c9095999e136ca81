"""CPU oracle for the fused FP8 block-quantized MoE layer forward.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, literal NumPy
definition of what the GPU path computes.  It exists to check the HIP
library, and nothing in the product may import it: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code, table or constant generator with the HIP
library under ``fp8_block_quantized_amd/``, and it never reads anything
that library produced.

Sources (the vLLM pages on quantization and MoE optimisations):
  * "Quantization and MoE Optimizations" (DeepWiki-style overview), sections
    "FusedMoE Class" (w13 gate+up and w2 stored [num_experts, N, K], a top-K
    router), "Modular Kernel Architecture" (quantize, dispatch, permute ->
    GEMM -> unpermute, gather), "Triton Fused MoE Kernel" (sorted-token
    blocks of BLOCK_SIZE_M rows per expert, float32 dequant after the
    accumulation, then the router-weight multiply) and "Weight Scale
    Granularities" (2-D BLOCK scales, GROUP scales of 128 elements).
  * "vllm.model_executor.layers.fused_moe.oracle.fp8" API page:
    ``make_fp8_moe_quant_config`` (block_shape, per-token activation
    scales) and the quant keys for dynamic 128-group activations with
    static 128-block weights, symmetric.
  * overview page, "W8A8BlockFp8LinearOp - Block FP8 GEMM Dispatch": the
    dense block-FP8 GEMM of DeepSeek-V3-style layers.
  * "vllm.model_executor.layers.quantization.online.nvfp4" API page,
    ``_quantize_moe_weight_to_nvfp4``: stacked (E, N, K) expert weights, an
    amax clamped below at 1e-8, scales stored as dequant multipliers.

Modules:
  e4m3    OCP FP8 E4M3 ("e4m3fn") decode / RNE-saturating encode.
  quant   per-token, per-128-group dynamic activation quantisation.
  router  softmax top-k routing with optional renormalisation.
  align   sort-and-pad of (token, slot) pairs by expert (moe_align).
  moe     the whole layer: quant -> GEMM1 -> SiLU*mul -> requant -> GEMM2 ->
          weighted combine, with weights dequantised to float64.
  linear  the dense block-FP8 linear layer (the E = 1 neighbour of the layer's
          second GEMM): quant -> block-scaled product -> bf16.

Parity status of each function is stated in its docstring; every function
here is pinned by a test in ``tests/test_oracle_*.py``.
"""
