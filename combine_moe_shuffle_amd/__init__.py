"""MI355X-native MoE token dispatch/combine.

Four stages, each a hand-written HIP kernel for gfx950 behind a C ABI
(``include/moe_shuffle.h``, built into ``libmoe_shuffle.so`` in this package):

  moe_shuffle              top-k routing + stable counting sort of the
                           (token, expert) pairs by expert
  moe_gather_scale[_quant] expert-ordered gather of token rows times their
                           router score, bf16 or FP8-E4M3 rowwise
  moe_scatter_add          deterministic fp32 combine back to token order
  moe_finalize_rmsnorm     weighted top-k reduction + shared-expert add +
                           RMSNorm, with optional MXFP8 output

``combine_moe_shuffle_amd.ops`` holds the torch-tensor bindings (argument
marshalling only). Nothing is loaded at import; the first op call loads the
library and raises if it is missing.
"""
__all__ = ["ops", "workloads"]
