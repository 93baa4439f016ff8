"""MI355X-native DeepSeek-R1-style MoE layer: Python binding of libmoe.so.

The layer's steps are the C-ABI calls declared in include/moe.h
(moe_route, moe_permute, moe_expert_ffn, moe_combine, moe_balanced_partition,
moe_gather_rows, moe_quantize_tokens with moe_expert_ffn_gate_up_tokens, and for online rebalancing moe_count_accumulate,
moe_coactivation, moe_affinity_partition), implemented as HIP kernels for gfx950. This package only
marshals arguments; ``build()`` compiles the library with hipcc.
"""
from ._lib import (BF16, F32, FP8_E4M3, SIGMOID, SOFTMAX, EXPORTS, MoEError, lib, make_weights,
                   moe_affinity_partition, moe_balanced_partition, moe_coactivation,
                   moe_combine, moe_count_accumulate, moe_expert_ffn, moe_expert_ffn_down,
                   moe_expert_ffn_gate_up, moe_expert_ffn_gate_up_tokens, moe_expert_ffn_noalloc,
                   NOALLOC_SCRATCH_BYTES,
                   moe_expert_ffn_workspace_size, moe_gather_rows, moe_layer_fused,
                   moe_layer_fused_workspace_size, moe_permute,
                   moe_permute_workspace_size, moe_quantize_tokens, moe_route, moe_route_select,
                   moe_route_select_workspace_size)
from .layer import LayerBuffers, MoELayer


def build(verbose: bool = False) -> str:
    from .build import build as _build
    return _build(verbose)
