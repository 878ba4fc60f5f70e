"""DeepSeekMoE layer forward on MI355X (gfx950): FP8 block-scaled experts,
sigmoid + bias group-limited routing, behind the C ABI of libmoe_fp8.so."""
from . import _lib  # noqa: F401
from ._lib import (MoEError, fp8_quant_1x128, fp8_quant_128x128,  # noqa: F401
                   fp8_quant_128x1_grouped, fp8_transpose_128x128, grouped_fp8_gemm,
                   grouped_fp8_gemm_dgrad,
                   grouped_fp8_gemm_swiglu, grouped_fp8_gemm_swiglu_keep, grouped_fp8_wgrad, moe_bias_update, moe_combine,
                   moe_combine_backward, moe_permute, moe_permute_noalloc,
                   moe_permute_workspace_bytes, moe_route,
                   moe_route_scores, moe_route_workspace_bytes, moe_router_backward,
                   moe_router_backward_dense, moe_router_backward_dense_workspace_bytes,
                   moe_router_dcentroids, moe_seq_balance, moe_seq_balance_workspace_bytes,
                   swiglu_backward, swiglu_backward_grouped, wgrad_chunks)
from .layer import BackwardBuffers, Buffers, LayerShape, MoELayer  # noqa: F401
