"""MoE FFN layer on AMD Instinct MI355X (gfx950): router, top-k, dispatch,
permutation, grouped SwiGLU expert GEMMs, shared experts and combine as HIP
kernels behind a C ABI (include/moe_ffn.h).  This package holds the kernels
(csrc/), their build step and a thin ctypes binding."""
from .api import (Fp8Weights, dims, moe_combine, moe_grouped_ffn, moe_grouped_ffn_fp8,
                  moe_grouped_ffn_workspace_bytes, moe_layer, moe_layer_fp8, moe_layer_noalloc, moe_layer_pipelined,
                  moe_layer_pipelined_workspace_bytes, moe_layer_single_launch, moe_layer_workspace_bytes,
                  moe_permute, moe_permute_workspace_bytes, moe_quantize_fp8, moe_route,
                  moe_route_workspace_bytes, moe_set_stage_events, quantize_ffn_fp8, workspace)
from ._lib import MoeError, MOE_FLAG_IDS_IN
