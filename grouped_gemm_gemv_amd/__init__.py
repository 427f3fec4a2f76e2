"""MI355X-native single-GPU MoE layer forward pass (libmoe + thin binding).

The HIP library is loaded on first use; importing the package does not touch
the GPU.
"""
from .api import (
    Dispatch,
    ForwardViews,
    Shape,
    moe_combine,
    moe_ffn_down,
    moe_ffn_down_fp8,
    moe_ffn_gate_up_fp8,
    moe_forward_fp8,
    moe_pack_blocked16,
    LAYOUT_ROWS,
    LAYOUT_BLOCKED16,
    PASS_BOTH,
    moe_ffn_gate_up,
    moe_ffn_gate_up_gather,
    moe_forward,
    moe_forward_noalloc,
    moe_grouped_ffn,
    moe_permute,
    moe_route,
    query,
    workspace,
    workspace_size,
)

__all__ = [
    "Dispatch", "ForwardViews", "Shape", "moe_combine", "moe_ffn_down", "moe_ffn_gate_up", "moe_ffn_gate_up_gather", "moe_forward", "moe_forward_noalloc",
    "moe_ffn_gate_up_fp8", "moe_ffn_down_fp8", "moe_forward_fp8", "moe_pack_blocked16",
    "LAYOUT_ROWS", "LAYOUT_BLOCKED16", "PASS_BOTH",
    "moe_grouped_ffn", "moe_permute", "moe_route", "query", "workspace", "workspace_size",
]
