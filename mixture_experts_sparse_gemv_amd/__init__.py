"""MI355X-native forward pass of a Mixture-of-Experts FFN layer.

The computation lives in libmoe_mi355x.so (hand-written HIP for gfx950, C ABI
declared in include/moe.h); `moe` is its thin ctypes binding."""
from . import moe
from .moe import (moe_capacity, moe_workspace_size, moe_router_topk, moe_dispatch,
                  moe_expert_ffn, moe_expert_up, moe_expert_down, moe_combine, moe_aux_stats,
                  moe_ffn_forward, make_problem, make_weights, workspace, MoeError)

__all__ = ["moe", "moe_capacity", "moe_workspace_size", "moe_router_topk", "moe_dispatch",
           "moe_expert_ffn", "moe_expert_up", "moe_expert_down", "moe_combine", "moe_aux_stats",
           "moe_ffn_forward", "make_problem", "make_weights", "workspace", "MoeError"]
