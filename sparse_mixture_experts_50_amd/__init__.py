"""Sparse Mixture-of-Experts FFN layer forward for MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of
include/moe.h (libmoe.so, built in-tree).  This package is the thin torch
binding: torch supplies device memory and streams only.
"""
from ._lib import MoeError, MoeDesc, MoeRouting, MoeWeights, lib  # noqa: F401
from .layer import (MoeLayer, Routing, Weights, make_desc,  # noqa: F401
                    moe_bias_update, moe_capacity, moe_combine,
                    moe_ffn_down, moe_ffn_up, moe_forward, moe_forward_noalloc,
                    moe_gemm_tail_split,
                    moe_gemm_variant,
                    moe_grouped_ffn, moe_permute, moe_route_dispatch,
                    moe_router_topk,
                    moe_workspace_size)

__version__ = "0.1.0"
