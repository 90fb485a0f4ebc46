"""MI355X (gfx950) local MoE forward chain: route -> dispatch -> SwiGLU experts -> combine.

The compute lives in libmoe.so (HIP kernels behind the C ABI of
include/moe.h); this package is a thin torch-facing binding.
"""
from ._lib import EXPORTS, LIB_PATH, MoeError, load
from .api import (DispatchedTokens, GroupRoutingOptions, RoutingOptions, RoutingPlan, SwiGluExperts, combine,
                  dispatch, route, route_sigmoid_grouped)

__all__ = [
    "DispatchedTokens", "GroupRoutingOptions", "RoutingOptions", "RoutingPlan", "SwiGluExperts", "MoeError",
    "route", "route_sigmoid_grouped", "dispatch", "combine", "load", "EXPORTS", "LIB_PATH",
]
