"""MI355X (gfx950) local MoE chain: route -> dispatch -> SwiGLU experts -> combine, and its backward.

The compute lives in libmoe.so (HIP kernels behind the C ABI of
include/moe.h); this package is a thin torch-facing binding.
"""
from ._lib import EXPORTS, LIB_PATH, MoeError, load
from .api import (DispatchedTokens, ExpertsCache, GroupRoutingOptions, RouterTrainingPlan, RouterWeightOptions,
                  RoutingOptions, RoutingPlan, SwiGluExperts, combine, combine_backward, dispatch, dispatch_backward,
                  route, route_sigmoid_grouped, router_backward, router_weights)

__all__ = [
    "DispatchedTokens", "GroupRoutingOptions", "RoutingOptions", "RoutingPlan", "SwiGluExperts", "MoeError",
    "route", "route_sigmoid_grouped", "dispatch", "combine", "load", "EXPORTS", "LIB_PATH",
    "ExpertsCache", "RouterTrainingPlan", "RouterWeightOptions", "combine_backward", "dispatch_backward",
    "router_backward", "router_weights",
]
