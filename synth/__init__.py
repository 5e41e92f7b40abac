"""Seeded synthetic inputs for the one-GPU share of an expert-parallel MoE layer.

This package is the only code shared by the CPU oracle and the GPU path. It
draws random numbers and lays them out; it contains none of the layer's
arithmetic (no routing, layout, expert FFN or combine).
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    Config,
    get_config,
    make_inputs,
    make_routing_inputs,
    make_x,
    make_expert_weights,
    tiny_config,
)
