"""Seeded synthetic inputs for the routed MoE FFN layer.

This package only draws and stores inputs (activations, router weight, expert
weights and their per-channel scales). It holds none of the layer's arithmetic:
both the HIP path and the CPU oracle consume what it produces.
"""
from .gen import (CONFIGS, MoEConfig, Workload, generate, shrink, to_bits,
                  ZIPF_ALPHA, host_expert, host_shared, router_inputs)

__all__ = ["CONFIGS", "MoEConfig", "Workload", "generate", "shrink", "to_bits",
           "ZIPF_ALPHA", "host_expert", "host_shared", "router_inputs"]
