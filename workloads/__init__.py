"""Seeded synthetic workloads for the MoE layer with zero-computation experts.

This package only draws random tensors of the right shapes and distributions.
It holds none of the layer's arithmetic (no routing, no softmax, no FFN), so it
can feed both the fp64 oracle and the HIP library without coupling them.
"""
from .configs import WORKLOADS, Workload, get_workload
from .gen import make_inputs, make_expert_weights, expert_seed, make_upstream_grad

__all__ = ["WORKLOADS", "Workload", "get_workload", "make_inputs", "make_upstream_grad",
           "make_expert_weights", "expert_seed"]
