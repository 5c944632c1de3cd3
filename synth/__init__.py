"""Seeded synthetic inputs for the paged-expert MoE layer.

Expert weights (fp32 N(0, 0.02^2) draws, rounded to bf16 or quantised to
128x128 block-e4m3 / group-128 int4), E-wide routed top-k ids and router
weights, and bf16 hidden states.  Everything is a pure function of
(seed, workload, layer, expert | step).

Both the GPU library's tests and benchmark and the CPU oracle draw their
inputs from here.  The module holds none of the method's arithmetic: no
expert FFN, no dequantisation, no residency planning.
"""
from .workloads import WORKLOADS, Workload, workload
from .gen import (
    expert_key,
    expert_draws,
    expert_tensors,
    hidden_states,
    decode_routing,
    prefill_routing,
    router_weights,
    routing_for,
    normal,
    round_bf16,
    f16_from_f32,
    e4m3_from_f32,
)

__all__ = [
    "WORKLOADS", "Workload", "workload", "expert_key", "expert_draws", "expert_tensors",
    "hidden_states", "decode_routing", "prefill_routing", "router_weights", "routing_for",
    "normal", "round_bf16", "f16_from_f32", "e4m3_from_f32",
]
