"""Seeded synthetic inputs for the routed MoE FFN layer (shared by the HIP path's
tests/bench and by the CPU oracle). Holds input generation only: none of the
layer's arithmetic lives here."""
from .gen import (  # noqa: F401
    WORKLOADS, Workload, workload, seed_seq, rng_for,
    bf16_bits_from_f32, x_bf16, router_logits, router_weights, expert_bias,
    expert_w4, expert_w8, layer_w4, layer_w8,
)
