"""Seeded synthetic Q/K/V workloads shaped like video-DiT self-attention calls.

This package only produces inputs and the per-workload settings; it holds none
of the attention method's arithmetic, so both the GPU path's tests and the CPU
oracle can draw from it without sharing any of the method's code.
"""
from .configs import CONFIGS, SparsePRSettings, WorkloadConfig, get_config
from .generator import bf16_round, make_head, make_inputs, make_step_inputs, token_grid

__all__ = [
    "CONFIGS", "SparsePRSettings", "WorkloadConfig", "get_config",
    "bf16_round", "make_head", "make_inputs", "make_step_inputs", "token_grid",
]
