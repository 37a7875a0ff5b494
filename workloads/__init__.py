"""Seeded synthetic inputs shaped like the video-DiT attention workloads.

This package holds only input generation: configuration records and seeded
Q/K/V tensors.  It contains none of the block-sparse attention arithmetic, so
both the CPU oracle and the GPU path can read the same inputs without sharing
any of the method's code.
"""
from .configs import CONFIGS, Config, get_config
from .generate import make_inputs, bf16_round, bf16_bits_to_f32, positional_term

__all__ = ["CONFIGS", "Config", "get_config", "make_inputs", "bf16_round",
           "bf16_bits_to_f32", "positional_term"]
