"""Seeded synthetic workloads for the token-choice MoE layer forward.

This package only draws inputs: it holds the five named layer shapes and the
seeded generators that fill x, the gate weights, the optional per-expert logit
bias and the per-expert FFN weights.  It computes nothing of the layer itself,
so both the GPU path and the CPU oracle can take their inputs from it without
sharing any of the method's arithmetic.
"""
from .configs import MoEConfig, PRESETS, preset
from .generate import generate, subseed, expert_numpy, to_numpy

__all__ = ["MoEConfig", "PRESETS", "preset", "generate", "subseed", "expert_numpy", "to_numpy"]
