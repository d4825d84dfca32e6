"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package holds none of the method's arithmetic: it only draws random
tensors with the shapes, distributions and structure of the workloads
(Qwen2.5-shaped layers, N(0, 1) activations, N(0, 0.02^2) weights with
sparse 20-sigma outliers, LoRA factors, AQN stages) and rounds the fp32
draws to bf16 bit patterns, which is how the inputs reach both sides.
"""
from .synth import (bf16_from_f32, normal_bf16, weight_bf16, lora_factors, norm_inputs,
                    LayerInputs, make_layer)
from .configs import CONFIGS, LayerShape, Workload

__all__ = ["bf16_from_f32", "normal_bf16", "weight_bf16", "lora_factors", "norm_inputs",
           "LayerInputs", "make_layer", "CONFIGS", "LayerShape", "Workload"]
