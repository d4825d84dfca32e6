"""The five workloads, as shapes.

1. Tiny layer: x [4, 256], W [512, 256], LoRA rank 8, s = 2, AQN stage 3 of
   10 (sigma 1e-2 -> 5e-4), noise length 256.
2. Decode on a Qwen2.5-7B-shaped MLP: M = 64 rollout tokens (8 prompts x 8
   samples); fused gate/up W [37888, 3584] and down W [3584, 18944];
   weights N(0, 0.02^2) with 0.1% outliers at 20 sigma; LoRA rank 32;
   AQN stage 1 of 10.
3. Prefill on Qwen2.5-7B shapes: M = 4096 tokens (8 prompts x 512);
   fused q/k/v W [4608, 3584] and down W [3584, 18944]; LoRA rank 32;
   AQN mid-schedule (stage 5 of 10).
4. Decode sweep on Qwen2.5-32B shapes (hidden 5120, intermediate 27648,
   40 q / 8 kv heads of dim 128): 64 layers of {qkv [7168, 5120],
   o [5120, 5120], gate/up [55296, 5120], down [5120, 27648]}, M = 128
   (8 prompts x 16 samples), LoRA rank 64, AQN stage 1.
5. Qwen2.5-14B-shaped model (48 layers, hidden 5120, intermediate 13824,
   40 q / 8 kv heads of dim 128 assumed): bulk quantization of every
   linear weight, then prefill M = 16384 through one layer's o, gate, up,
   down with LoRA rank 32, AQN stage 1.
"""
from dataclasses import dataclass, field
from typing import List


@dataclass(frozen=True)
class LayerShape:
    name: str
    n: int            # output features
    k: int            # input features


@dataclass
class Workload:
    name: str
    m: int
    r: int
    stage: int
    layers: List[LayerShape] = field(default_factory=list)
    n_layers: int = 1
    outlier_frac: float = 0.0
    lora_scale: float = 2.0
    num_stages: int = 10
    sigma_start: float = 1e-2
    sigma_end: float = 5e-4


CONFIGS = {
    "tiny": Workload("tiny", m=4, r=8, stage=3,
                     layers=[LayerShape("linear", 512, 256)]),
    "decode_7b_mlp": Workload(
        "decode_7b_mlp", m=64, r=32, stage=1, outlier_frac=1e-3,
        layers=[LayerShape("gate_up", 37888, 3584),
                LayerShape("down", 3584, 18944)]),
    "prefill_7b": Workload(
        "prefill_7b", m=4096, r=32, stage=5,
        layers=[LayerShape("qkv", 4608, 3584),
                LayerShape("down", 3584, 18944)]),
    "decode_32b_sweep": Workload(
        "decode_32b_sweep", m=128, r=64, stage=1, n_layers=64,
        layers=[LayerShape("qkv", 7168, 5120), LayerShape("o", 5120, 5120),
                LayerShape("gate_up", 55296, 5120),
                LayerShape("down", 5120, 27648)]),
    "quantize_prefill_14b": Workload(
        "quantize_prefill_14b", m=16384, r=32, stage=1, n_layers=48,
        layers=[LayerShape("q", 5120, 5120), LayerShape("k", 1024, 5120),
                LayerShape("v", 1024, 5120), LayerShape("o", 5120, 5120),
                LayerShape("gate", 13824, 5120),
                LayerShape("up", 13824, 5120),
                LayerShape("down", 5120, 13824)]),
}
