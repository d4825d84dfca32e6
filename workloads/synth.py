"""Seeded tensor generators (numpy, CPU).

Every tensor is drawn in fp32 from numpy's PCG64 generator seeded with an
explicit integer and rounded to bf16 (round to nearest even) as uint16 bit
patterns.  The same seed always gives the same bits on every machine.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


def bf16_from_f32(x):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def normal_bf16(shape, std, seed):
    rng = np.random.default_rng(seed)
    return bf16_from_f32(rng.standard_normal(shape, dtype=np.float32)
                         * np.float32(std))


def weight_bf16(n, k, std, seed, outlier_frac=0.0, outlier_sigmas=20.0):
    """W [n, k] ~ N(0, std^2); a fraction of positions (uniform, without
    replacement) replaced by +-outlier_sigmas*std with random sign."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    if outlier_frac > 0.0:
        count = int(round(outlier_frac * n * k))
        pos = rng.choice(n * k, size=count, replace=False)
        sign = np.where(rng.integers(0, 2, size=count) == 1, 1.0, -1.0)
        w.reshape(-1)[pos] = (sign * outlier_sigmas * std).astype(np.float32)
    return bf16_from_f32(w)


def lora_factors(n, k, r, seed, std_a=0.02, std_b=0.01):
    """LoRA A [r, k] ~ N(0, std_a^2) and B [n, r] ~ N(0, std_b^2)."""
    a = normal_bf16((r, k), std_a, seed)
    b = normal_bf16((n, r), std_b, seed + 1)
    return a, b


@dataclass
class LayerInputs:
    x: np.ndarray              # uint16 [m, k] bf16 bits
    w: np.ndarray              # uint16 [n, k] bf16 bits
    a: Optional[np.ndarray]    # uint16 [r, k] or None
    b: Optional[np.ndarray]    # uint16 [n, r] or None
    lora_scale: float
    stage: int                 # AQN stage k (0 = no noise)
    seed: int                  # noise key
    stream_id: int
    call_id: int


def make_layer(m, n, k, r, seed, w_std=0.02, outlier_frac=0.0,
               lora_scale=2.0, stage=1, stream_id=0, call_id=0):
    """One linear layer's inputs; per-tensor seeds are 1000*seed + index."""
    base = 1000 * int(seed)
    x = normal_bf16((m, k), 1.0, base + 0)
    w = weight_bf16(n, k, w_std, base + 1, outlier_frac=outlier_frac)
    if r > 0:
        a, b = lora_factors(n, k, r, base + 2)
    else:
        a = b = None
    return LayerInputs(x=x, w=w, a=a, b=b, lora_scale=float(lora_scale),
                       stage=int(stage), seed=int(seed),
                       stream_id=int(stream_id), call_id=int(call_id))


def norm_inputs(m, d, seed, w_mean=1.0, w_std=0.05):
    """Inputs of the noisy RMSNorm: x [m, d] ~ N(0, 1) and the RMSNorm
    scale w [d] ~ N(w_mean, w_std^2), both as bf16 bit patterns."""
    x = normal_bf16((m, d), 1.0, 1000 * seed + 21)
    rng = np.random.default_rng(1000 * seed + 22)
    w = bf16_from_f32((w_mean + w_std * rng.standard_normal(d)).astype(np.float32))
    return x, w
