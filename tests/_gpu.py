"""Helpers shared by the GPU parity tests: host<->device transfer of bf16
bit patterns and oracle references for sampled output columns."""
import numpy as np
import torch

from oracle import aqn, formats, linear, nvfp4

DEV = "cuda:0"


def dev16(a):
    """numpy uint16 bf16 bits -> torch int16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(bits):
    return formats.bf16_bits_to_f64(bits)


def oracle_noise(L, num_stages=10):
    if L.stage == 0:
        return None, 0.0
    sig = aqn.sigma(1e-2, 5e-4, num_stages, L.stage)
    return aqn.sample(L.seed, L.stream_id, L.call_id, sig, L.x.shape[1]), sig


def oracle_columns(L, cols, z):
    """Oracle y[:, cols] for layer inputs L (S from the whole tensor)."""
    w = formats.bf16_bits_to_f64(L.w)
    S = nvfp4.global_scale(nvfp4.tensor_amax(w))
    codes, scales = nvfp4.encode_with_scale(w[cols], S)
    w_hat = nvfp4.dequantize(codes, scales, S)
    b = None if L.b is None else L.b[cols]
    return linear.linear(L.x, w_hat, z, L.a, b, L.lora_scale)
