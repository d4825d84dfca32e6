"""GPU parity of the backward through the frozen NVFP4 weight
(qerl_linear_backward) against the fp64 oracle (oracle.linear.backward).

Bar: for dx (bf16) and for dA, dB (fp32) the layer metric, max error <= 2e-2
of max(|g*|, rms(g*)).  Error budget: x_t, t = s x_t A^T and gs = s dy B are
rounded to bf16 as in the forward (2^-9 each), fp32 sums, and dx's bf16
output (2^-9)."""
import numpy as np
import pytest
import torch

from oracle import aqn, formats, linear, nvfp4
from tests._gpu import dev16, host
from workloads import make_layer, normal_bf16

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402

TOL = 2e-2


def run_case(m, n, k, r, seed, noise=True, rows=None, sigma=1e-2, lora_full=False):
    """rows: check dx on these rows only; lora_full: with rows, still check
    the whole dA and dB (they sum over every token)."""
    L = make_layer(m, n, k, r, seed=seed)
    dy = normal_bf16((m, n), 1.0, 1000 * seed + 50)
    z = aqn.sample(seed, 0, 3, sigma, k) if noise else None
    codes, scales, S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
    zd = torch.from_numpy(z).to("cuda:0") if noise else None
    a = dev16(L.a) if r else None
    b = dev16(L.b) if r else None
    dx, da, db = q.qerl_linear_backward(dev16(dy), dev16(L.x), codes, scales, S, a, b,
                                        L.lora_scale, zd)
    torch.cuda.synchronize()
    w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))
    dyf = formats.bf16_bits_to_f64(dy)
    got_dx = formats.bf16_bits_to_f64(host(dx).reshape(m, k))
    if rows is None:
        rdx, rda, rdb = linear.backward(dyf, L.x, w_hat, z, L.a if r else None,
                                        L.b if r else None, L.lora_scale)
        e = {"dx": linear.max_rel_error(got_dx, rdx)}
        if r:
            e["dA"] = linear.max_rel_error(host(da), rda)
            e["dB"] = linear.max_rel_error(host(db), rdb)
    else:
        # dx rows depend only on the same rows of dy and x
        rdx, _, _ = linear.backward(dyf[rows], L.x[rows], w_hat, z, L.a if r else None,
                                    L.b if r else None, L.lora_scale)
        e = {"dx": linear.max_rel_error(got_dx[rows], rdx)}
        if r and lora_full:
            _, rda, rdb = linear.backward(dyf, L.x, w_hat, z, L.a, L.b, L.lora_scale)
            e["dA"] = linear.max_rel_error(host(da), rda)
            e["dB"] = linear.max_rel_error(host(db), rdb)
    if noise and sigma >= 0.1 and rows is None:
        # the bar must see the noise: the gradients without it are far off
        ndx, nda, _ = linear.backward(dyf, L.x, w_hat, None, L.a if r else None,
                                      L.b if r else None, L.lora_scale)
        assert linear.max_rel_error(ndx, rdx) > 10 * TOL
        if r:
            assert linear.max_rel_error(nda, rda) > 10 * TOL
    print(f"backward m={m} n={n} k={k} r={r} noise={noise} " +
          " ".join(f"{kk}={v:.3g}" for kk, v in e.items()), flush=True)
    for kk, v in e.items():
        assert v <= TOL, (kk, v)


@pytest.mark.parametrize("m,n,k,r", [
    (4, 64, 64, 8),          # one token tile, one column tile
    (37, 96, 160, 16),       # ragged m, k not a multiple of 128
    (130, 272, 384, 40),     # n % 32 == 16, r not a multiple of 16 or 32
    (64, 512, 1024, 32),     # two token tiles per workgroup
    (256, 1024, 512, 32),    # four token tiles per workgroup
    (48, 160, 288, 72),      # three 32-wide groups of the LoRA rank in dA / dB
    (70, 128, 256, 128),     # the largest rank: four groups
])
def test_backward_parity(m, n, k, r):
    run_case(m, n, k, r, seed=m + n)


def test_backward_without_lora_and_without_noise():
    run_case(8, 128, 256, 0, seed=5)
    run_case(32, 128, 256, 8, seed=6, noise=False)


def test_backward_7b_qkv_sized_sampled_rows():
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(9).choice(4096, 30, replace=False)]))
    run_case(4096, 4608, 3584, 32, seed=9, rows=rows)


@pytest.mark.parametrize("m,n,k,r", [
    (600, 512, 1024, 32),    # three 256-token chunks of the dA / dB sums, the last ragged
    (513, 256, 768, 72),     # two full chunks and one token more, three rank groups
])
def test_backward_multi_chunk(m, n, k, r):
    run_case(m, n, k, r, seed=m + k)


@pytest.mark.parametrize("m,n,k,r", [
    (96, 256, 512, 32),      # one chunk
    (600, 512, 1024, 32),    # several chunks
])
def test_backward_noise_dominant(m, n, k, r):
    # sigma = 0.25: the noise changes dx and dA by about a quarter, so a
    # dropped, flipped or shifted noise channel fails the bar by far
    run_case(m, n, k, r, seed=3 * m + n, sigma=0.25)


def test_backward_7b_down_m4096_full_lora_grads():
    # the benched backward: 7B down layer at 4096 tokens (16 chunks of the
    # dA / dB sums); dA and dB in full, dx on sampled rows
    rows = np.unique(np.concatenate([[0, 4095],
                                     np.random.default_rng(12).choice(4096, 24, replace=False)]))
    run_case(4096, 3584, 18944, 32, seed=12, rows=rows, lora_full=True)
