"""GPU checks of the tiled weight layout (qerl_nvfp4_tile128) and of the
decode entry points that read it (qerl_linear_decode_tiled and its
prepared half): the tiles hold exactly the documented bytes, the tiled
layer is bit-identical to qerl_linear_decode where both run the 128-token
kernel, and it matches the fp64 oracle (2e-2, the layer metric) at any m."""
import numpy as np
import pytest
import torch

from oracle import aqn, formats, linear, nvfp4
from tests._gpu import dev16, host, oracle_columns
from workloads import make_layer

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402

TOL = 2e-2


def untile(tiles, n, k):
    """Standard (codes [n, k/2], scales [n, k/16]) from the documented tiled
    layout, and the bytes of the padding rows."""
    nsub, nb = tiles.shape[0], tiles.shape[1]
    t = tiles.reshape(nsub, nb, 2304)
    cod = t[:, :, :2048].reshape(nsub, nb, 2, 2, 32, 16)     # st, b, kh, h, c, byte
    sca = t[:, :, 2048:].reshape(nsub, nb, 2, 2, 32, 2)
    # row 32 st + c, code byte 64 b + 32 kh + 16 h + j; scale byte 8 b + 4 kh + 2 h + j
    codes = cod.transpose(0, 4, 1, 2, 3, 5).reshape(nsub * 32, nb * 64)
    scales = sca.transpose(0, 4, 1, 2, 3, 5).reshape(nsub * 32, nb * 8)
    return codes[:n], scales[:n], codes[n:], scales[n:]


@pytest.mark.parametrize("n,k", [(64, 128), (300, 640), (37, 5120)])
def test_tile_layout(n, k):
    L = make_layer(1, n, k, 0, seed=n + k, outlier_frac=1e-3)
    codes, scales, S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
    tiles = q.qerl_nvfp4_tile128(codes, scales)
    torch.cuda.synchronize()
    assert tiles.numel() == q.qerl_nvfp4_tile128_bytes(n, k)
    c2, s2, cpad, spad = untile(host(tiles), n, k)
    assert np.array_equal(c2, host(codes)) and np.array_equal(s2, host(scales))
    assert not cpad.any() and not spad.any()


class Tiled:
    def __init__(self, L, sigma):
        self.L = L
        self.x = dev16(L.x)
        self.codes, self.scales, self.S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
        self.tiles = q.qerl_nvfp4_tile128(self.codes, self.scales)
        self.a = None if L.a is None else dev16(L.a)
        self.b = None if L.b is None else dev16(L.b)
        self.z = None
        if sigma:
            self.z = q.qerl_aqn_sample(L.seed, L.stream_id, L.call_id, sigma, L.x.shape[1],
                                       device="cuda:0")

    def tiled(self):
        n = self.L.w.shape[0]
        y = q.qerl_linear_decode_tiled(self.x, self.tiles, self.S, n, self.a, self.b,
                                       self.L.lora_scale, self.z)
        torch.cuda.synchronize()
        return host(y)

    def standard(self):
        y = q.qerl_linear_decode(self.x, self.codes, self.scales, self.S, self.a, self.b,
                                 self.L.lora_scale, self.z)
        torch.cuda.synchronize()
        return host(y)


@pytest.mark.parametrize("m,n,k,r,sigma", [
    (128, 1000, 5120, 64, 1e-2),    # the 32B shapes' rank, ragged rows
    (96, 300, 1152, 24, 0.25),      # three token tiles, noise-dominant
    (200, 512, 640, 8, 1e-2),       # a 128-token chunk, then 72 tokens (both 128-token kernel)
    (128, 64, 384, 0, 0.0),         # no LoRA, no noise, one 64-row group
])
def test_tiled_matches_standard_bitwise(m, n, k, r, sigma):
    L = make_layer(m, n, k, r, seed=m + 2 * n, outlier_frac=1e-3, call_id=5)
    g = Tiled(L, sigma)
    yt = g.tiled()
    if m % 128 == 0 or m % 128 > 64:
        assert np.array_equal(yt, g.standard())
    z = None if not sigma else aqn.sample(L.seed, L.stream_id, L.call_id, sigma, k)
    err = linear.max_rel_error(formats.bf16_bits_to_f64(yt), oracle_columns(L, np.arange(n), z))
    assert err <= TOL, err


@pytest.mark.parametrize("m,n,k,r", [(1, 256, 512, 8), (40, 700, 2048, 32), (64, 96, 8192, 72)])
def test_tiled_small_m_against_oracle(m, n, k, r):
    # fewer than 65 tokens also run the 128-token kernel (rows past m are zeros)
    L = make_layer(m, n, k, r, seed=3 * m + n, outlier_frac=1e-3, call_id=6)
    g = Tiled(L, 1e-2)
    z = aqn.sample(L.seed, L.stream_id, L.call_id, 1e-2, k)
    err = linear.max_rel_error(formats.bf16_bits_to_f64(g.tiled()),
                               oracle_columns(L, np.arange(n), z))
    assert err <= TOL, err


def test_tiled_prepared_halves_and_determinism():
    m, n, k, r = 128, 2048, 2560, 64
    L = make_layer(m, n, k, r, seed=91, call_id=1)
    g = Tiled(L, 1e-2)
    y1, y2 = g.tiled(), g.tiled()
    assert np.array_equal(y1, y2)
    ws = q.tiled_workspace(m, n, k, r, "cuda:0")
    q.qerl_linear_prepare(g.x, n, g.a, L.lora_scale, g.z, ws)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(2):
        q.qerl_linear_decode_tiled_prepared(m, g.tiles, g.S, n, k, g.b, y, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(y), y1)
