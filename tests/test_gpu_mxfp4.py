"""GPU parity of the MXFP4 variant: the quantizer bit-exact against the
oracle (codes and E8M0 scales), the NVFP4-layout form bit-exact (E4M3
scales and S), and the MXFP4 layer through the linear calls within the
layer tolerance of the fp64 oracle on the MXFP4 dequantized weight."""
import numpy as np
import pytest
import torch

from oracle import aqn, formats, linear, mxfp4
from tests._gpu import dev16, host
from workloads import bf16_from_f32, make_layer, weight_bf16

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402


def bits(v):
    return bf16_from_f32(np.asarray(v, dtype=np.float32))


def check_quantize(w):
    codes, scales, flag = q.qerl_quantize_mxfp4(dev16(w))
    s4, g, rflag = q.qerl_mxfp4_to_nvfp4(codes, scales)
    torch.cuda.synchronize()
    pc, ps, bad = mxfp4.quantize(w)
    assert int(flag.item()) == 0 and not bad
    assert np.array_equal(host(codes), pc)
    assert np.array_equal(host(scales), ps)
    want_s4, want_S, ok = mxfp4.to_nvfp4_scales(pc, ps)
    assert int(rflag.item()) == (0 if ok else 1)
    assert np.array_equal(host(s4), want_s4)
    assert host(g)[0] == np.float32(want_S)


def test_quantize_random_weights_with_outliers():
    check_quantize(weight_bf16(96, 512, 0.02, seed=41, outlier_frac=0.01))


def test_quantize_every_bf16_magnitude_in_one_block_context():
    mags = np.arange(0, 0x4100, dtype=np.uint16)
    rows = np.zeros((len(mags), 32), dtype=np.uint16)
    rows[:, 0] = bits(6.0)
    rows[:, 1] = mags
    rows[:, 2] = mags | 0x8000                      # the negative values too
    check_quantize(rows)


def test_quantize_tiny_zero_and_signed_zero_blocks():
    w = np.zeros((4, 64), dtype=np.float32)
    w[0, :32] = 2.0 ** -130                          # bf16 subnormal block
    w[1, :32] = np.linspace(-3e-39, 3e-39, 32)       # subnormals of both signs
    w[2, 5] = -0.0
    w[3, 40] = 1e30
    check_quantize(bits(w))


def test_range_flag():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1.0
    w[0, 40] = 2.0 ** -30
    codes, scales, _ = q.qerl_quantize_mxfp4(dev16(bits(w)))
    _, _, rflag = q.qerl_mxfp4_to_nvfp4(codes, scales)
    torch.cuda.synchronize()
    assert int(rflag.item()) == 1


@pytest.mark.parametrize("m,n,k,r,entry", [(64, 512, 1024, 16, "decode"),
                                           (128, 512, 1024, 16, "decode"),
                                           (300, 384, 2048, 32, "prefill")])
def test_mxfp4_layer(m, n, k, r, entry):
    L = make_layer(m, n, k, r, seed=43, outlier_frac=0.001, stage=2)
    codes, scales, _ = q.qerl_quantize_mxfp4(dev16(L.w))
    s4, g, rflag = q.qerl_mxfp4_to_nvfp4(codes, scales)
    sig = q.qerl_aqn_sigma(1e-2, 5e-4, 10, 2)
    z = q.qerl_aqn_sample(L.seed, L.stream_id, L.call_id, sig, k, device="cuda:0")
    fn = q.qerl_linear_decode if entry == "decode" else q.qerl_linear_prefill
    y = fn(dev16(L.x), codes, s4, g, dev16(L.a), dev16(L.b), L.lora_scale, z)
    torch.cuda.synchronize()
    assert int(rflag.item()) == 0
    pc, ps, _ = mxfp4.quantize(L.w)
    zo = aqn.sample(L.seed, L.stream_id, L.call_id, aqn.sigma(1e-2, 5e-4, 10, 2), k)
    ref = linear.linear(L.x, mxfp4.dequantize(pc, ps), zo, L.a, L.b, L.lora_scale)
    err = linear.max_rel_error(formats.bf16_bits_to_f64(host(y).reshape(m, n)), ref)
    print(f"mxfp4 layer {entry} m={m} n={n} k={k} err={err:.4g}", flush=True)
    assert err <= 2e-2


@pytest.mark.parametrize("m,n,k,r", [(64, 37888 // 8, 3584, 32), (50, 1024, 18944, 32), (3, 160, 512, 8),
                                     (128, 1000, 5120, 64), (100, 96, 2560, 32)])
def test_power_of_two_decode_is_bit_identical(m, n, k, r):
    # the scaled-conversion dequantization gives the same bf16 weights, so the
    # whole result must match the general decode call bit for bit
    L = make_layer(m, n, k, r, seed=44, outlier_frac=0.001, stage=1)
    codes, scales, _ = q.qerl_quantize_mxfp4(dev16(L.w))
    s4, g, _ = q.qerl_mxfp4_to_nvfp4(codes, scales)
    z = q.qerl_aqn_sample(L.seed, 0, 0, 1e-2, k, device="cuda:0")
    args = (dev16(L.x), codes, s4, g, dev16(L.a), dev16(L.b), L.lora_scale, z)
    y0 = q.qerl_linear_decode(*args)
    y1 = q.qerl_linear_decode_mxfp4(*args)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def _pow2_or_zero(b):
    """From the E4M3 decode table: zero, or a positive power of two."""
    if b & 0x80 or (b & 0x7F) == 0x7F:      # negative, or NaN
        return False
    v = formats.E4M3_VALUES[b & 0x7F]
    return v == 0.0 or float(np.log2(v)).is_integer()


def test_pow2_scale_check_every_byte():
    bad_bytes = 0
    for b in range(256):
        scales = torch.full((1, 1), b, dtype=torch.uint8, device="cuda:0")
        flag = q.qerl_nvfp4_check_pow2_scales(scales, 16)
        want = 0 if _pow2_or_zero(b) else 1
        bad_bytes += want
        assert int(flag.item()) == want, b
    assert 0 < bad_bytes < 256


def test_pow2_scale_check_on_weights():
    w = weight_bf16(96, 512, 0.02, seed=43, outlier_frac=0.01)
    codes, scales, _ = q.qerl_quantize_mxfp4(dev16(w))
    s4, _, rflag = q.qerl_mxfp4_to_nvfp4(codes, scales)
    assert int(q.qerl_nvfp4_check_pow2_scales(s4, 512).item()) == 0
    _, nv_scales, _, _ = q.qerl_quantize_nvfp4(dev16(w))
    want = 0 if all(_pow2_or_zero(int(b)) for b in host(nv_scales).ravel()) else 1
    assert want == 1
    assert int(q.qerl_nvfp4_check_pow2_scales(nv_scales, 512).item()) == want
    # one bad byte in a large tensor, at its very end
    big = torch.zeros((3000, 4096 // 16), dtype=torch.uint8, device="cuda:0")
    assert int(q.qerl_nvfp4_check_pow2_scales(big, 4096).item()) == 0
    big[-1, -1] = 0x39          # 1.125 * 2^0
    assert int(q.qerl_nvfp4_check_pow2_scales(big, 4096).item()) == 1
