"""GPU quantizer parity: codes, block scales and S bit-exact against the
oracle, on exhaustive bf16 sweeps, constructed ties, special values and the
workloads' weight distributions (full size, sampled rows)."""
import numpy as np
import pytest
import torch

from oracle import formats, nvfp4
from workloads import bf16_from_f32, weight_bf16, CONFIGS
from tests._gpu import dev16, host

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402  (fails loudly if unbuilt)


def gpu_quantize(w_bits):
    codes, scales, S, flag = q.qerl_quantize_nvfp4(dev16(w_bits))
    torch.cuda.synchronize()
    return host(codes), host(scales), np.float32(host(S)[0]), int(host(flag)[0])


def assert_same(w_bits):
    c, s, S, flag = gpu_quantize(w_bits)
    rc, rs, rS = nvfp4.quantize(w_bits)
    assert flag == 0
    assert np.float32(S).view(np.uint32) == np.float32(rS).view(np.uint32)
    assert np.array_equal(s, rs), np.argwhere(s != rs)[:5]
    assert np.array_equal(c, rc), np.argwhere(c != rc)[:5]


def test_tiny_layer_weight():
    assert_same(weight_bf16(512, 256, 0.02, 1))


def test_exhaustive_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    bits = bits[finite]                                    # 65280 values
    rng = np.random.default_rng(0)
    for _ in range(3):
        assert_same(rng.permutation(bits).reshape(-1, 64))


@pytest.mark.parametrize("lo,hi", [(-24, 4), (-10, 10), (-133, -100), (100, 127)])
def test_exponent_windows(lo, hi):
    """All bf16 magnitudes with exponent in [lo, hi), both signs, shuffled."""
    e = np.arange(lo, hi)
    mant = np.arange(128)
    exp_field = np.clip(e + 127, 0, 254)
    bits = ((exp_field[:, None] << 7) | mant[None, :]).ravel().astype(np.uint16)
    bits = np.concatenate([bits, bits | 0x8000])
    bits = bits[: len(bits) // 16 * 16]
    rng = np.random.default_rng(lo + 1000)
    assert_same(rng.permutation(bits).reshape(-1, 16))


def test_constructed_ties_every_block_scale():
    """Every nonzero E4M3 block scale, with elements exactly on every E2M1
    midpoint (ties) and on every grid point, S a power of two."""
    S = 2.0 ** -12
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    grid = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    rows = []
    for code in range(1, 127):
        sb = formats.E4M3_VALUES[code]
        for vals in (mids, grid):
            row = [6.0 * sb * S] + [v * sb * S for v in vals] + \
                  [-v * sb * S for v in vals] + [-0.0]
            rows.append(row)
    rows[0][0] = 6.0 * 448.0 * S
    w = np.array(rows, dtype=np.float64)
    bits = bf16_from_f32(w.astype(np.float32))
    assert np.array_equal(formats.bf16_bits_to_f64(bits), w)   # inputs exact
    assert_same(bits)


def test_zero_tiny_and_signed_zero():
    w = np.zeros((3, 32), dtype=np.uint16)
    w[1, 5] = 0x8000
    assert_same(w)
    tiny = np.zeros((2, 32), dtype=np.uint16)
    tiny[0, 0] = 0x0001                    # smallest bf16 subnormal: S -> 0
    tiny[1, 7] = 0x8005
    assert_same(tiny)
    sub = np.full((2, 32), 0x0080, dtype=np.uint16)    # 2^-126: S subnormal fp32
    sub[0, 3] = 0x0100
    assert_same(sub)


def test_nonfinite_flag():
    w = weight_bf16(8, 64, 0.02, 3)
    for bad in (0x7F80, 0xFF80, 0x7FC0):
        w2 = w.copy()
        w2[5, 17] = bad
        assert gpu_quantize(w2)[3] == 1
    assert gpu_quantize(w)[3] == 0


def test_deterministic_and_outliers():
    w = weight_bf16(1024, 512, 0.02, 4, outlier_frac=1e-3)
    a, b = gpu_quantize(w), gpu_quantize(w)
    assert all(np.array_equal(x, y) for x, y in zip(a[:2], b[:2])) and a[2] == b[2]
    assert_same(w)


@pytest.mark.parametrize("name,idx", [("decode_7b_mlp", 0), ("decode_7b_mlp", 1),
                                      ("quantize_prefill_14b", 1)])
def test_full_size_sampled_rows(name, idx):
    cfg = CONFIGS[name]
    shape = cfg.layers[idx]
    w = weight_bf16(shape.n, shape.k, 0.02, 100 + idx, outlier_frac=cfg.outlier_frac)
    c, s, S, flag = gpu_quantize(w)
    assert flag == 0
    wf = formats.bf16_bits_to_f64(w)
    rS = nvfp4.global_scale(nvfp4.tensor_amax(wf))
    assert np.float32(S).view(np.uint32) == np.float32(rS).view(np.uint32)
    rng = np.random.default_rng(idx)
    rows = np.unique(np.concatenate([[0, shape.n - 1], rng.choice(shape.n, 96, replace=False)]))
    rc, rs = nvfp4.encode_with_scale(wf[rows], rS)
    assert np.array_equal(s[rows], rs)
    assert np.array_equal(c[rows], rc)


def test_batch_matches_single_calls():
    """qerl_quantize_nvfp4_batch: every tensor bit-identical to its own call
    (and to the oracle), across tensors of very different sizes, a zero
    tensor, a subnormal-S tensor and a non-finite one (its flag alone set)."""
    shapes = [(1, 16), (3, 48), (512, 256), (1024, 5120), (2, 32), (37, 80), (2, 32),
              (4608, 3584), (8, 64)]
    ws = [weight_bf16(n, k, 0.02, 200 + i, outlier_frac=1e-3) for i, (n, k) in enumerate(shapes)]
    ws[4] = np.zeros((2, 32), dtype=np.uint16)
    ws[6] = np.full((2, 32), 0x0080, dtype=np.uint16)
    ws[8] = ws[8].copy()
    ws[8][3, 9] = 0x7F80
    outs = q.qerl_quantize_nvfp4_batch([dev16(w) for w in ws])
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        c, s, S, flag = (host(t) for t in outs[i])
        c1, s1, S1, flag1 = gpu_quantize(w)
        assert int(flag[0]) == flag1 == (1 if i == 8 else 0), i
        if i == 8:
            continue
        assert np.float32(S[0]).view(np.uint32) == np.float32(S1).view(np.uint32), i
        assert np.array_equal(s, s1) and np.array_equal(c, c1), i
        if w.size <= 512 * 256:
            rc, rs, rS = nvfp4.quantize(w)
            assert np.float32(S[0]).view(np.uint32) == np.float32(rS).view(np.uint32), i
            assert np.array_equal(s, rs) and np.array_equal(c, rc), i


def test_batch_single_tensor_and_reuse():
    w = weight_bf16(256, 512, 0.02, 7)
    (c, s, S, flag), = q.qerl_quantize_nvfp4_batch([dev16(w)])
    rc, rs, rS = nvfp4.quantize(w)
    assert int(host(flag)[0]) == 0
    assert np.float32(host(S)[0]).view(np.uint32) == np.float32(rS).view(np.uint32)
    assert np.array_equal(host(s), rs) and np.array_equal(host(c), rc)
    # the same outputs again, through a bound call (slots hold S from before)
    ws = [dev16(weight_bf16(64, 128, 0.02, 8)), dev16(w)]
    outs = q.qerl_quantize_nvfp4_batch(ws)
    call = q.bind_quantize_nvfp4_batch(ws, outs)
    for _ in range(2):
        call()
        torch.cuda.synchronize()
        assert np.array_equal(host(outs[1][0]), rc) and np.array_equal(host(outs[1][1]), rs)
