"""GPU parity of the attention half of a decode layer and of the whole
chained decode layer (noisy RMSNorm -> q/k/v -> attention stub -> o ->
noisy RMSNorm -> gate/up -> SiLU(gate) * up -> down), with one noise vector
per call or one noise row per token (the per-rollout variant).

Bars: the attention stub copies values, so it is bit-exact; the row sampler
is within one fp32 ulp of the oracle (as qerl_aqn_sample); every linear
call is within 2e-2 of max(|y*|, rms(y*)).  A chain composes four linear
calls, each within 2e-2 of its exact output and each of relative gain
about one (random weights between RMSNorms), so to first order its output is
within the sum, 4 x 2e-2 = 8e-2; each call of a chain returns bf16, and the
oracle chain rounds to bf16 (nearest even) at the same points and is
otherwise fp64.  The chain cases use sigma = 0.25, at which dropping the
noise (or sharing one row) moves the output by several times that bar."""
import numpy as np
import pytest
import torch

from oracle import aqn, attention, formats, linear, nvfp4, rmsnorm, swiglu
from tests._gpu import dev16, host, oracle_columns
from workloads import make_layer, norm_inputs, normal_bf16

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402

TOL = 2e-2
DEV = "cuda:0"


def round_bf16(v):
    mant, expo = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.rint(mant * 256.0) / 256.0, expo)


def ulp_diff(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


@pytest.mark.parametrize("m,hq,hkv,dh", [(1, 4, 4, 8), (64, 28, 4, 128), (130, 40, 8, 128)])
def test_attention_stub_bitexact(m, hq, hkv, dh):
    qkv = normal_bf16((m, (hq + 2 * hkv) * dh), 1.0, 60 + m)
    out = q.qerl_attention_stub(dev16(qkv), hq, hkv, dh)
    torch.cuda.synchronize()
    ref = attention.decode_attention(qkv, hq, hkv, dh)
    assert np.array_equal(formats.bf16_bits_to_f64(host(out)), ref)


@pytest.mark.parametrize("m,d", [(1, 256), (64, 5120), (128, 27648)])
def test_row_sampler(m, d):
    z = host(q.qerl_aqn_sample_rows(7, 1, 9, 0.01, m, d, device=DEV))
    torch.cuda.synchronize()
    z0 = host(q.qerl_aqn_sample(7, 1, 9, 0.01, d, device=DEV))
    assert np.array_equal(z[0], z0)
    rows = sorted({0, m // 2, m - 1})
    ref = np.stack([aqn.sample(7, 1, 9, 0.01, d, row=i) for i in rows])
    assert ulp_diff(z[rows], ref).max() <= 1


@pytest.mark.parametrize("m,n,k,r,entry", [
    (64, 512, 1024, 32, "decode"),      # LDS-staged decode
    (128, 600, 1280, 64, "decode"),     # 128-token kernel, split K
    (17, 200, 1040, 24, "decode"),      # general kernel
    (96, 64, 8192, 8, "decode"),        # split K finish
    (300, 384, 1024, 16, "prefill"),    # prefill GEMM
])
def test_rownoise_linear(m, n, k, r, entry):
    # sigma = 0.25: per-row noise changes y by about a quarter, so a shared
    # vector (or a wrong row) in place of the rows fails the bar by far
    L = make_layer(m, n, k, r, seed=m + n, outlier_frac=1e-3, call_id=4)
    codes, scales, S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
    zr = q.qerl_aqn_sample_rows(L.seed, 0, 4, 0.25, m, k, device=DEV)
    fn = q.qerl_linear_decode_rownoise if entry == "decode" else q.qerl_linear_prefill_rownoise
    y = fn(dev16(L.x), codes, scales, S, dev16(L.a), dev16(L.b), L.lora_scale, zr)
    torch.cuda.synchronize()
    z = aqn.sample_rows(L.seed, 0, 4, 0.25, m, k)
    ref = oracle_columns(L, np.arange(n), z)
    err = linear.max_rel_error(formats.bf16_bits_to_f64(host(y)), ref)
    shared = linear.max_rel_error(oracle_columns(L, np.arange(n), z[0]), ref)
    print(f"rownoise {entry} m={m} n={n} k={k} err={err:.3g} (shared-vector ref {shared:.3g})",
          flush=True)
    assert err <= TOL and shared > 10 * TOL


class Layer:
    """One decoder layer's weights (NVFP4 on the GPU, oracle dequantization
    on the host) and LoRA factors."""

    def __init__(self, n, k, r, seed):
        L = make_layer(1, n, k, r, seed=seed)
        self.L = L
        self.codes, self.scales, self.S, _ = q.qerl_quantize_nvfp4(dev16(L.w))
        self.a, self.b = dev16(L.a), dev16(L.b)
        self.w_hat = nvfp4.dequantize(*nvfp4.quantize(L.w))


CHAIN_TOL = 4 * TOL


def chained_layer(m, hidden, inter, hq, hkv, dh, r, per_row, seed, sig=0.25):
    """Runs the chain on the GPU and in the oracle; returns (max rel error
    against the bf16-rounded oracle chain, against the unrounded one, and
    the error of the oracle chain without noise against the noisy one)."""
    x, w1 = norm_inputs(m, hidden, seed=seed)
    _, w2 = norm_inputs(1, hidden, seed=seed + 1)
    qkv_l = Layer((hq + 2 * hkv) * dh, hidden, r, seed + 2)
    o_l = Layer(hidden, hq * dh, r, seed + 3)
    gu_l = Layer(2 * inter, hidden, r, seed + 4)
    dn_l = Layer(hidden, inter, r, seed + 5)
    widths = [hidden, hq * dh, hidden, inter]
    if per_row:
        zs = [aqn.sample_rows(seed, 0, c, sig, m, d) for c, d in enumerate(widths)]
        zd = [q.qerl_aqn_sample_rows(seed, 0, c, sig, m, d, device=DEV)
              for c, d in enumerate(widths)]
    else:
        zs = [aqn.sample(seed, 0, c, sig, d) for c, d in enumerate(widths)]
        zd = [q.qerl_aqn_sample(seed, 0, c, sig, d, device=DEV) for c, d in enumerate(widths)]

    # GPU chain, one library call per step.  Per-call noise: the q/k/v and
    # gate/up groups take theirs in the RMSNorm scale (Eq. 10), o and down in
    # their own input (Eq. 12).  Per-row noise: every linear call takes its
    # rows (the RMSNorms are plain).
    lin = q.qerl_linear_decode_rownoise if per_row else q.qerl_linear_decode
    h = q.qerl_rmsnorm_noisy(dev16(x), dev16(w1), None if per_row else zd[0], 1e-6)
    qkv = lin(h, qkv_l.codes, qkv_l.scales, qkv_l.S, qkv_l.a, qkv_l.b, 2.0,
              zd[0] if per_row else None)
    att = q.qerl_attention_stub(qkv, hq, hkv, dh)
    o = lin(att, o_l.codes, o_l.scales, o_l.S, o_l.a, o_l.b, 2.0, zd[1])
    h2 = q.qerl_rmsnorm_noisy(o, dev16(w2), None if per_row else zd[2], 1e-6)
    gu = lin(h2, gu_l.codes, gu_l.scales, gu_l.S, gu_l.a, gu_l.b, 2.0, zd[2] if per_row else None)
    if per_row:
        y = lin(q.qerl_swiglu(gu), dn_l.codes, dn_l.scales, dn_l.S, dn_l.a, dn_l.b, 2.0, zd[3])
    else:
        y = q.qerl_linear_decode_swiglu(gu, dn_l.codes, dn_l.scales, dn_l.S, dn_l.a, dn_l.b, 2.0,
                                        zd[3])
    torch.cuda.synchronize()
    got = formats.bf16_bits_to_f64(host(y))

    def lv(inp, lay, z):
        return linear.linear_values(inp, lay.w_hat, z, lay.L.a, lay.L.b, 2.0)

    def chain(rnd, zs=zs):
        h_r = rnd(rmsnorm.rmsnorm_noisy(x, w1, None if per_row else zs[0], 1e-6))
        qkv_r = rnd(lv(h_r, qkv_l, zs[0] if per_row else None))
        # attention over the one-position context of each row
        q_, k_, v_ = attention.split_qkv(qkv_r, hq, hkv, dh)
        att_r = np.stack([attention.attend(q_[i], k_[i][None], v_[i][None], hq, hkv)
                          for i in range(m)]).reshape(m, hq * dh)
        o_r = rnd(lv(att_r, o_l, zs[1]))
        # the second RMSNorm on fp64 values (Eq. 10 as in oracle.rmsnorm)
        ms = np.mean(o_r * o_r, axis=1, keepdims=True)
        wn = formats.bf16_bits_to_f64(w2) + (0.0 if per_row else zs[2].astype(np.float64))
        h2_r = rnd(wn * (o_r / np.sqrt(ms + 1e-6)))
        gu_r = rnd(lv(h2_r, gu_l, zs[2] if per_row else None))
        act_r = rnd(swiglu.silu(gu_r[:, :inter]) * gu_r[:, inter:])
        return lv(act_r, dn_l, zs[3])

    ref = chain(round_bf16)
    quiet = chain(round_bf16, [np.zeros_like(z) for z in zs])
    return (linear.max_rel_error(got, ref), linear.max_rel_error(got, chain(lambda v: v)),
            linear.max_rel_error(quiet, ref))


@pytest.mark.parametrize("per_row", [False, True])
@pytest.mark.parametrize("m,hidden,inter,hq,hkv,dh,r,sig", [
    (16, 512, 1024, 4, 2, 128, 8, 0.25),
    (64, 3584, 4096, 28, 4, 128, 32, 0.25),   # Qwen2.5-7B head layout, reduced intermediate
    (128, 1024, 2048, 8, 2, 128, 64, 0.25),   # 128 tokens: the single-pass kernel
    (64, 1024, 2048, 8, 2, 128, 32, 1e-2),    # the workloads' stage-1 sigma
])
def test_chained_decode_layer(m, hidden, inter, hq, hkv, dh, r, sig, per_row):
    err, err_unrounded, noise_effect = chained_layer(m, hidden, inter, hq, hkv, dh, r, per_row,
                                                     seed=200 + m, sig=sig)
    print(f"chained layer m={m} hidden={hidden} sigma={sig} per_row={per_row}: "
          f"max_rel_error={err:.4g} (unrounded fp64 chain {err_unrounded:.4g}; the chain "
          f"without noise differs by {noise_effect:.3g})", flush=True)
    assert err <= CHAIN_TOL
    if sig >= 0.1:
        assert noise_effect > 4 * CHAIN_TOL
