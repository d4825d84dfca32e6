"""GPU linear-layer parity: qerl_linear_decode / qerl_linear_prefill (bf16
out) against the fp64 oracle, max relative error <= 2e-2 with the
rms(y*) floor, on the tiny layer in full, on ragged and degenerate shapes,
and on the full-size decode and prefill layers (sampled columns).

Error budget of the HIP path (all relative to the output scale): rounding
x_t = x (1 + z) to bf16 (2^-9 per element, averaging out over k),
rounding s x_t A^T to bf16 (2^-9 of the LoRA term), fp32 accumulation,
and the bf16 output rounding (2^-9).  Observed errors are ~4e-3; the 2e-2
bound leaves a wide margin and still catches any wrong index, scale or
sign."""
import numpy as np
import pytest
import torch

from oracle import aqn, formats, linear, nvfp4
from workloads import make_layer, CONFIGS
from tests._gpu import dev16, host, oracle_noise, oracle_columns

pytestmark = pytest.mark.gpu
import nvfp4_weight_quantized_qerl_amd as q   # noqa: E402

TOL = 2e-2


class GpuLayer:
    """Device copies of a layer's inputs, quantized on the GPU.  The noise
    has the layer's stage sigma unless `sigma` is given."""

    def __init__(self, L, num_stages=10, sigma=None):
        self.L = L
        self.x = dev16(L.x)
        wdev = dev16(L.w)
        self.codes, self.scales, self.S, flag = q.qerl_quantize_nvfp4(wdev)
        del wdev
        self.a = None if L.a is None else dev16(L.a)
        self.b = None if L.b is None else dev16(L.b)
        self.z = None
        if sigma is None and L.stage > 0:
            sigma = q.qerl_aqn_sigma(1e-2, 5e-4, num_stages, L.stage)
        if sigma:
            self.z = q.qerl_aqn_sample(L.seed, L.stream_id, L.call_id, sigma, L.x.shape[1],
                                       device="cuda:0")

    def run(self, entry="decode", **kw):
        fn = q.qerl_linear_decode if entry == "decode" else q.qerl_linear_prefill
        y = fn(self.x, self.codes, self.scales, self.S, self.a, self.b, self.L.lora_scale,
               self.z, **kw)
        torch.cuda.synchronize()
        return formats.bf16_bits_to_f64(host(y))


def check(L, cols=None, entries=("decode", "prefill"), sigma=None):
    g = GpuLayer(L, sigma=sigma)
    if sigma is None:
        z, _ = oracle_noise(L)
    else:
        z = aqn.sample(L.seed, L.stream_id, L.call_id, sigma, L.x.shape[1])
    n = L.w.shape[0]
    cols = np.arange(n) if cols is None else cols
    ref = oracle_columns(L, cols, z)
    if sigma is not None and sigma >= 0.1:
        # The bar must see the noise: the same layer without it is far off.
        assert linear.max_rel_error(oracle_columns(L, cols, None), ref) > 10 * TOL
    errs = {}
    for e in entries:
        y = g.run(e)
        assert y.shape == (L.x.shape[0], n)
        err = linear.max_rel_error(y[:, cols], ref)
        errs[e] = err
        assert err <= TOL, (e, err)
    print(f"linear m={L.x.shape[0]} n={n} k={L.x.shape[1]} " +
          " ".join(f"{e}={v:.3g}" for e, v in errs.items()), flush=True)
    return errs


def test_tiny_layer_full():
    cfg = CONFIGS["tiny"]
    L = make_layer(cfg.m, cfg.layers[0].n, cfg.layers[0].k, cfg.r, seed=0, stage=cfg.stage)
    errs = check(L)
    assert max(errs.values()) < 1e-2


@pytest.mark.parametrize("m,n,k,r,stage", [
    (1, 64, 64, 8, 3),        # single token
    (5, 17, 48, 0, 1),        # ragged n, k % 64 != 0, no LoRA
    (33, 100, 272, 24, 2),    # ragged m / n / k, r not a multiple of 16
    (64, 520, 1024, 32, 0),   # no noise
    (130, 96, 512, 64, 5),    # m > 128: several m chunks
    (2, 1, 16, 1, 1),         # one output, one K step, rank 1
    (64, 96, 8192, 32, 1),    # few rows, long K: split-K across workgroups
    (128, 640, 5120, 64, 1),  # m = 128 (4 m tiles)
    (200, 300, 320, 16, 4),   # prefill-ish ragged
    (150, 200, 272, 12, 2),   # prefill GEMM: partial last K step, r % 8 != 0
    (257, 130, 1040, 40, 3),  # prefill GEMM: ragged M tile, ragged N tile
    (96, 384, 2048, 0, 1),    # prefill GEMM without LoRA
    (40, 200, 4096, 12, 2),   # split-K finish, r % 8 != 0; t summed by the split launch
    (64, 130, 6144, 72, 1),   # split-K finish, r > 64 (B row read in the loop)
    (17, 64, 1040, 24, 3),    # split-K in the general kernel (k % 256 != 0)
    (40, 2048, 256, 8, 1),    # LDS-staged, unsplit with t summed inside the launch (2 token tiles)
    (20, 2048, 256, 8, 2),    # the same with one token tile
])
def test_shapes(m, n, k, r, stage):
    L = make_layer(m, n, k, r, seed=m * 7 + n, stage=stage, outlier_frac=1e-3)
    check(L)


def test_no_noise_is_bit_identical_to_zero_noise_and_no_lora_b_zero():
    L = make_layer(16, 256, 256, 8, seed=21, stage=0)
    g = GpuLayer(L)
    y0 = g.run()
    g.z = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    assert np.array_equal(g.run(), y0)
    g.z = None
    g.b = torch.zeros_like(g.b)
    yb0 = g.run()
    g.a = g.b = None
    assert np.array_equal(g.run(), yb0)


def test_zero_weight_gives_lora_only():
    L = make_layer(8, 64, 128, 8, seed=22, stage=2)
    L.w = np.zeros_like(L.w)
    g = GpuLayer(L)
    assert float(host(g.S)[0]) == 0.0
    z, _ = oracle_noise(L)
    ref = 2.0 * linear.lora_down(L.x, z, L.a) @ formats.bf16_bits_to_f64(L.b).T
    assert linear.max_rel_error(g.run(), ref) <= TOL


@pytest.mark.parametrize("m,n,k,r", [
    (64, 96, 8192, 32),      # K split: the finishing kernel applies S and t B^T
    (32, 16384, 512, 8),     # unsplit: the contraction kernel's own epilogue
    (50, 16384, 256, 16),    # ragged m, unsplit
    (128, 96, 2048, 40),     # the 128-token kernel, r not a multiple of 16 or 32
    (200, 96, 2048, 40),     # two 128-token chunks, K split in both
    (3, 96, 768, 8),         # one 32-row tile
    (100, 300, 2048, 24),    # 128-token kernel, 100 tokens, ragged last row group, K split
    (128, 2056, 256, 24),    # 128-token kernel unsplit: its epilogue waits for t from the launch
    (100, 4104, 384, 16),    # the same with 100 tokens and a ragged last row group
    (96, 2056, 256, 24),     # the same with three token tiles (t rows past 96 read as zeros)
    (40, 2048, 256, 8),      # LDS-staged, unsplit, t summed inside the launch
    (20, 2048, 256, 8),      # the same with one token tile
])
def test_deterministic_and_prepared_halves(m, n, k, r):
    # The whole call and its two halves give the same bits.  The halves run
    # the prepare with its own LoRA-down reduction launch, then the
    # contraction and, when K is split, the finish.  A whole call whose first
    # contraction splits K (or is an unsplit 128-token launch) leaves the
    # reduction to workgroups of that launch.  Both use one reduction routine.  Repeated calls, and
    # repeated contractions from one prepared workspace, must agree.
    L = make_layer(m, n, k, r, seed=23, stage=1)
    g = GpuLayer(L)
    y1, y2 = g.run(), g.run()
    assert np.array_equal(y1, y2)
    ws = q.workspace(m, n, k, r, "cuda:0")
    for _ in range(2):       # whole calls on one workspace (its sync words are reused)
        assert np.array_equal(g.run(workspace=ws), y1)
    q.qerl_linear_prepare(g.x, n, g.a, L.lora_scale, g.z, ws)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(3):       # repeated contractions from one prepared workspace
        q.qerl_linear_decode_prepared(m, g.codes, g.scales, g.S, k, g.b, y, ws)
        torch.cuda.synchronize()
        assert np.array_equal(formats.bf16_bits_to_f64(host(y)), y1)


def _sample_cols(n, seed, count=160):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, count, replace=False)]))


@pytest.mark.parametrize("idx", [0, 1])
def test_decode_7b_mlp_full_size(idx):
    cfg = CONFIGS["decode_7b_mlp"]
    s = cfg.layers[idx]
    L = make_layer(cfg.m, s.n, s.k, cfg.r, seed=1 + idx, stage=cfg.stage,
                   outlier_frac=cfg.outlier_frac, call_id=idx)
    check(L, cols=_sample_cols(s.n, idx), entries=("decode",))


@pytest.mark.parametrize("idx", [0, 1])
def test_prefill_7b_full_size(idx):
    cfg = CONFIGS["prefill_7b"]
    s = cfg.layers[idx]
    L = make_layer(cfg.m, s.n, s.k, cfg.r, seed=11 + idx, stage=cfg.stage, call_id=idx)
    check(L, cols=_sample_cols(s.n, 10 + idx, 64), entries=("prefill",))


@pytest.mark.parametrize("idx", [0, 3])
def test_decode_32b_layer_shapes(idx):
    cfg = CONFIGS["decode_32b_sweep"]
    s = cfg.layers[idx]
    L = make_layer(cfg.m, s.n, s.k, cfg.r, seed=31 + idx, stage=cfg.stage, call_id=idx)
    check(L, cols=_sample_cols(s.n, 30 + idx, 96), entries=("decode",))


# Noise large enough to dominate the output (sigma = 0.25: the noise term is
# about a quarter of y), so that a dropped, sign-flipped or shifted noise
# channel fails the 2e-2 bar by far on every kernel path.
@pytest.mark.parametrize("m,n,k,r,entry", [
    (64, 1024, 3584, 32, "decode"),     # LDS-staged, unsplit
    (64, 96, 8192, 32, "decode"),       # LDS-staged, split K + finish
    (17, 200, 1040, 24, "decode"),      # general kernel (k % 256 != 0), split K
    (128, 640, 5120, 64, "decode"),     # 128 tokens
    (96, 200, 4096, 40, "decode"),      # 96 tokens, ragged rank
    (300, 520, 1024, 32, "prefill"),    # prefill GEMM, ragged M tile
])
def test_noise_dominant(m, n, k, r, entry):
    L = make_layer(m, n, k, r, seed=5 * m + k, call_id=7)
    check(L, entries=(entry,), sigma=0.25)


def test_noise_dominant_prefill_7b_down_full_size():
    cfg = CONFIGS["prefill_7b"]
    s = cfg.layers[1]
    L = make_layer(cfg.m, s.n, s.k, cfg.r, seed=12, call_id=1)
    check(L, cols=_sample_cols(s.n, 44, 48), entries=("prefill",), sigma=0.25)


@pytest.mark.parametrize("idx", [1, 2])
def test_decode_32b_layer_shapes_o_and_gate_up(idx):
    # the o projection (5120 x 5120) and the fused gate/up (55296 x 5120) of
    # the 32B sweep at its 128 tokens and rank 64
    cfg = CONFIGS["decode_32b_sweep"]
    s = cfg.layers[idx]
    L = make_layer(cfg.m, s.n, s.k, cfg.r, seed=31 + idx, stage=cfg.stage, call_id=idx)
    check(L, cols=_sample_cols(s.n, 30 + idx, 96), entries=("decode",))


@pytest.mark.parametrize("idx", [3, 4, 6])
def test_prefill_14b_m16384_sampled(idx):
    # one layer of the 14B model at 16384 prefill tokens: o, gate and down
    # (up has gate's shape), rank 32, stage 1
    cfg = CONFIGS["quantize_prefill_14b"]
    s = cfg.layers[idx]
    L = make_layer(cfg.m, s.n, s.k, cfg.r, seed=51 + idx, stage=cfg.stage, call_id=idx)
    check(L, cols=_sample_cols(s.n, 50 + idx, 32), entries=("prefill",))


# The single-pass 128-token contraction (k % 128 == 0, three or four 32-row
# token tiles per chunk): 256 weight rows per workgroup, K split across
# workgroups for narrow layers, four weight register sets (block counts per
# split that leave a tail of one, two or three blocks).
@pytest.mark.parametrize("m,n,k,r,stage", [
    (128, 512, 640, 32, 1),      # 5 blocks over 2 splits: tails of 2 and 3
    (128, 300, 896, 24, 2),      # 7 blocks, ragged last row group, r % 16 != 0
    (128, 2048, 1152, 64, 3),    # 9 blocks, 8 row groups
    (70, 777, 1024, 8, 1),       # 70 tokens: three tiles, ragged output rows
    (96, 64, 384, 72, 4),        # one subtile of rows, 3 blocks, rank 72 (B read in the loop)
    (128, 20000, 256, 0, 1),     # no LoRA, unsplit (79 row groups), 2 blocks
    (100, 2056, 256, 24, 2),     # unsplit, 16-byte y stores: 100 tokens, last group 8 rows wide
    (128, 1001, 256, 16, 1),     # unsplit, n % 8 != 0: 2-byte y stores
    (128, 7168, 5120, 64, 0),    # the 32B qkv shape, no noise
    (160, 640, 1280, 32, 2),     # a 128-token chunk and a 32-token remainder
    (224, 384, 768, 16, 1),      # a 128-token chunk and a 96-token chunk
    (96, 2056, 256, 24, 3),      # unsplit, three token tiles, t summed inside the launch
])
def test_decode_128_tokens(m, n, k, r, stage):
    L = make_layer(m, n, k, r, seed=3 * m + n + k, stage=stage, outlier_frac=1e-3, call_id=2)
    check(L, entries=("decode",))


@pytest.mark.parametrize("m,n,k,r", [(128, 512, 640, 32), (128, 4096, 2560, 64), (96, 300, 1024, 8)])
def test_decode_128_tokens_deterministic(m, n, k, r):
    L = make_layer(m, n, k, r, seed=77, stage=1)
    g = GpuLayer(L)
    y1, y2 = g.run(), g.run()
    assert np.array_equal(y1, y2)
