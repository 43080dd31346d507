"""The seeded generators: storage rounding and Q8_0 encoding are what they claim."""
import numpy as np
import pytest

from mla_flash_attention_amd import synth


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # ties to even
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)


def test_f16_rounding_matches_numpy():
    x = np.random.default_rng(1).standard_normal(10000).astype(np.float32)
    assert np.array_equal(synth.f32_to_f16_bits(x), x.astype(np.float16).view(np.uint16))


def test_q8_0_round_trip_bound():
    """|x - q*d16| <= d*(1/2 + 2^-16) + 127*|d - d16| per element (d = amax/127 in fp32)."""
    x = np.random.default_rng(2).standard_normal((300, 576)).astype(np.float32)
    x[0, :32] = 0.0                                     # d = 0 block
    x[1, :32] = np.linspace(-1, 1, 32, dtype=np.float32)
    qb = synth.quantize_q8_0(x)
    assert qb.shape == (300, 612)
    blk = qb.reshape(300, 18, 34)
    d16 = blk[:, :, 0:2].copy().view(np.float16).astype(np.float64)[..., 0]
    codes = blk[:, :, 2:].view(np.int8).astype(np.float64)
    amax = np.abs(x.reshape(300, 18, 32)).max(-1).astype(np.float32)
    d = (amax / np.float32(127)).astype(np.float64)
    err = np.abs(x.reshape(300, 18, 32) - codes * d16[..., None])
    bound = d * (0.5 + 2 ** -16) + 127 * np.abs(d - d16)
    assert np.all(err <= bound[..., None] + 1e-30)
    assert np.all(codes[0, 0] == 0) and d16[0, 0] == 0
    assert np.abs(codes).max() <= 127


def test_sparse_mask_fraction_and_runs():
    bits = synth.sparse_runs_mask(131072, synth.rng(5, 2))
    kept = bits == 0
    assert set(np.unique(bits)) <= {0, synth.F16_NEG_INF}
    assert 0.06 < kept.mean() < 0.14
    edges = np.flatnonzero(np.diff(np.r_[0, kept.astype(np.int8), 0]))
    runs = edges[1::2] - edges[0::2]
    assert runs.min() >= 1 and runs.max() <= 256


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_shapes(cfg):
    spec = synth.CONFIGS[cfg]
    small = dict(n_kv=min(spec["n_kv"], 256), n_tok=min(spec["n_tok"], 8))
    p = synth.make_config(cfg, **small)
    assert p.q.shape == (spec["n_seq"], small["n_tok"], spec["n_head"], 576)
    row = 612 if spec["kv_type"] == synth.TYPE_Q8_0 else 576
    assert p.kv.shape[-1] == row and p.kv.shape[-2] == small["n_kv"]
    assert (p.mask is not None) == (cfg == 5)


def test_seeded_determinism():
    a = synth.make_config(2, n_kv=64)
    b = synth.make_config(2, n_kv=64)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.kv, b.kv)
