"""Pins of the per-head (non-absorbed, DK=192 / DV=128) oracle: torch's fp64 scaled
dot-product attention per head with an explicit causal mask (a library special case),
agreement with the latent oracle when every head shares one key row and V is its first
128 columns, equivariance under a permutation of heads (catches a head index that K and V
do not share), and one kept key giving its value row.  (Shape: the Metal tensor-API FA
news item lists DK=192/DV=128; the Vulkan FA page section 3.3 describes per-head K/V.)"""
import numpy as np
import torch

import oracle
from mla_flash_attention_amd import synth

BF16, F16 = synth.TYPE_BF16, synth.TYPE_F16


def _f64(bits, t):
    return oracle.decode(np.ascontiguousarray(bits).reshape(-1), t).reshape(bits.shape)


def test_matches_torch_sdpa_fp64_causal_and_masked():
    for causal, mask_kind, (n_tok, n_kv) in ((True, None, (37, 90)), (False, "random", (20, 64)),
                                              (True, "runs_bias", (64, 64))):
        p = synth.make_mha_problem(n_tok, 4, n_kv, seed=n_tok + n_kv, causal=causal, mask_kind=mask_kind)
        got = oracle.mha_attention(p.q, p.q_type, p.k, p.v, p.kv_type, p.scale, causal=causal, mask=p.mask)
        q = torch.from_numpy(_f64(p.q, BF16)).permute(1, 0, 2)       # [H][n_tok][192]
        k = torch.from_numpy(_f64(p.k, BF16)).permute(1, 0, 2)
        v = torch.from_numpy(_f64(p.v, BF16)).permute(1, 0, 2)
        bias = torch.zeros(n_tok, n_kv, dtype=torch.float64)
        if p.mask is not None:
            bias += torch.from_numpy(_f64(p.mask, F16))
        if causal:
            t = torch.arange(n_tok)[:, None]
            j = torch.arange(n_kv)[None, :]
            bias = bias.masked_fill(j > n_kv - n_tok + t, float("-inf"))
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=bias, scale=float(p.scale))
        ref = torch.nan_to_num(ref, nan=0.0).permute(1, 0, 2).reshape(-1, 128).numpy()
        assert np.max(np.abs(got - ref)) < 1e-12


def test_shared_heads_equal_the_latent_oracle():
    n_tok, H, n_kv = 9, 4, 50
    p = synth.make_mha_problem(n_tok, H, n_kv, seed=3, causal=True)
    row = p.k[:, 0, :]                                            # one 192-wide key row per cell
    k = np.repeat(row[:, None, :], H, axis=1)
    v = np.repeat(row[:, None, :128], H, axis=1)
    got = oracle.mha_attention(p.q, BF16, k, v, BF16, p.scale, causal=True)
    ref = oracle.attention(p.q[None], BF16, row[None], BF16, 1, n_tok, H, n_kv, p.scale, causal=True,
                           dk=192, dv=128)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_head_permutation_equivariance():
    p = synth.make_mha_problem(12, 6, 40, seed=4, causal=True)
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = oracle.mha_attention(p.q, BF16, p.k, p.v, BF16, p.scale, causal=True).reshape(12, 6, -1)
    b = oracle.mha_attention(p.q[:, perm], BF16, p.k[:, perm], p.v[:, perm], BF16, p.scale, causal=True)
    assert np.array_equal(a[:, perm], b.reshape(12, 6, -1))


def test_one_kept_key_gives_its_value():
    p = synth.make_mha_problem(3, 2, 5, seed=5, causal=False)
    mask = np.full((3, 5), synth.F16_NEG_INF, dtype=np.uint16)
    mask[:, 2] = 0
    got = oracle.mha_attention(p.q, BF16, p.k, p.v, BF16, p.scale, causal=False, mask=mask).reshape(3, 2, -1)
    vals = _f64(p.v, BF16)
    for t in range(3):
        assert np.array_equal(got[t], vals[2])
