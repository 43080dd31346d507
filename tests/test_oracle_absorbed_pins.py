"""Pins for oracle.absorbed_attention (latent attention with the per-head projections
absorbed either side).

The pages describe the absorbed path as logically the step-by-step one ("Vulkan backend
fused Flash Attention: DeepSeek MLA local inference", section 3.3): decompress each cached
latent row into per-head keys (W_UK) and values (W_UV), then run ordinary per-head
softmax attention with 192-wide keys (128 + the shared 64 RoPE dims).  The first pin
computes exactly that, by brute force in fp64 on tiny inputs, and checks the oracle
against it; the others check special cases that reduce to the latent-attention oracle
(identity projections) and linearity in W_UV."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0


def _cache_f64(p):
    kv = p.kv
    if p.kv_type == Q8:
        return oracle.decode_q8_0_rows(kv.reshape(-1, kv.shape[-1]), 576).reshape(kv.shape[0], p.n_kv, 576)
    return oracle.decode(kv, p.kv_type).reshape(kv.shape[0], p.n_kv, 576)


def brute_non_absorbed(p):
    """Decompress, then per-head attention: the step-by-step definition, fp64."""
    qn = oracle.decode(p.q_nope, p.q_type).reshape(p.n_seq, p.n_tok, p.n_head, 128)
    qp = oracle.decode(p.q_pe, p.q_type).reshape(p.n_seq, p.n_tok, p.n_head, 64)
    wk = oracle.decode(p.w_uk, p.q_type).reshape(p.n_head, 512, 128)
    wv = oracle.decode(p.w_uv, p.q_type).reshape(p.n_head, 128, 512)
    cache = _cache_f64(p)
    scale = float(np.float32(p.scale))
    out = np.zeros((p.n_seq, p.n_tok, p.n_head, 128))
    for s in range(p.n_seq):
        c = cache[0 if cache.shape[0] == 1 else s]
        length = p.n_kv if p.kv_len is None else int(min(max(p.kv_len[s], 0), p.n_kv))
        for h in range(p.n_head):
            k_nope = c[:length, :512] @ wk[h]            # [j][128]: W_UK[h]^T applied to each row
            k = np.concatenate([k_nope, c[:length, 512:]], axis=1)   # [j][192]
            v = c[:length, :512] @ wv[h].T               # [j][128]
            for t in range(p.n_tok):
                q = np.concatenate([qn[s, t, h], qp[s, t, h]])
                sc = np.empty(length)
                for j in range(length):
                    bias = 0.0
                    if p.mask is not None:
                        bias = float(oracle.decode(p.mask[s, t, j:j + 1], F16)[0])
                    if p.causal and j > length - p.n_tok + t:
                        bias = -np.inf
                    sc[j] = -np.inf if bias == -np.inf else scale * float(q @ k[j]) + bias
                if length == 0 or np.all(sc == -np.inf):
                    continue
                w = np.exp(sc - sc.max())
                out[s, t, h] = (w / w.sum()) @ v
    return out.reshape(-1, 128)


def absorbed(p, **kw):
    return oracle.absorbed_attention(p.q_nope, p.q_pe, p.q_type, p.w_uk, p.w_uv, p.kv, p.kv_type, p.n_seq,
                                     p.n_tok, p.n_head, p.n_kv, p.scale, causal=p.causal, mask=p.mask,
                                     kv_len=p.kv_len, **kw)


@pytest.mark.parametrize("kw", [
    dict(n_seq=2, n_tok=1, n_head=3, n_kv=37, q_type=BF16, kv_type=BF16, seed=1),
    dict(n_seq=1, n_tok=3, n_head=2, n_kv=20, q_type=F16, kv_type=F16, seed=2, causal=True),
    dict(n_seq=2, n_tok=2, n_head=2, n_kv=64, q_type=F16, kv_type=Q8, seed=3, mask_kind="runs_bias"),
    dict(n_seq=3, n_tok=2, n_head=2, n_kv=40, q_type=BF16, kv_type=BF16, seed=4, causal=True, ragged=True),
])
def test_absorbed_equals_decompressed_attention(kw):
    p = synth.make_absorbed_problem(**kw)
    got = absorbed(p)
    ref = brute_non_absorbed(p)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12), np.abs(got - ref).max()


def test_identity_projections_reduce_to_latent_attention():
    """W_UK embeds the 128 key dims as the first 128 latent dims, W_UV reads them back:
    the result is the latent-attention oracle on q = [q_nope, 0, q_pe], first 128 columns."""
    p = synth.make_absorbed_problem(2, 2, 3, 50, BF16, BF16, seed=5, causal=True)
    one = synth.round_bits(np.ones(1, np.float32), BF16)[0]
    wk = np.zeros((3, 512, 128), np.uint16)
    wv = np.zeros((3, 128, 512), np.uint16)
    for d in range(128):
        wk[:, d, d] = one
        wv[:, d, d] = one
    p.w_uk, p.w_uv = wk, wv
    q = np.zeros((2, 2, 3, 576), np.uint16)
    q[..., :128] = p.q_nope
    q[..., 512:] = p.q_pe
    ref = oracle.attention(q, BF16, p.kv, BF16, 2, 2, 3, 50, p.scale, causal=True)[:, :128]
    got = absorbed(p)
    assert np.array_equal(got, ref)


def test_linear_in_w_uv():
    p = synth.make_absorbed_problem(1, 1, 2, 30, BF16, BF16, seed=6)
    a = absorbed(p)
    p.w_uv = synth.round_bits(oracle.decode(p.w_uv, BF16).astype(np.float32) * 2, BF16)   # exact doubling
    assert np.array_equal(absorbed(p), 2 * a)


def test_rows_subset_matches_full():
    p = synth.make_absorbed_problem(2, 3, 4, 33, F16, F16, seed=7, causal=True)
    full = absorbed(p)
    rows = np.array([0, 5, 11, 23, 17])
    assert np.array_equal(absorbed(p, rows=rows), full[rows])
