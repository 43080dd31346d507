"""Pins of the oracle's extensions to results fixed by other means, not by retyping them:
per-sequence valid lengths and multi-token causal rows reduce to the plain oracle on a
truncated cache; the logit softcap has a large-cap limit (plain attention), a tiny-cap
limit (the mean of V) and must act before the mask bias (bias shifts stay invisible);
ALiBi slopes of 1 reproduce the plain mask path and power-of-two slopes equal a scaled
mask; a sink of -inf changes nothing, a sink follows the exact normaliser identity
out_sink = out * L / (L + exp(sink - m)) with (m, L) the plain row statistics, and a
dominant sink drives the output to 0.  (Feature readings: Metal tensor-API FA kernel
news item, which lists sinks, ALiBi and logit softcap for the 576/512 shape.)"""
import numpy as np

import oracle
from mla_flash_attention_amd import synth

BF16 = synth.TYPE_BF16


def _run(p, **kw):
    args = dict(causal=p.causal, mask=p.mask, kv_len=p.kv_len, alibi=p.alibi, sinks=p.sinks,
                softcap=p.softcap)
    args.update(kw)
    return oracle.attention(p.q, p.q_type, p.kv, p.kv_type, p.n_seq, p.n_tok, p.n_head, p.n_kv,
                            p.scale, **args)


def test_kv_len_equals_truncated_cache():
    p = synth.make_problem(kind="decode", n_seq=3, n_head=16, n_kv=90, seed=21, ragged=True)
    got = _run(p).reshape(p.n_seq, p.n_head, -1)
    for s in range(p.n_seq):
        L = int(p.kv_len[s])
        ref = oracle.attention(p.q[s:s + 1], BF16, p.kv[s:s + 1, :L], BF16, 1, 1, p.n_head, L, p.scale)
        assert np.array_equal(got[s], ref.reshape(p.n_head, -1))


def test_multi_token_causal_rows_equal_single_token_decodes():
    p = synth.make_problem(kind="decode", n_seq=2, n_tok=3, n_head=16, n_kv=70, seed=22, ragged=True,
                           causal=True)
    got = _run(p).reshape(p.n_seq, p.n_tok, p.n_head, -1)
    for s in range(p.n_seq):
        L = int(p.kv_len[s])
        for t in range(p.n_tok):
            visible = L - p.n_tok + t + 1
            ref = oracle.attention(p.q[s:s + 1, t:t + 1], BF16, p.kv[s:s + 1, :visible], BF16, 1, 1,
                                   p.n_head, visible, p.scale)
            assert np.array_equal(got[s, t], ref.reshape(p.n_head, -1))


def test_kv_len_zero_gives_zero_rows():
    p = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=40, seed=23)
    out, m, l = oracle.attention(p.q, BF16, p.kv, BF16, 2, 1, 16, 40, p.scale, kv_len=[0, 40],
                                 return_stats=True)
    assert np.all(out[:16] == 0) and np.all(m[:16] == -np.inf) and np.all(l[:16] == 0)
    assert np.array_equal(out[16:], oracle.attention(p.q[1:], BF16, p.kv[1:], BF16, 1, 1, 16, 40, p.scale))


def test_softcap_large_cap_is_plain_attention():
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=200, seed=24)
    a = _run(p, softcap=1e6)
    b = _run(p)
    assert np.max(np.abs(a - b)) < 1e-9


def test_softcap_tiny_cap_is_mean_of_values():
    """|cap * tanh(x / cap)| <= cap, so a tiny cap flattens every score to ~0: uniform weights."""
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=150, seed=25, mask_kind="random")
    got = _run(p, softcap=1e-6)
    kept = p.mask[0, 0] != synth.F16_NEG_INF
    vals = oracle.decode(p.kv[0].reshape(-1), BF16).reshape(150, synth.DK)[:, :512]
    # the random mask's finite biases still weigh the cells: softmax over the biases alone
    bias = oracle.decode(p.mask[0, 0], synth.TYPE_F16)
    w = np.where(kept, np.exp(bias - bias[kept].max()), 0.0)
    ref = (w[:, None] * vals).sum(0) / w.sum()
    assert np.max(np.abs(got - ref[None, :])) < 1e-5


def test_softcap_acts_before_the_bias():
    """A constant bias on every kept cell cancels in the softmax only if it is added after
    the cap; capping the biased score would change the relative weights."""
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=120, seed=26, softcap=2.0)
    zero = np.zeros((1, 1, 120), dtype=np.uint16)
    shifted = np.full((1, 1, 120), synth.f32_to_f16_bits(np.float32(3.0)), dtype=np.uint16)
    a = _run(p, mask=zero)
    b = _run(p, mask=shifted)
    assert np.max(np.abs(a - b)) < 1e-12
    # and the cap is active at this size: it changes the output
    assert np.max(np.abs(a - _run(p, mask=zero, softcap=0.0))) > 1e-4


def test_alibi_unit_slopes_reproduce_the_mask_path():
    p = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=100, seed=27, mask_kind="random")
    a = _run(p, alibi=np.ones(16, dtype=np.float32))
    b = _run(p, alibi=None)
    assert np.array_equal(a, b)


def test_alibi_power_of_two_slopes_equal_a_scaled_mask():
    p = synth.make_problem(kind="decode", n_seq=1, n_tok=1, n_head=16, n_kv=300, seed=28,
                           mask_kind="distance")
    slopes = np.array([2.0 ** -(h % 4) for h in range(16)], dtype=np.float32)
    got = _run(p, alibi=slopes).reshape(16, -1)
    mvals = oracle.decode(p.mask.reshape(-1), synth.TYPE_F16)
    for h in range(16):
        scaled = synth.f32_to_f16_bits((mvals * slopes[h]).astype(np.float32)).reshape(1, 1, -1)
        assert np.array_equal(oracle.decode(scaled.reshape(-1), synth.TYPE_F16), mvals * slopes[h])
        ref = _run(p, alibi=None, mask=scaled).reshape(16, -1)
        assert np.array_equal(got[h], ref[h])


def test_alibi_zero_slope_keeps_only_the_drops():
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=130, seed=29, mask_kind="random")
    zero_or_drop = np.where(p.mask == synth.F16_NEG_INF, synth.F16_NEG_INF, 0).astype(np.uint16)
    a = _run(p, alibi=np.zeros(16, dtype=np.float32))
    b = _run(p, alibi=None, mask=zero_or_drop)
    assert np.array_equal(a, b)


def test_sink_of_minus_infinity_changes_nothing():
    p = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=80, seed=30)
    a = _run(p, sinks=np.full(16, -np.inf, dtype=np.float32))
    assert np.array_equal(a, _run(p, sinks=None))


def test_sink_normaliser_identity():
    p = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=80, seed=31, sinks=True, mask_kind="runs_bias")
    got = _run(p)
    plain, m, L = oracle.attention(p.q, BF16, p.kv, BF16, 2, 1, 16, 80, p.scale, mask=p.mask,
                                   return_stats=True)
    sink = np.tile(p.sinks.astype(np.float64), 2)
    has = m > -np.inf
    factor = np.where(has, L / (L + np.exp(np.minimum(sink - m, 700.0))), 0.0)
    assert np.max(np.abs(got - plain * factor[:, None])) < 1e-12


def test_dominant_sink_and_fully_masked_rows():
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=60, seed=32, mask_kind="none_kept")
    out, m, L = oracle.attention(p.q, BF16, p.kv, BF16, 1, 1, 16, 60, p.scale, mask=p.mask,
                                 sinks=np.full(16, 1.5, dtype=np.float32), return_stats=True)
    assert np.all(out == 0) and np.all(m == 1.5) and np.all(L == 1.0)
    q = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=60, seed=33)
    out = _run(q, sinks=np.full(16, 1e4, dtype=np.float32))
    assert np.all(out == 0)
