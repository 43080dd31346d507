"""Pins for the CPU oracle: each test checks it against something other than itself.

* conversions: exhaustive over every bit pattern, against numpy / torch decoders;
* Q8_0: exhaustive over every int8 code and every finite f16 scale, against numpy;
* attention: mpmath brute force at 50 digits on tiny inputs, and torch's float64
  scaled_dot_product_attention (multi-query special case: K/V broadcast to every head)
  at reduced and full shapes;
* invariants and closed forms: weights sum to one, one key returns its V row,
  identical keys return the mean of V, a -inf key contributes nothing, permutation,
  mask shift, scale 0, the two-key logistic form, causal = explicit mask;
* compaction: the naive filter, and hand-derived examples in tests/golden/.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------- conversions
def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True)


def test_bf16_decode_exhaustive():
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, oracle.BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref, equal_nan=True)


def test_q8_0_decode_exhaustive():
    """Every int8 code times every finite f16 scale equals the exact product."""
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    scales = all_bits[np.isfinite(all_bits.view(np.float16))]
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8).reshape(8, 32)
    nblk = scales.size * 8
    blocks = np.empty((nblk, 34), dtype=np.uint8)
    blocks[:, 0:2] = np.repeat(scales, 8).view(np.uint8).reshape(-1, 2)
    blocks[:, 2:] = np.tile(codes, (scales.size, 1)).view(np.uint8)
    got = oracle.decode(blocks.reshape(-1), oracle.Q8_0).reshape(nblk, 32)
    d = np.repeat(scales, 8).view(np.float16).astype(np.float64)
    ref = np.tile(codes, (scales.size, 1)).astype(np.float64) * d[:, None]
    assert np.array_equal(got, ref)


# ------------------------------------------------------------- helpers
def _problem(n_seq=1, n_tok=1, n_head=2, n_kv=5, dk=16, dv=8, q_type=oracle.BF16,
             kv_type=oracle.BF16, seed=0, mask=None, scale=0.3, gain=1.0):
    g = np.random.default_rng(seed)
    qf = (g.standard_normal((n_seq, n_tok, n_head, dk)) * gain).astype(np.float32)
    kf = g.standard_normal((n_seq, n_kv, dk)).astype(np.float32)
    q = synth.round_bits(qf, q_type)
    kv = synth.quantize_q8_0(kf) if kv_type == oracle.Q8_0 else synth.round_bits(kf, kv_type)
    return dict(q=q, q_type=q_type, kv=kv, kv_type=kv_type, n_seq=n_seq, n_tok=n_tok,
                n_head=n_head, n_kv=n_kv, scale=np.float32(scale), dk=dk, dv=dv, mask=mask)


def _run(p, **kw):
    args = dict(p)
    args.update(kw)
    return oracle.attention(args["q"], args["q_type"], args["kv"], args["kv_type"],
                            args["n_seq"], args["n_tok"], args["n_head"], args["n_kv"],
                            args["scale"], mask=args["mask"], dk=args["dk"], dv=args["dv"],
                            causal=args.get("causal", False),
                            return_stats=args.get("return_stats", False))


def _np_decode(bits, type_id):
    """Independent decoders (numpy / torch) used by the pins, not the oracle's."""
    if type_id == oracle.F16:
        return bits.view(np.float16).astype(np.float64)
    if type_id == oracle.BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError


def _np_dequant_q8_0(rows, dk):
    nb = dk // 32
    r = rows.reshape(-1, nb, 34)
    d = r[:, :, 0:2].copy().view(np.float16).astype(np.float64)  # [n, nb, 1]
    c = r[:, :, 2:].view(np.int8).astype(np.float64)
    return (c * d).reshape(*rows.shape[:-1], dk)


def _kv_f64(p):
    if p["kv_type"] == oracle.Q8_0:
        return _np_dequant_q8_0(p["kv"], p["dk"])
    return _np_decode(p["kv"], p["kv_type"])


# ------------------------------------------------------------- brute force
def _mp_attention(qv, kv, dv, scale, bias):
    import mpmath
    mpmath.mp.dps = 50
    s = []
    for j in range(kv.shape[0]):
        if bias[j] == -math.inf:
            s.append(None)
            continue
        dot = mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b)) for a, b in zip(qv, kv[j]))
        s.append(mpmath.mpf(float(scale)) * dot + mpmath.mpf(float(bias[j])))
    kept = [x for x in s if x is not None]
    if not kept:
        return [0.0] * dv
    m = max(kept)
    w = [mpmath.e ** (x - m) if x is not None else mpmath.mpf(0) for x in s]
    tot = mpmath.fsum(w)
    return [float(mpmath.fsum(w[j] * mpmath.mpf(float(kv[j][d])) for j in range(len(w))) / tot)
            for d in range(dv)]


@pytest.mark.parametrize("kv_type,dk,dv", [(oracle.BF16, 12, 8), (oracle.F16, 9, 9),
                                           (oracle.Q8_0, 64, 32)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_mpmath(kv_type, dk, dv, seed):
    q_type = oracle.F16 if kv_type == oracle.F16 else oracle.BF16
    n_kv = [1, 5, 8][seed]
    g = np.random.default_rng(100 + seed)
    mask = None
    if seed == 2:
        mbits = synth.f32_to_f16_bits(g.uniform(-2, 2, (1, 1, n_kv)).astype(np.float32))
        mbits[0, 0, [1, 4]] = synth.F16_NEG_INF
        mask = mbits
    p = _problem(n_head=2, n_kv=n_kv, dk=dk, dv=dv, q_type=q_type, kv_type=kv_type,
                 seed=seed, mask=mask, gain=2.0)
    got = _run(p)
    qv = _np_decode(p["q"], q_type).reshape(2, dk)
    kvf = _kv_f64(p).reshape(n_kv, dk)
    bias = np.zeros(n_kv) if mask is None else mask.reshape(-1).view(np.float16).astype(np.float64)
    for h in range(2):
        ref = np.array(_mp_attention(qv[h], kvf, dv, p["scale"], bias))
        assert np.allclose(got[h], ref, rtol=1e-12, atol=1e-13), (h, got[h], ref)


# ------------------------------------------------------------- library routine
def _sdpa_ref(p, causal=False):
    """torch float64 SDPA with the single latent head broadcast to every query head."""
    import torch
    dk, dv = p["dk"], p["dv"]
    qv = torch.from_numpy(_np_decode(p["q"], p["q_type"]))  # [S, T, H, dk]
    qv = qv.reshape(p["n_seq"], p["n_tok"], p["n_head"], dk).permute(0, 2, 1, 3)
    kf = torch.from_numpy(_kv_f64(p)).reshape(p["n_seq"], 1, p["n_kv"], dk)
    k = kf.expand(p["n_seq"], p["n_head"], p["n_kv"], dk)
    v = kf[..., :dv].expand(p["n_seq"], p["n_head"], p["n_kv"], dv)
    attn_mask = None
    if p["mask"] is not None:
        mk = torch.from_numpy(p["mask"].view(np.float16).astype(np.float64))
        attn_mask = mk.reshape(p["n_seq"], 1, p["n_tok"], p["n_kv"])
    if causal:
        t = torch.arange(p["n_tok"])[:, None]
        j = torch.arange(p["n_kv"])[None, :]
        cm = torch.where(j > p["n_kv"] - p["n_tok"] + t, -math.inf, 0.0).double()
        attn_mask = cm if attn_mask is None else attn_mask + cm
    o = torch.nn.functional.scaled_dot_product_attention(
        qv, k, v, attn_mask=attn_mask, scale=float(p["scale"]))
    return o.permute(0, 2, 1, 3).reshape(-1, dv).numpy()


@pytest.mark.parametrize("q_type,kv_type", [(oracle.F16, oracle.F16), (oracle.BF16, oracle.BF16),
                                            (oracle.BF16, oracle.Q8_0), (oracle.F16, oracle.Q8_0)])
def test_sdpa_reduced_shape(q_type, kv_type):
    p = _problem(n_seq=2, n_tok=1, n_head=16, n_kv=300, dk=576, dv=512, q_type=q_type,
                 kv_type=kv_type, seed=7, scale=1 / math.sqrt(192))
    got = _run(p)
    ref = _sdpa_ref(p)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_sdpa_with_mask_and_causal():
    g = np.random.default_rng(3)
    n_tok, n_kv = 6, 40
    mbits = synth.f32_to_f16_bits(g.uniform(-3, 3, (1, n_tok, n_kv)).astype(np.float32))
    mbits[g.random((1, n_tok, n_kv)) < 0.3] = synth.F16_NEG_INF
    p = _problem(n_seq=1, n_tok=n_tok, n_head=4, n_kv=n_kv, dk=576, dv=512, seed=4,
                 mask=mbits, scale=1 / math.sqrt(192), gain=3.0)
    got = _run(p, causal=True)
    ref = _sdpa_ref(p, causal=True)
    finite = np.isfinite(ref).all(axis=1)      # SDPA returns NaN for rows with no kept key
    assert finite.sum() > 0
    assert np.allclose(got[finite], ref[finite], rtol=1e-10, atol=1e-12)
    assert np.all(got[~finite] == 0.0)


def test_causal_square_is_torch_is_causal():
    import torch
    p = _problem(n_seq=1, n_tok=24, n_head=3, n_kv=24, dk=64, dv=32, seed=5, scale=0.2)
    got = _run(p, causal=True)
    qv = torch.from_numpy(_np_decode(p["q"], p["q_type"])).reshape(1, 24, 3, 64).permute(0, 2, 1, 3)
    kf = torch.from_numpy(_kv_f64(p)).reshape(1, 1, 24, 64)
    o = torch.nn.functional.scaled_dot_product_attention(
        qv, kf.expand(1, 3, 24, 64), kf[..., :32].expand(1, 3, 24, 32), is_causal=True,
        scale=float(p["scale"]))
    assert np.allclose(got, o.permute(0, 2, 1, 3).reshape(-1, 32).numpy(), rtol=1e-11, atol=1e-13)


def test_sdpa_full_c1_shape():
    prob = synth.make_config(1)
    got = oracle.attention_problem(prob)
    p = dict(q=prob.q, q_type=prob.q_type, kv=prob.kv, kv_type=prob.kv_type, n_seq=1, n_tok=1,
             n_head=16, n_kv=1024, scale=prob.scale, dk=576, dv=512, mask=None)
    assert np.allclose(got, _sdpa_ref(p), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------- invariants
def test_weights_sum_to_one():
    p = _problem(n_head=4, n_kv=50, dk=64, dv=32, seed=11, gain=3.0)
    ones = synth.round_bits(np.ones(1, np.float32), oracle.BF16)[0]
    p["kv"][..., :32] = ones                      # V = all ones, keys still differ in cols 32..63
    out = _run(p)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-13)


def test_single_key_returns_its_v_row():
    p = _problem(n_head=3, n_kv=1, dk=64, dv=48, seed=12, gain=5.0)
    out = _run(p)
    v = _kv_f64(p).reshape(64)[:48]
    assert np.allclose(out, v[None, :], rtol=0, atol=1e-14)


def test_identical_keys_return_mean_of_v():
    """q is zero on every column where keys differ, so all scores are equal."""
    p = _problem(n_head=2, n_kv=17, dk=64, dv=32, seed=13)
    zero = synth.round_bits(np.zeros(1, np.float32), oracle.BF16)[0]
    p["q"][..., :32] = zero                       # q sees only cols 32..63
    p["kv"][0, :, 32:] = p["kv"][0, 0, 32:]       # identical there for every key
    out = _run(p)
    mean_v = _kv_f64(p).reshape(17, 64)[:, :32].mean(axis=0)
    assert np.allclose(out, mean_v[None, :], rtol=1e-13, atol=1e-14)


def test_masked_key_contributes_nothing():
    g = np.random.default_rng(14)
    mask = np.zeros((1, 1, 30), np.uint16)
    mask[0, 0, [3, 17, 29]] = synth.F16_NEG_INF
    p = _problem(n_head=4, n_kv=30, dk=64, dv=32, seed=14, mask=mask, gain=2.0)
    a = _run(p)
    for j in (3, 17, 29):
        p["kv"][0, j] = synth.round_bits(g.standard_normal(64).astype(np.float32) * 100, oracle.BF16)
    b = _run(p)
    assert np.array_equal(a, b)


def test_permutation_of_keys():
    g = np.random.default_rng(15)
    mbits = synth.f32_to_f16_bits(g.uniform(-1, 1, (1, 1, 40)).astype(np.float32))
    mbits[0, 0, ::7] = synth.F16_NEG_INF
    p = _problem(n_head=4, n_kv=40, dk=64, dv=32, seed=15, mask=mbits, gain=2.0)
    a = _run(p)
    perm = g.permutation(40)
    p["kv"] = p["kv"][:, perm]
    p["mask"] = p["mask"][:, :, perm]
    b = _run(p)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_mask_constant_shift():
    g = np.random.default_rng(16)
    vals = g.choice(np.array([0.0, -1.0, -2.5, 0.5], np.float32), size=(1, 1, 33))
    m0 = synth.f32_to_f16_bits(vals)
    m1 = synth.f32_to_f16_bits(vals + np.float32(1.25))   # exact in f16
    m0[0, 0, 5] = m1[0, 0, 5] = synth.F16_NEG_INF
    p = _problem(n_head=3, n_kv=33, dk=64, dv=32, seed=16, mask=m0)
    a = _run(p)
    b = _run(p, mask=m1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_scale_zero_gives_mean_of_kept_v():
    mask = np.zeros((1, 1, 20), np.uint16)
    mask[0, 0, [0, 9]] = synth.F16_NEG_INF
    p = _problem(n_head=2, n_kv=20, dk=64, dv=32, seed=17, mask=mask, scale=0.0, gain=9.0)
    out = _run(p)
    v = _kv_f64(p).reshape(20, 64)[:, :32]
    keep = np.ones(20, bool)
    keep[[0, 9]] = False
    assert np.allclose(out, v[keep].mean(axis=0)[None], rtol=1e-13, atol=1e-14)


def test_two_keys_logistic_closed_form():
    """q and both keys nonzero only in column 0 (exact values): s_i = scale*q0*k_i0,
    p_1 = 1/(1 + exp(s_2 - s_1)), out = p_1 v_1 + p_2 v_2."""
    f = lambda x: synth.round_bits(np.asarray(x, np.float32), oracle.F16)
    q = np.zeros((1, 1, 1, 8), np.uint16)
    q[..., 0] = f(1.5)
    kv = np.zeros((1, 2, 8), np.uint16)
    kv[0, 0] = f([2.0, 0, 0, 0, 1.0, -3.0, 0.25, 0])
    kv[0, 1] = f([-1.0, 0, 0, 0, 4.0, 2.0, 0.5, 1])
    scale = np.float32(0.75)
    out = oracle.attention(q, oracle.F16, kv, oracle.F16, 1, 1, 1, 2, scale, dk=8, dv=8)
    s1, s2 = 0.75 * 1.5 * 2.0, 0.75 * 1.5 * -1.0
    p1 = 1.0 / (1.0 + math.exp(s2 - s1))
    v = np.array([[2.0, 0, 0, 0, 1.0, -3.0, 0.25, 0], [-1.0, 0, 0, 0, 4.0, 2.0, 0.5, 1]])
    assert np.allclose(out[0], p1 * v[0] + (1 - p1) * v[1], rtol=1e-14, atol=1e-15)


def test_causal_equals_explicit_mask():
    n_tok, n_kv = 5, 9
    p = _problem(n_tok=n_tok, n_head=2, n_kv=n_kv, dk=64, dv=32, seed=18)
    a = _run(p, causal=True)
    m = np.zeros((1, n_tok, n_kv), np.uint16)
    for t in range(n_tok):
        m[0, t, n_kv - n_tok + t + 1:] = synth.F16_NEG_INF
    b = _run(p, mask=m)
    assert np.array_equal(a, b)


def test_fully_masked_row_is_zero():
    mask = np.full((1, 1, 12), synth.F16_NEG_INF, np.uint16)
    p = _problem(n_head=2, n_kv=12, dk=64, dv=32, seed=19, mask=mask)
    out, m, l = _run(p, return_stats=True)
    assert np.all(out == 0.0) and np.all(np.isneginf(m)) and np.all(l == 0.0)


def test_row_subset_matches_full():
    prob = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=200, seed=20)
    full = oracle.attention_problem(prob)
    rows = np.array([31, 0, 17, 5])
    sub = oracle.attention_problem(prob, rows=rows)
    assert np.array_equal(sub, full[rows])


def test_statistical_sanity_exponential_tilting():
    """For N(0,1) keys and many cells, out ~ scale * q[:512] (not a pass gate of parity,
    a sanity check that q and k are not transposed or mis-strided)."""
    prob = synth.make_problem(kind="decode", n_seq=1, n_head=8, n_kv=20000, seed=21)
    out = oracle.attention_problem(prob)
    qv = _np_decode(prob.q, prob.q_type).reshape(8, 576)[:, :512] * float(prob.scale)
    corr = np.corrcoef(out.reshape(-1), qv.reshape(-1))[0, 1]
    assert corr > 0.9


# ------------------------------------------------------------- compaction
@pytest.mark.parametrize("case", ["empty", "full", "first", "last", "alternating", "runs"])
def test_compaction_naive_filter(case):
    n = 4099
    bits = np.full(n, synth.F16_NEG_INF, np.uint16)
    if case == "full":
        bits[:] = 0
    elif case == "first":
        bits[0] = 0
    elif case == "last":
        bits[-1] = 0
    elif case == "alternating":
        bits[::2] = 0x3C00
    elif case == "runs":
        bits = synth.sparse_runs_mask(n, np.random.default_rng(5), max_gap=300, max_run=90)
    idx, cnt = oracle.mask_compact(bits)
    ref = np.flatnonzero(bits != synth.F16_NEG_INF)
    assert cnt[0] == ref.size
    assert np.array_equal(idx[0, :cnt[0]], ref)


def test_compaction_keeps_nan_and_finite():
    bits = np.array([0xFC00, 0x7E00, 0x0000, 0x8000, 0xFC00, 0x7C00, 0xFBFF], np.uint16)
    idx, cnt = oracle.mask_compact(bits)
    assert cnt[0] == 5 and list(idx[0, :5]) == [1, 2, 3, 5, 6]


def test_golden_fixtures():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)
    for c in cases["compaction"]:
        bits = synth.f32_to_f16_bits(np.array(c["mask"], np.float32))
        idx, cnt = oracle.mask_compact(bits)
        assert cnt[0] == c["count"] and list(idx[0, :cnt[0]]) == c["idx"], c["cite"]
    for c in cases["attention"]:
        f = lambda x: synth.round_bits(np.asarray(x, np.float32), oracle.F16)
        dk = len(c["q"])
        q = f(c["q"]).reshape(1, 1, 1, dk)
        kv = f(c["keys"]).reshape(1, -1, dk)
        n_kv = kv.shape[1]
        mask = None if c.get("mask") is None else f(c["mask"]).reshape(1, 1, n_kv)
        out = oracle.attention(q, oracle.F16, kv, oracle.F16, 1, 1, 1, n_kv,
                               np.float32(c["scale"]), mask=mask, dk=dk, dv=c["dv"])
        assert np.allclose(out[0], c["out"], rtol=1e-12, atol=1e-14), c["cite"]
    for c in cases["causal_visibility"]:
        n_tok, n_kv = c["n_tok"], c["n_kv"]
        for t, vis in enumerate(c["visible"]):
            assert [j for j in range(n_kv) if j <= n_kv - n_tok + t] == vis, c["cite"]
    facts = cases["page_facts"]
    assert facts["kv_lora_rank"] + facts["n_embd_head_qk_rope"] == facts["latent_row"] == synth.DK
    assert synth.q8_0_row_bytes() == facts["latent_row"] // 32 * facts["q8_0_block_bytes"]
    assert facts["score_matrix_bytes"] == facts["score_seq"] ** 2 * 4
