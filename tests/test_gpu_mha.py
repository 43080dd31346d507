"""GPU parity of mla_fa_prefill_mha (per-head attention, 192-wide keys and 128-wide values:
the non-absorbed MLA prefill shape) against the fp64 oracle: relative L2 <= 5e-3 and max
|error| <= 2e-2 over the whole output, the bar of the latent path's parity tests."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, to_dev

pytestmark = pytest.mark.gpu

BF16, F16 = synth.TYPE_BF16, synth.TYPE_F16
DK, DV = synth.MHA_DK, synth.MHA_DV


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def _padded(a: np.ndarray, width: int):
    """Rows of `a` (uint16, last dim flattened) placed in a wider device buffer; returns
    the strided view with a.shape."""
    import torch
    n = a.shape[0]
    flat = np.ascontiguousarray(a).reshape(n, -1)
    buf = np.zeros((n, width), dtype=np.uint16)
    buf[:, :flat.shape[1]] = flat
    t = to_dev(buf)
    return torch.as_strided(t, a.shape, (width,) + tuple(int(np.prod(a.shape[i + 1:])) for i in range(1, a.ndim)))


def run_mha(p, k_pad=0, v_pad=0, mask_pad=None):
    """Run the per-head kernel on problem p; k_pad / v_pad extra elements per key row,
    mask_pad the mask row stride (None = n_kv rounded up to 8)."""
    import torch
    from mla_flash_attention_amd import binding as B
    q = to_dev(p.q)
    k = _padded(p.k, p.n_head * DK + k_pad) if k_pad else to_dev(p.k)
    v = _padded(p.v, p.n_head * DV + v_pad) if v_pad else to_dev(p.v)
    mask = None
    if p.mask is not None:
        ms = mask_pad if mask_pad is not None else (p.n_kv + 7) // 8 * 8
        mask = _padded(p.mask, ms)
    out = torch.full((p.n_tok, p.n_head, DV), float("nan"), dtype=torch.float32, device="cuda")
    B.mla_fa_prefill_mha(q, p.q_type, k, v, p.kv_type, p.scale, out, causal=p.causal, mask=mask)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, DV).astype(np.float64)


def ref_mha(p, rows=None):
    return oracle.mha_attention(p.q, p.q_type, p.k, p.v, p.kv_type, p.scale, causal=p.causal, mask=p.mask,
                                rows=rows)


@pytest.mark.parametrize("n_tok,n_head,n_kv,t,causal,seed", [
    (300, 4, 400, BF16, True, 1),     # two token tiles, ragged; chunk at the end of a longer cache
    (300, 4, 300, F16, True, 2),      # square causal: token 0 sees one key
    (257, 3, 257, BF16, True, 3),     # one token past a tile; odd head count
    (64, 2, 1000, BF16, False, 4),    # non-causal, ragged last key tile
    (1, 8, 77, F16, False, 5),        # one token
    (1, 8, 1, BF16, True, 6),         # one token, one key
    (700, 2, 700, F16, True, 7),      # three token tiles, 11 key tiles
])
def test_mha_dense(n_tok, n_head, n_kv, t, causal, seed):
    p = synth.make_mha_problem(n_tok, n_head, n_kv, t, t, seed=seed, causal=causal)
    got = run_mha(p)
    assert_parity(got, ref_mha(p), f"mha {n_tok}x{n_head} n_kv={n_kv} causal={causal}")


@pytest.mark.parametrize("mask_kind,n_kv,causal,t", [
    ("random", 333, False, BF16),     # row length not a multiple of 8 (stride padded to 336)
    ("runs_bias", 520, True, F16),
    ("random", 256, True, BF16),      # tight stride: mask rows exactly n_kv long
])
def test_mha_masked(mask_kind, n_kv, causal, t):
    n_tok = min(260, n_kv) if causal else 96
    p = synth.make_mha_problem(n_tok, 2, n_kv, t, t, seed=11, causal=causal, mask_kind=mask_kind)
    got = run_mha(p, mask_pad=n_kv if n_kv % 8 == 0 else None)
    assert_parity(got, ref_mha(p), f"mha mask {mask_kind} n_kv={n_kv}")


def test_mha_none_kept_rows_are_zero():
    p = synth.make_mha_problem(40, 2, 130, BF16, BF16, seed=12, causal=False, mask_kind="random")
    p.mask[5] = synth.F16_NEG_INF
    p.mask[33] = synth.F16_NEG_INF
    got = run_mha(p).reshape(p.n_tok, p.n_head, DV)
    assert np.all(got[5] == 0.0) and np.all(got[33] == 0.0)
    assert_parity(got.reshape(-1, DV), ref_mha(p), "mha rows with no kept key")


def test_mha_strided_rows():
    p = synth.make_mha_problem(200, 4, 260, BF16, BF16, seed=13, causal=True)
    got = run_mha(p, k_pad=64, v_pad=8)
    assert_parity(got, ref_mha(p), "mha strided K/V rows")


def test_mha_large_scores():
    # scale 1: scores in the tens, so the running max moves by more than the lazy-rescale threshold
    p = synth.make_mha_problem(320, 2, 640, F16, F16, seed=14, causal=True, scale=1.0)
    got = run_mha(p)
    assert_parity(got, ref_mha(p), "mha large scores")


def test_mha_repeat_is_bitwise_stable():
    p = synth.make_mha_problem(300, 2, 500, BF16, BF16, seed=15, causal=True)
    a, b = run_mha(p), run_mha(p)
    assert np.array_equal(a, b)


def test_mha_full_size():
    """2048 tokens x 128 heads over a 4096-key cache (causal), the benched launch: every
    output row against the oracle."""
    n_tok, n_head, n_kv = 2048, 128, 4096
    p = synth.make_mha_problem(n_tok, n_head, n_kv, BF16, BF16, seed=16, causal=True)
    got = run_mha(p)
    assert_parity(got, ref_mha(p), "mha 2048x128 n_kv=4096")
