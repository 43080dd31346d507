"""GPU parity of mla_fa_absorbed (latent attention with the per-head W_UK / W_UV
projections either side) against the fp64 oracle, to the bar of the other parity tests:
relative L2 <= 5e-3 and max |error| <= 2e-2 over the whole output."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, to_dev

pytestmark = pytest.mark.gpu

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def run_absorbed(p, n_split=0):
    import torch
    from mla_flash_attention_amd import binding as B
    out = torch.full((p.n_seq, p.n_tok, p.n_head, 128), float("nan"), dtype=torch.float32, device="cuda")
    kv_len = None if p.kv_len is None else torch.from_numpy(np.ascontiguousarray(p.kv_len)).cuda()
    B.mla_fa_absorbed(to_dev(p.q_nope), to_dev(p.q_pe), p.q_type, to_dev(p.w_uk), to_dev(p.w_uv), to_dev(p.kv),
                      p.kv_type, p.scale, out, kv_len=kv_len, causal=p.causal,
                      mask=None if p.mask is None else to_dev(p.mask), n_split=n_split)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, 128).astype(np.float64)


def ref_absorbed(p, rows=None):
    return oracle.absorbed_attention(p.q_nope, p.q_pe, p.q_type, p.w_uk, p.w_uv, p.kv, p.kv_type, p.n_seq, p.n_tok,
                                     p.n_head, p.n_kv, p.scale, causal=p.causal, mask=p.mask, kv_len=p.kv_len,
                                     rows=rows)


@pytest.mark.parametrize("kw,n_split", [
    (dict(n_seq=2, n_tok=1, n_head=16, n_kv=300, q_type=BF16, kv_type=BF16, seed=1), 0),
    (dict(n_seq=2, n_tok=1, n_head=16, n_kv=300, q_type=BF16, kv_type=BF16, seed=1), 1),
    (dict(n_seq=2, n_tok=1, n_head=32, n_kv=1000, q_type=F16, kv_type=F16, seed=2), 4),
    (dict(n_seq=2, n_tok=1, n_head=16, n_kv=700, q_type=F16, kv_type=Q8, seed=3), 0),
    (dict(n_seq=3, n_tok=3, n_head=32, n_kv=500, q_type=BF16, kv_type=BF16, seed=4, causal=True, ragged=True), 0),
    (dict(n_seq=2, n_tok=2, n_head=16, n_kv=400, q_type=BF16, kv_type=BF16, seed=5, mask_kind="runs_bias"), 2),
    (dict(n_seq=1, n_tok=200, n_head=16, n_kv=400, q_type=BF16, kv_type=BF16, seed=6, causal=True), 1),
    (dict(n_seq=1, n_tok=130, n_head=48, n_kv=260, q_type=F16, kv_type=F16, seed=7, causal=True), 0),
    # 16 and 17 rows with splits (decode-sized batches), a Q8_0 cache at 128 heads
    (dict(n_seq=8, n_tok=2, n_head=64, n_kv=900, q_type=BF16, kv_type=BF16, seed=10, causal=True), 3),
    (dict(n_seq=17, n_tok=1, n_head=32, n_kv=700, q_type=F16, kv_type=F16, seed=11), 5),
    (dict(n_seq=3, n_tok=1, n_head=128, n_kv=2000, q_type=BF16, kv_type=Q8, seed=12), 0),
    # many splits: the fused merge's later load batches (more than 32 splits), and 1024
    # splits over 2000 cells, where most splits are empty
    (dict(n_seq=5, n_tok=1, n_head=64, n_kv=9000, q_type=BF16, kv_type=BF16, seed=13), 100),
    (dict(n_seq=2, n_tok=1, n_head=16, n_kv=2000, q_type=F16, kv_type=F16, seed=14), 1024),
])
def test_absorbed(kw, n_split):
    p = synth.make_absorbed_problem(**kw)
    got = run_absorbed(p, n_split)
    assert_parity(got, ref_absorbed(p), f"absorbed {kw} split={n_split}")


def test_absorbed_repeat_is_bitwise_stable():
    p = synth.make_absorbed_problem(2, 2, 16, 333, BF16, BF16, seed=8, causal=True)
    assert np.array_equal(run_absorbed(p, 2), run_absorbed(p, 2))


def test_absorbed_full_size_decode():
    """4 sequences x 128 heads over 32768-cell caches (the decode workload's shape), the
    benched launch: every output row against the oracle."""
    p = synth.make_absorbed_problem(4, 1, 128, 32768, BF16, BF16, seed=9)
    got = run_absorbed(p)
    assert_parity(got, ref_absorbed(p), "absorbed 4x128h n_kv=32768")
