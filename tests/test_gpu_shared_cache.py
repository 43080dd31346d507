"""GPU parity when several sequences attend to one cache (kv_seq_stride = 0, passed by
the binding for a [1][n_kv][row] cache): a shared prefix, as with parallel sampling or
beam search.  Each sequence keeps its own query, mask, length and index list; only the
cache rows are common.  Whole outputs against the oracle (which reads the same single
cache for every sequence), at the usual bar: relative L2 <= 5e-3, max |error| <= 2e-2."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, run_decode, to_dev

pytestmark = pytest.mark.gpu

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def shared(p):
    """Keep the first sequence's cache as the one cache of every sequence."""
    p.kv = np.ascontiguousarray(p.kv[:1])
    return p


@pytest.mark.parametrize("kv_type,q_type,n_split", [(BF16, BF16, 0), (Q8, BF16, 0), (F16, F16, 1), (Q8, F16, 3)])
def test_shared_cache_decode(kv_type, q_type, n_split):
    p = shared(synth.make_problem(kind="decode", n_seq=4, n_head=128, n_kv=6000, q_type=q_type, kv_type=kv_type,
                                  seed=101 + kv_type, mask_kind="runs_bias"))
    got, _ = run_decode(p, n_split=n_split)
    assert_parity(got, oracle.attention_problem(p), f"shared decode kv{kv_type} split{n_split}")


def test_shared_cache_sparse():
    """Per-sequence mask rows compacted to per-sequence lists over the one cache."""
    p = shared(synth.make_problem(kind="sparse", n_seq=3, n_head=64, n_kv=30000, q_type=BF16, kv_type=Q8, seed=105))
    got, ex = run_decode(p, chunked=True)
    idx_ref, cnt_ref = oracle.mask_compact(p.mask.reshape(p.n_seq, p.n_kv))
    cnt = ex["count"].cpu().numpy()
    assert np.array_equal(cnt, cnt_ref)
    idx = ex["idx"].cpu().numpy()
    for s in range(p.n_seq):
        assert np.array_equal(idx[s, :cnt[s]], idx_ref[s, :cnt[s]])
    assert_parity(got, oracle.attention_problem(p), "shared sparse")


@pytest.mark.parametrize("n_split", [1, 0])
def test_shared_cache_ragged_attend(n_split):
    """Prefixes of one cache: every sequence sees its own valid length of the common
    rows, two causal query tokens each."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = shared(synth.make_problem(kind="decode", n_seq=5, n_tok=2, n_head=64, n_kv=4000, q_type=BF16, kv_type=BF16,
                                  seed=106, ragged=True, causal=True))
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ws = B.workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, n_split)
    B.mla_fa_attend(to_dev(p.q), p.q_type, to_dev(p.kv), p.kv_type, p.scale, out,
                    kv_len=torch.from_numpy(np.ascontiguousarray(p.kv_len)).cuda(), causal=True, n_split=n_split,
                    workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64)
    assert_parity(got, oracle.attention_problem(p), f"shared ragged split{n_split}")


def test_shared_cache_absorbed():
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_absorbed_problem(n_seq=4, n_tok=1, n_head=128, n_kv=3000, q_type=BF16, kv_type=BF16, seed=107)
    p.kv = np.ascontiguousarray(p.kv[:1])
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, 128), dtype=torch.float32, device="cuda")
    B.mla_fa_absorbed(to_dev(p.q_nope), to_dev(p.q_pe), p.q_type, to_dev(p.w_uk), to_dev(p.w_uv), to_dev(p.kv),
                      p.kv_type, p.scale, out)
    torch.cuda.synchronize()
    ref = oracle.absorbed_attention(p.q_nope, p.q_pe, p.q_type, p.w_uk, p.w_uv, p.kv, p.kv_type, p.n_seq, p.n_tok,
                                    p.n_head, p.n_kv, p.scale)
    assert_parity(out.cpu().numpy().reshape(-1, 128).astype(np.float64), ref, "shared absorbed")
