"""GPU parity of mla_fa_attend (per-sequence valid lengths, multi-token causal rows, logit
softcap, ALiBi slopes, attention sinks) against the fp64 oracle, to the same bar as the
other parity tests: relative L2 <= 5e-3 and max |error| <= 2e-2 over the whole output."""
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


def run_attend(p, n_split=0):
    import torch
    from mla_flash_attention_amd import binding as B
    q = to_dev(p.q)
    kv = to_dev(p.kv)
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    mask = None if p.mask is None else to_dev(p.mask)
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = B.workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, n_split)
    B.mla_fa_attend(q, p.q_type, kv, p.kv_type, p.scale, out, kv_len=f(p.kv_len), causal=p.causal,
                    mask=mask, alibi=f(p.alibi), sinks=f(p.sinks), softcap=p.softcap, n_split=n_split,
                    workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64)


def _case(label, n_split=0, **kw):
    p = synth.make_problem(kind="decode", **kw)
    got = run_attend(p, n_split=n_split)
    return assert_parity(got, oracle.attention_problem(p), label)


@pytest.mark.parametrize("n_split", [1, 0])
def test_ragged_decode(n_split):
    _case(f"ragged split{n_split}", n_split, n_seq=4, n_head=128, n_kv=3000, seed=41, ragged=True)


@pytest.mark.parametrize("n_split", [1, 3, 0])
def test_ragged_multi_token_causal(n_split):
    _case(f"ragged causal split{n_split}", n_split, n_seq=3, n_tok=4, n_head=64, n_kv=700, seed=42,
          ragged=True, causal=True)


@pytest.mark.parametrize("softcap", [2.0, 30.0])
@pytest.mark.parametrize("n_split", [1, 0])
def test_softcap(softcap, n_split):
    _case(f"softcap {softcap} split{n_split}", n_split, n_seq=2, n_head=128, n_kv=2000, seed=43,
          softcap=softcap, q_gain=2.0)


@pytest.mark.parametrize("n_split", [1, 0])
def test_alibi_distance_mask(n_split):
    _case(f"alibi split{n_split}", n_split, n_seq=2, n_tok=3, n_head=128, n_kv=1500, seed=44, ragged=True,
          alibi=True, mask_kind="distance", causal=True)


@pytest.mark.parametrize("n_split", [1, 2, 0])
def test_sinks(n_split):
    _case(f"sinks split{n_split}", n_split, n_seq=2, n_head=128, n_kv=1000, seed=45, sinks=True,
          mask_kind="runs_bias")


@pytest.mark.parametrize("kv_type,q_type", [(BF16, BF16), (F16, F16), (Q8, BF16), (Q8, F16)])
@pytest.mark.parametrize("n_split", [1, 0])
def test_everything_combined(kv_type, q_type, n_split):
    _case(f"combined kv{kv_type} q{q_type} split{n_split}", n_split, n_seq=3, n_tok=2, n_head=80, n_kv=1300,
          seed=46, q_type=q_type, kv_type=kv_type, ragged=True, causal=True, alibi=True,
          mask_kind="distance", sinks=True, softcap=20.0)


@pytest.mark.parametrize("n_split", [1, 0])
def test_empty_and_short_sequences(n_split):
    """Lengths 0, 1 and n_tok - 1 (causal rows left with no cell output 0, with or without a sink)."""
    p = synth.make_problem(kind="decode", n_seq=4, n_tok=3, n_head=16, n_kv=200, seed=47, causal=True,
                           sinks=True)
    p.kv_len = np.array([0, 1, 2, 200], dtype=np.int32)
    got = run_attend(p, n_split=n_split)
    ref = oracle.attention_problem(p)
    assert_parity(got, ref, f"empty/short split{n_split}")
    assert np.all(got[:3 * 16] == 0)


def test_pair_shape_request_falls_back_with_extras(monkeypatch):
    monkeypatch.setenv("MLA_FA_SHAPE", "p128")
    _case("p128 request with extras", 0, n_seq=2, n_head=128, n_kv=900, seed=48, ragged=True, sinks=True,
          softcap=15.0)


@pytest.mark.parametrize("n_head", [16, 48])
def test_small_head_counts(n_head):
    _case(f"h{n_head} extras", 0, n_seq=2, n_tok=2, n_head=n_head, n_kv=400, seed=49 + n_head, ragged=True,
          causal=True, sinks=True, alibi=True, mask_kind="distance")


@pytest.mark.parametrize("variant", ["plain", "softcap_sinks_alibi"])
def test_ragged_full_size(variant):
    """The benched ragged workload at full size in its launch configuration: 8 sequences of
    U{2..32768} valid cells x 2 causal query tokens x 128 heads, automatic split count;
    plain, and with softcap 50, sinks and ALiBi over a distance mask.  Whole output."""
    kw = {} if variant == "plain" else dict(softcap=50.0, sinks=True, alibi=True, mask_kind="distance")
    _case(f"ragged full {variant}", 0, n_seq=8, n_tok=2, n_head=128, n_kv=32768, seed=6, ragged=True,
          causal=True, **kw)
