"""GPU parity of the pair kernel (the p64 / p128 workgroup shapes, selected here through
the MLA_FA_SHAPE tuning override): the same oracle and tolerances as the other parity
tests, over cases that reach every branch of its stage pipeline: one-stage and ragged
last stages, head sets padded with absent heads, split and unsplit calls, masks with
fully masked stages, causal prefill, f16 and bf16, and rows whose scores keep rising."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, run_decode, run_prefill

pytestmark = pytest.mark.gpu

BF16, F16 = synth.TYPE_BF16, synth.TYPE_F16
SHAPES = ["p64", "p128"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("n_kv,n_head,n_split", [(1, 128, 1), (31, 128, 0), (33, 80, 2), (95, 16, 1),
                                                 (1000, 128, 0), (4097, 64, 3), (4096, 112, 1)])
def test_pair_decode(shape, n_kv, n_head, n_split, monkeypatch):
    monkeypatch.setenv("MLA_FA_SHAPE", shape)
    p = synth.make_problem(kind="decode", n_seq=2, n_head=n_head, n_kv=n_kv, q_type=BF16, kv_type=BF16,
                           seed=7 * n_kv + n_head)
    got, _ = run_decode(p, n_split=n_split)
    assert_parity(got, oracle.attention_problem(p), f"{shape} decode kv{n_kv} h{n_head} split{n_split}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mask_kind", ["random", "runs_bias", "none_kept"])
def test_pair_masked_f16(shape, mask_kind, monkeypatch):
    monkeypatch.setenv("MLA_FA_SHAPE", shape)
    p = synth.make_problem(kind="decode", n_seq=2, n_head=128, n_kv=3000, q_type=F16, kv_type=F16,
                           seed=11, mask_kind=mask_kind)
    got, _ = run_decode(p, n_split=4)
    assert_parity(got, oracle.attention_problem(p), f"{shape} masked {mask_kind}")


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("n_tok,n_kv", [(1, 1), (5, 7), (70, 300), (128, 1000)])
def test_pair_prefill_causal(shape, n_tok, n_kv, monkeypatch):
    monkeypatch.setenv("MLA_FA_SHAPE", shape)
    p = synth.make_problem(kind="prefill", n_tok=n_tok, n_head=128, n_kv=n_kv, q_type=BF16, kv_type=BF16,
                           seed=n_tok + n_kv, causal=True)
    got = run_prefill(p)
    assert_parity(got, oracle.attention_problem(p), f"{shape} prefill t{n_tok} kv{n_kv}")


@pytest.mark.parametrize("shape", SHAPES)
def test_pair_rising_scores(shape, monkeypatch):
    """Every stage raises the running max (a RoPE dim grows with the key index), so every
    stage rescales O through the published factors."""
    monkeypatch.setenv("MLA_FA_SHAPE", shape)
    p = synth.make_problem(kind="decode", n_seq=1, n_head=128, n_kv=700, q_type=BF16, kv_type=BF16, seed=3)
    # rise per 32-key stage: 32 * 0.6 * 4 * scale * log2(e) ~ 8 log2 units, the lazy
    # rescale threshold, so the running max is replaced at almost every stage
    kvf = np.zeros((1, 700, synth.DK), dtype=np.float32)
    kvf[0, :, :512] = np.random.default_rng(1).standard_normal((700, 512), dtype=np.float32)
    kvf[0, :, 575] = np.arange(700, dtype=np.float32) * 0.6
    p.kv = synth.round_bits(kvf, BF16)
    qf = np.zeros((1, 1, 128, synth.DK), dtype=np.float32)
    qf[..., 575] = 4.0
    qf[..., :512] = np.random.default_rng(2).standard_normal((1, 1, 128, 512), dtype=np.float32)
    p.q = synth.round_bits(qf, BF16)
    got, _ = run_decode(p, n_split=1)
    assert_parity(got, oracle.attention_problem(p), f"{shape} rising scores")
