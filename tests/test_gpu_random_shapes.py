"""Seeded random configurations of every entry point against the fp64 oracle, to the
same bar as the other parity tests (relative L2 <= 5e-3, max |error| <= 2e-2; compaction
bit-exact).  Each case draws its parameters from a generator seeded by the case number,
within the documented ranges, at sizes the oracle finishes quickly; the drawn parameters
are part of the failure message."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, run_decode, run_prefill

pytestmark = pytest.mark.gpu

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0
N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def _types(g):
    kv = [BF16, F16, Q8][int(g.integers(3))]
    q = {BF16: BF16, F16: F16, Q8: [BF16, F16][int(g.integers(2))]}[kv]
    return q, kv


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode(case):
    g = np.random.default_rng(9000 + case)
    q_type, kv_type = _types(g)
    kind = ["decode", "sparse"][int(g.integers(2))]
    kw = dict(kind=kind, n_seq=int(g.integers(1, 5)), n_head=16 * int(g.integers(1, 9)),
              n_kv=int(g.integers(1, 5000)), q_type=q_type, kv_type=kv_type, seed=int(g.integers(1 << 30)))
    if kind == "decode" and g.random() < 0.5:
        kw["mask_kind"] = ["runs", "runs_bias", "random"][int(g.integers(3))]
    if g.random() < 0.3:
        kw["q_gain"] = float(g.choice([0.25, 4.0]))
    n_split = int(g.choice([0, 0, 1, 2, 7]))
    p = synth.make_problem(**kw)
    got, _ = run_decode(p, n_split=n_split)
    assert_parity(got, oracle.attention_problem(p), f"decode case {case}: {kw} n_split={n_split}")


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_random_prefill(case):
    g = np.random.default_rng(9100 + case)
    q_type, kv_type = _types(g)
    n_kv = int(g.integers(1, 1200))
    causal = bool(g.random() < 0.7)
    n_tok = int(g.integers(1, n_kv + 1)) if causal else int(g.integers(1, 300))
    kw = dict(kind="prefill", n_tok=n_tok, n_head=16 * int(g.integers(1, 9)), n_kv=n_kv, q_type=q_type,
              kv_type=kv_type, seed=int(g.integers(1 << 30)), causal=causal)
    if g.random() < 0.3:
        kw["mask_kind"] = "runs_bias"
    p = synth.make_problem(**kw)
    got = run_prefill(p, n_split=int(g.choice([1, 1, 3])))
    assert_parity(got, oracle.attention_problem(p), f"prefill case {case}: {kw}")


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_random_attend(case):
    from tests.test_gpu_attend import run_attend
    g = np.random.default_rng(9200 + case)
    q_type, kv_type = _types(g)
    n_tok = int(g.integers(1, 4))
    kw = dict(kind="decode", n_seq=int(g.integers(1, 5)), n_tok=n_tok, n_head=16 * int(g.integers(1, 9)),
              n_kv=int(g.integers(n_tok, 3000)), q_type=q_type, kv_type=kv_type, seed=int(g.integers(1 << 30)),
              ragged=bool(g.random() < 0.7), causal=bool(g.random() < 0.6))
    if g.random() < 0.4:
        kw["softcap"] = float(g.choice([5.0, 30.0]))
    if g.random() < 0.4:
        kw["sinks"] = True
    if g.random() < 0.4:
        kw["alibi"] = True
        kw["mask_kind"] = "distance"
    p = synth.make_problem(**kw)
    n_split = int(g.choice([0, 1, 3]))
    got = run_attend(p, n_split=n_split)
    assert_parity(got, oracle.attention_problem(p), f"attend case {case}: {kw} n_split={n_split}")


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_random_compaction(case):
    import torch
    from mla_flash_attention_amd import binding as B
    from tests.gpu_common import to_dev
    g = np.random.default_rng(9300 + case)
    n_rows, n = int(g.integers(1, 6)), int(g.integers(1, 200000))
    density = float(g.choice([0.0, 0.01, 0.1, 0.5, 0.99, 1.0]))
    m = np.where(g.random((n_rows, n)) < density, np.uint16(0), np.uint16(synth.F16_NEG_INF)).astype(np.uint16)
    stride = n + int(g.integers(0, 20))
    host = np.full((n_rows, stride), 0x1234, np.uint16)
    host[:, :n] = m
    mask = to_dev(host)[:, :n]
    idx_ref, cnt_ref = oracle.mask_compact(m)
    for entry in ("one", "chunked"):
        idx = torch.full((n_rows, n), -9, dtype=torch.int32, device="cuda")
        cnt = torch.full((n_rows,), -9, dtype=torch.int32, device="cuda")
        if entry == "one":
            B.fa_mask_compact(mask, idx, cnt)
        else:
            need = B.fa_mask_compact_workspace_size(n_rows, n)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            B.fa_mask_compact_ws(mask, idx, cnt, ws)
        torch.cuda.synchronize()
        ci, ii = cnt.cpu().numpy(), idx.cpu().numpy()
        what = f"compaction case {case} ({entry}): rows {n_rows} n {n} stride {stride} density {density}"
        assert np.array_equal(ci, cnt_ref), what
        for r in range(n_rows):
            assert np.array_equal(ii[r, :ci[r]], idx_ref[r, :ci[r]]), what
            assert np.all(ii[r, ci[r]:] == -9), what


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_random_prefill_mha(case):
    from tests.test_gpu_mha import ref_mha, run_mha
    g = np.random.default_rng(9400 + case)
    t = [BF16, F16][int(g.integers(2))]
    n_kv = int(g.integers(1, 1500))
    causal = bool(g.random() < 0.7)
    n_tok = int(g.integers(1, n_kv + 1)) if causal else int(g.integers(1, 600))
    kw = dict(n_tok=n_tok, n_head=int(g.integers(1, 5)), n_kv=n_kv, q_type=t, kv_type=t,
              seed=int(g.integers(1 << 30)), causal=causal)
    if g.random() < 0.3:
        kw["mask_kind"] = "runs_bias"
    p = synth.make_mha_problem(**kw)
    assert_parity(run_mha(p), ref_mha(p), f"per-head prefill case {case}: {kw}")


@pytest.mark.parametrize("case", range(N_CASES // 3))
def test_random_absorbed(case):
    from tests.test_gpu_absorbed import ref_absorbed, run_absorbed
    g = np.random.default_rng(9500 + case)
    q_type, kv_type = _types(g)
    n_tok = int(g.integers(1, 4))
    kw = dict(n_seq=int(g.integers(1, 4)), n_tok=n_tok, n_head=16 * int(g.integers(1, 5)),
              n_kv=int(g.integers(n_tok, 2000)), q_type=q_type, kv_type=kv_type, seed=int(g.integers(1 << 30)),
              causal=bool(g.random() < 0.5), ragged=bool(g.random() < 0.5))
    p = synth.make_absorbed_problem(**kw)
    n_split = int(g.choice([0, 1, 3]))
    assert_parity(run_absorbed(p, n_split=n_split), ref_absorbed(p), f"absorbed case {case}: {kw} n_split={n_split}")
