"""GPU parity of sparse attention with one mask row per query token: every (sequence,
token) row's f16 mask is compacted to its ascending list of kept cells (multi-row
fa_mask_compact / fa_mask_compact_ws), and mla_fa_attend attends each row over its own
list ("llama.cpp Vulkan backend adds sparse Flash Attention for quantized K/V": sparse FA
for quantised K/V, compaction per mask row, 128k cells).  The lists must match the
oracle's naive filter bit for bit; the outputs must match the oracle's dense masked
attention (a dropped cell contributes nothing) to the usual bar: whole-output relative L2
<= 5e-3, max |error| <= 2e-2."""
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


def run_sparse_attend(p, n_split=0, chunked=True):
    """Compact the n_seq*n_tok mask rows, then attend through the lists.
    Returns (out [rows*heads][512] float64, idx [rows][n_kv], count [rows])."""
    import torch
    from mla_flash_attention_amd import binding as B
    rows = p.n_seq * p.n_tok
    mask = to_dev(p.mask.reshape(rows, p.n_kv))
    idx = torch.full((rows, p.n_kv), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    if chunked:
        need = B.fa_mask_compact_workspace_size(rows, p.n_kv)
        cws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        B.fa_mask_compact_ws(mask, idx, cnt, cws if need else None)
    else:
        B.fa_mask_compact(mask, idx, cnt)
    q = to_dev(p.q)
    kv = to_dev(p.kv)
    out = torch.full((p.n_seq, p.n_tok, p.n_head, synth.DV), float("nan"), dtype=torch.float32, device="cuda")
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ws = B.workspace_for(rows, p.n_head, p.n_kv, p.kv_type, n_split)
    B.mla_fa_attend(q, p.q_type, kv, p.kv_type, p.scale, out, mask=to_dev(p.mask),
                    kv_idx=idx.view(p.n_seq, p.n_tok, p.n_kv), kv_idx_count=cnt.view(p.n_seq, p.n_tok),
                    alibi=f(p.alibi), sinks=f(p.sinks), softcap=p.softcap, n_split=n_split, workspace=ws)
    torch.cuda.synchronize()
    return (out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64), idx.cpu().numpy(),
            cnt.cpu().numpy())


def check(p, label, n_split=0, chunked=True):
    got, idx, cnt = run_sparse_attend(p, n_split=n_split, chunked=chunked)
    idx_ref, cnt_ref = oracle.mask_compact(p.mask.reshape(p.n_seq * p.n_tok, p.n_kv))
    assert np.array_equal(cnt, cnt_ref), label
    for r in range(cnt.size):
        assert np.array_equal(idx[r, :cnt[r]], idx_ref[r, :cnt[r]]), f"{label}: row {r}"
    return assert_parity(got, oracle.attention_problem(p), label)


def causal_runs(p):
    """Drop, in each token's mask row, the cells past that token's causal edge (token t of
    n_tok sees cells j <= n_kv - n_tok + t): causality expressed through the mask."""
    for t in range(p.n_tok):
        p.mask[:, t, p.n_kv - p.n_tok + t + 1:] = synth.F16_NEG_INF
    return p


@pytest.mark.parametrize("kv_type,q_type", [(BF16, BF16), (F16, F16), (Q8, BF16), (Q8, F16)])
@pytest.mark.parametrize("n_split", [1, 0])
def test_sparse_multi_token(kv_type, q_type, n_split):
    p = synth.make_problem(kind="sparse", n_seq=2, n_tok=3, n_head=128, n_kv=9000, q_type=q_type,
                           kv_type=kv_type, seed=70 + kv_type, mask_kind="runs_bias")
    check(causal_runs(p), f"sparse tokens kv{kv_type} q{q_type} split{n_split}", n_split)


@pytest.mark.parametrize("chunked", [False, True])
def test_sparse_multi_token_extras(chunked):
    """Per-token lists with sinks, softcap and ALiBi slopes over a distance mask whose far
    cells are dropped (so the lists are the runs of nearby cells)."""
    p = synth.make_problem(kind="decode", n_seq=2, n_tok=2, n_head=64, n_kv=3000, q_type=BF16, kv_type=Q8,
                           seed=75, mask_kind="distance", alibi=True, sinks=True, softcap=25.0)
    far = p.mask.view(np.float16).astype(np.float32) < -300
    p.mask[far] = synth.F16_NEG_INF
    check(p, f"sparse tokens extras chunked={chunked}", chunked=chunked)


def test_sparse_rows_with_no_kept_cell():
    p = synth.make_problem(kind="sparse", n_seq=2, n_tok=2, n_head=16, n_kv=700, seed=76, sinks=True)
    p.mask[0, 1] = synth.F16_NEG_INF
    p.mask[1, 0] = synth.F16_NEG_INF
    check(p, "sparse rows with none kept")
    got, _, _ = run_sparse_attend(p)
    got = got.reshape(2, 2, 16, synth.DV)
    assert np.all(got[0, 1] == 0) and np.all(got[1, 0] == 0)


@pytest.mark.parametrize("n_tok", [1, 2])
def test_sparse_q8_0_131072_cells(n_tok):
    """The sparse workload's shape over a Q8_0 cache: 131,072 cells, 128 heads, ~10% kept
    in runs of 1-256 (one mask row per query token), automatic split count, chunked
    compaction; the whole output against the oracle."""
    p = synth.make_problem(kind="sparse", n_seq=1, n_tok=n_tok, n_head=128, n_kv=131072, q_type=BF16,
                           kv_type=Q8, seed=5)
    check(p, f"sparse q8_0 131072 x {n_tok} tok")
