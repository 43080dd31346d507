"""GPU parity of split calls whose rows carry device-side lengths (mla_fa_attend with
per-sequence valid lengths, or with per-row index lists).  Such calls share their
rows x n_split partial slots out in proportion to the rows' lengths, on the device; these
cases drive that plan to its corners: one long row among empty ones (it takes nearly every
slot), every row empty, the largest row count the plan holds (one piece per row) and one
row past it (the even split), an explicit split count far above what the chip needs, and
index lists of very different lengths.  Whole outputs against the oracle at the usual
bar: relative L2 <= 5e-3, max |error| <= 2e-2."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, to_dev
from tests.test_gpu_attend import run_attend
from tests.test_gpu_sparse_tokens import check as check_sparse

pytestmark = pytest.mark.gpu

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def _with_lengths(lengths, n_split=0, **kw):
    lengths = np.asarray(lengths, dtype=np.int32)
    p = synth.make_problem(kind="decode", n_seq=lengths.size, **kw)
    p.kv_len = lengths
    got = run_attend(p, n_split=n_split)
    return p, got, oracle.attention_problem(p)


@pytest.mark.parametrize("kv_type", [BF16, Q8])
def test_one_long_row_among_empty(kv_type):
    """Rows of 0, 0, 5000, 0 and 1 cells: the long row takes all but one of the pieces."""
    p, got, ref = _with_lengths([0, 0, 5000, 0, 1], n_head=64, n_kv=5000, seed=61, kv_type=kv_type,
                                q_type=BF16)
    assert_parity(got, ref, f"one long row kv{kv_type}")
    rows = got.reshape(p.n_seq, p.n_head, synth.DV)
    assert np.all(rows[[0, 1, 3]] == 0)


def test_every_row_empty():
    p, got, ref = _with_lengths([0, 0, 0], n_head=128, n_kv=700, seed=62, sinks=True)
    assert np.all(got == 0)
    assert_parity(got, ref, "all empty")


@pytest.mark.parametrize("n_seq,n_tok", [(128, 2), (257, 1)])
def test_row_count_limit(n_seq, n_tok):
    """256 causal rows (one piece each: the plan's budget equals the row count) and 257
    rows (past the plan's limit: every row split evenly instead)."""
    p = synth.make_problem(kind="decode", n_seq=n_seq, n_tok=n_tok, n_head=16, n_kv=300, seed=63, ragged=True,
                           causal=n_tok > 1)
    got = run_attend(p, n_split=2)
    assert_parity(got, oracle.attention_problem(p), f"{n_seq}x{n_tok} rows")


def test_split_count_far_above_the_chip():
    """n_split = 200 for 6 rows: the plan still keeps one piece per workgroup slot."""
    p = synth.make_problem(kind="decode", n_seq=3, n_tok=2, n_head=128, n_kv=9000, seed=64, ragged=True,
                           causal=True, sinks=True, softcap=30.0)
    got = run_attend(p, n_split=200)
    assert_parity(got, oracle.attention_problem(p), "n_split 200")


@pytest.mark.parametrize("kv_type", [BF16, Q8])
def test_index_lists_of_different_lengths(kv_type):
    """Per-token index lists of ~all, ~half, a few and no cells in one call."""
    p = synth.make_problem(kind="sparse", n_seq=2, n_tok=2, n_head=64, n_kv=6000, q_type=BF16, kv_type=kv_type,
                           seed=65)
    g = np.random.default_rng(65)
    keep = [g.random(p.n_kv) < f for f in (0.97, 0.5, 0.003, 0.0)]
    for r, k in enumerate(keep):
        s, t = divmod(r, p.n_tok)
        p.mask[s, t] = np.where(k, np.uint16(0), np.uint16(synth.F16_NEG_INF))
    check_sparse(p, f"uneven lists kv{kv_type}")


def test_workspace_redzones():
    """The plan's pieces and its row table stay inside a workspace of exactly
    mla_fa_workspace_size bytes, and the output inside its buffer."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=5, n_tok=2, n_head=128, n_kv=4000, seed=66, ragged=True,
                           causal=True)
    rows, pad = p.n_seq * p.n_tok, 4096
    n_out = rows * p.n_head * synth.DV
    obuf = torch.full((n_out + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n_out].view(p.n_seq, p.n_tok, p.n_head, synth.DV)
    ws_bytes = B.mla_fa_workspace_size(rows, p.n_head, p.n_kv, p.kv_type, 0)
    wbuf = torch.full((ws_bytes + 2 * pad,), 77, dtype=torch.uint8, device="cuda")
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B.mla_fa_attend(to_dev(p.q), p.q_type, to_dev(p.kv), p.kv_type, p.scale, out, kv_len=f(p.kv_len), causal=True,
                    n_split=0, workspace=wbuf[pad:pad + ws_bytes])
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64)
    assert_parity(got, oracle.attention_problem(p), "redzones")
    assert torch.all(obuf[:pad] == 12345.0) and torch.all(obuf[-pad:] == 12345.0)
    assert torch.all(wbuf[:pad] == 77) and torch.all(wbuf[-pad:] == 77)


@pytest.mark.parametrize("lengths,n_tok", [([0, 0, 20000, 0, 1, 3], 1), ([9000, 3, 4500, 0, 12000, 700, 2, 6000], 2)])
def test_absorbed_ragged(lengths, n_tok):
    """The absorbed decode over rows of very different lengths: the split attention
    follows the plan and the fused merge + output projection reads each row's slots
    (rows of a 4-row block holding different piece counts, some none)."""
    from tests.test_gpu_absorbed import ref_absorbed, run_absorbed
    p = synth.make_absorbed_problem(n_seq=len(lengths), n_tok=n_tok, n_head=128, n_kv=20000, q_type=BF16,
                                    kv_type=BF16, seed=68 + n_tok, causal=n_tok > 1)
    p.kv_len = np.asarray(lengths, dtype=np.int32)
    got = run_absorbed(p, n_split=0)
    assert_parity(got, ref_absorbed(p), f"absorbed ragged n_tok={n_tok}")


@pytest.mark.parametrize("kv_type", [BF16, Q8])
def test_sparse_decode_uneven_lists(kv_type):
    """mla_fa_decode over the index lists of several sequences shares its slots by the
    lists' lengths; the two-phase calls (partials, then merge) keep n_split pieces per
    row.  Lists of ~all, a few, none and half of the cells: both forms against the
    oracle, and the plan's output against the two-phase one."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="sparse", n_seq=4, n_head=128, n_kv=12000, q_type=BF16, kv_type=kv_type, seed=69)
    g = np.random.default_rng(69)
    keep = [g.random(p.n_kv) < f for f in (0.98, 0.004, 0.0, 0.5)]
    for s, k in enumerate(keep):
        p.mask[s, 0] = np.where(k, np.uint16(0), np.uint16(synth.F16_NEG_INF))
    mask = to_dev(p.mask.reshape(p.n_seq, p.n_kv))
    idx = torch.zeros((p.n_seq, p.n_kv), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((p.n_seq,), dtype=torch.int32, device="cuda")
    B.fa_mask_compact(mask, idx, cnt)
    q, kv = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK)), to_dev(p.kv)
    ns = B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    assert ns > 1
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)
    outs = []
    for two_phase in (False, True):
        out = torch.full((p.n_seq, p.n_head, synth.DV), float("nan"), dtype=torch.float32, device="cuda")
        kw = dict(mask=mask, kv_idx=idx, kv_idx_count=cnt, n_split=ns, workspace=ws)
        if two_phase:
            B.mla_fa_decode_partials(q, p.q_type, kv, p.kv_type, p.scale, out, **kw)
            B.mla_fa_merge_partials(p.n_seq, p.n_head, ns, out, ws)
        else:
            B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, **kw)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64))
    ref = oracle.attention_problem(p)
    assert_parity(outs[0], ref, f"plan kv{kv_type}")
    assert_parity(outs[1], ref, f"two-phase kv{kv_type}")
    assert_parity(outs[0], outs[1], f"plan vs two-phase kv{kv_type}")
    assert np.all(outs[0][2 * p.n_head:3 * p.n_head] == 0)      # the sequence with no kept cell


def _expected_table(tiles, budget):
    """The plan as documented: the smallest chunk C (in tiles) with
    sum_r ceil(tiles_r / C) <= budget; row r gets ceil(tiles_r / C) pieces, numbered row
    by row.  Returns [(first slot, pieces)] per row."""
    C = 1
    while sum(-(-t // C) for t in tiles) > budget:
        C += 1
    out, first = [], 0
    for t in tiles:
        n = -(-t // C)
        out.append((first if n else 0, n))
        first += n
    return out


@pytest.mark.parametrize("lengths,n_tok", [([11112, 6450, 7284, 19326, 11379, 21065, 9351, 25407], 2),
                                           ([0, 5000, 1, 64, 65, 0, 30000], 1),
                                           ([3000] * 20, 3)])
def test_row_table_is_the_smallest_chunk_plan(lengths, n_tok):
    """The row table the attention launch leaves in the workspace tail matches the plan
    stated in plain terms: per row its first slot and piece count for the smallest
    chunk that fits the budget (rows x n_split slots, at most one piece per workgroup
    the chip holds: CUs / 2 head groups of 64 heads)."""
    import torch
    from mla_flash_attention_amd import binding as B
    n_seq, n_head, n_kv = len(lengths), 128, 32768
    p = synth.make_problem(kind="decode", n_seq=n_seq, n_tok=n_tok, n_head=n_head, n_kv=n_kv, seed=70,
                           causal=n_tok > 1)
    p.kv_len = np.asarray(lengths, dtype=np.int32)
    rows = n_seq * n_tok
    ns = B.mla_fa_auto_splits(rows, n_head, n_kv, p.kv_type)
    ws = B.workspace_for(rows, n_head, n_kv, p.kv_type, ns)
    ws.fill_(0x77)
    out = torch.empty((n_seq, n_tok, n_head, synth.DV), dtype=torch.float32, device="cuda")
    B.mla_fa_attend(to_dev(p.q), p.q_type, to_dev(p.kv), p.kv_type, p.scale, out,
                    kv_len=torch.from_numpy(p.kv_len).cuda(), causal=n_tok > 1, n_split=ns, workspace=ws)
    torch.cuda.synchronize()
    tail = ns * rows * n_head * 1040
    table = ws[tail:tail + 4 * rows].cpu().numpy().view(np.int32)
    got = [(int(v) & 0xFFFF, int(v) >> 16) for v in table]
    got = [(f if n else 0, n) for f, n in got]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    budget = min(rows * ns, max(rows, cus // 2))
    tiles = []
    for L in lengths:
        for t in range(n_tok):
            end = max(0, L - n_tok + t + 1) if n_tok > 1 else L
            tiles.append(-(-end // 64))
    assert got == _expected_table(tiles, budget)
    assert sum(n for _, n in got) <= budget
    assert_parity(out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64), oracle.attention_problem(p),
                  f"table case {lengths[:3]}")
