"""HIP graph capture of the path (torch.cuda.CUDAGraph around calls through the C ABI).

A serving loop captures its decode step once and replays it; the library's calls
record only kernel launches on the caller's stream (no allocation, no memset, no host
synchronisation), so a captured call must replay the eager result exactly.  Each case
runs the call eagerly, captures it, and replays the graph three times; before every
replay the outputs are poisoned with NaN by eager work and the device is synchronised,
and every replay must match the eager result bit for bit.  The eager results themselves
are checked against the oracle (whole output, rel-L2 <= 5e-3, max |error| <= 2e-2)."""
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


def check_replays(call, outputs, extra=None, scratch=()):
    """call(): the launches to capture; outputs: tensors the call writes (any dtype),
    compared whole; extra(): an additional check after every replay (for outputs only
    partly defined, such as an index list past its count); scratch: buffers the call
    uses internally (a workspace), filled with junk before every replay."""
    import torch
    call()                                               # eager, on the current stream
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for k in range(3):
        for o in outputs:                                # eager work between replays
            if o.is_floating_point():
                o.fill_(float("nan"))
            else:
                o.fill_(-7)
        junk.fill_(float(k))
        for t in scratch:
            t.fill_(0x5A + k)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            assert torch.equal(o.view(torch.uint8) if o.dtype != torch.uint8 else o,
                               e.view(torch.uint8) if e.dtype != torch.uint8 else e), f"replay {k}"
        if extra:
            extra()
    return [e.cpu() for e in eager]


def _decode_inputs(p):
    import torch
    q = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK))
    kv = to_dev(p.kv)
    mask = None if p.mask is None else to_dev(p.mask.reshape(p.n_seq, p.n_kv))
    out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    return q, kv, mask, out


@pytest.mark.parametrize("kv_type,q_type", [(BF16, BF16), (Q8, BF16)])
def test_graph_split_decode(kv_type, q_type):
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=3, n_head=128, n_kv=5000, q_type=q_type, kv_type=kv_type, seed=81,
                           mask_kind="runs_bias")
    q, kv, mask, out = _decode_inputs(p)
    ns = B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    assert ns > 1
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)
    (got,) = check_replays(lambda: B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, n_split=ns,
                                                   workspace=ws), [out])
    assert_parity(got.numpy().astype(np.float64), oracle.attention_problem(p), "graph split decode")


def test_graph_noalloc_decode():
    """The allocation-free entry point is the one meant for capture: its partials live in
    the library's per-GPU scratch."""
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=4, n_head=64, n_kv=3000, q_type=F16, kv_type=F16, seed=82)
    q, kv, mask, out = _decode_inputs(p)
    (got,) = check_replays(lambda: B.mla_fa_decode_noalloc(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask), [out])
    assert_parity(got.numpy().astype(np.float64), oracle.attention_problem(p), "graph noalloc decode")


def test_graph_sparse_step():
    """The sparse step as a serving loop would capture it: chunked compaction of the mask
    row, then attention over the kept list (the count stays on the device)."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="sparse", n_seq=1, n_head=128, n_kv=40000, q_type=BF16, kv_type=Q8, seed=83)
    q, kv, mask, out = _decode_inputs(p)
    idx = torch.zeros((p.n_seq, p.n_kv), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((p.n_seq,), dtype=torch.int32, device="cuda")
    cws = torch.empty(max(B.fa_mask_compact_workspace_size(p.n_seq, p.n_kv), 1), dtype=torch.uint8, device="cuda")
    ns = B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)

    def step():
        B.fa_mask_compact_ws(mask, idx, cnt, cws)
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, kv_idx=idx, kv_idx_count=cnt,
                        n_split=ns, workspace=ws)
    idx_ref, cnt_ref = oracle.mask_compact(p.mask.reshape(p.n_seq, p.n_kv))
    n = int(cnt_ref[0])

    def kept_prefix():                  # the list is defined up to its count only
        assert np.array_equal(idx[0, :n].cpu().numpy(), idx_ref[0, :n])
    got, gcnt = check_replays(step, [out, cnt], extra=kept_prefix)
    assert np.array_equal(gcnt.numpy(), cnt_ref)
    assert_parity(got.numpy().astype(np.float64), oracle.attention_problem(p), "graph sparse step")


@pytest.mark.parametrize("n_split", [0, 1])
def test_graph_absorbed_decode(n_split):
    """Three launches per call: query projection, attention, and the output projection
    (fused with the merge when split)."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_absorbed_problem(n_seq=3, n_tok=1, n_head=128, n_kv=2500, q_type=BF16, kv_type=BF16, seed=84)
    f = lambda a: to_dev(a)
    qn, qp, wk, wv, kv = f(p.q_nope), f(p.q_pe), f(p.w_uk), f(p.w_uv), f(p.kv)
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, 128), dtype=torch.float32, device="cuda")
    ws = B.absorbed_workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, n_split)
    (got,) = check_replays(lambda: B.mla_fa_absorbed(qn, qp, p.q_type, wk, wv, kv, p.kv_type, p.scale, out,
                                                     n_split=n_split, workspace=ws), [out])
    ref = oracle.absorbed_attention(p.q_nope, p.q_pe, p.q_type, p.w_uk, p.w_uv, p.kv, p.kv_type, p.n_seq, p.n_tok,
                                    p.n_head, p.n_kv, p.scale)
    assert_parity(got.numpy().astype(np.float64).reshape(-1, 128), ref, f"graph absorbed n_split={n_split}")


@pytest.mark.parametrize("sparse", [False, True])
def test_graph_ragged_attend(sparse):
    """mla_fa_attend over rows of device-side lengths: the length-proportional plan, its
    row table in the workspace tail and the merge that reads it, replayed with the
    workspace overwritten by junk before every replay."""
    import torch
    from mla_flash_attention_amd import binding as B
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if sparse:
        p = synth.make_problem(kind="sparse", n_seq=2, n_tok=2, n_head=128, n_kv=7000, q_type=BF16, kv_type=Q8,
                               seed=87)
        rows = p.n_seq * p.n_tok
        idx = torch.zeros((p.n_seq, p.n_tok, p.n_kv), dtype=torch.int32, device="cuda")
        cnt = torch.zeros((p.n_seq, p.n_tok), dtype=torch.int32, device="cuda")
        B.fa_mask_compact(to_dev(p.mask.reshape(rows, p.n_kv)), idx.view(rows, p.n_kv), cnt.view(rows))
        extra_args = dict(mask=to_dev(p.mask), kv_idx=idx, kv_idx_count=cnt)
    else:
        p = synth.make_problem(kind="decode", n_seq=5, n_tok=2, n_head=128, n_kv=9000, q_type=BF16, kv_type=BF16,
                               seed=88, ragged=True, causal=True, sinks=True, softcap=30.0)
        rows = p.n_seq * p.n_tok
        extra_args = dict(kv_len=f(p.kv_len), causal=True, sinks=f(p.sinks), softcap=p.softcap)
    q, kv = to_dev(p.q), to_dev(p.kv)
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ws = B.workspace_for(rows, p.n_head, p.n_kv, p.kv_type, 0)
    assert ws is not None
    (got,) = check_replays(lambda: B.mla_fa_attend(q, p.q_type, kv, p.kv_type, p.scale, out, n_split=0, workspace=ws,
                                                   **extra_args), [out], scratch=[ws])
    assert_parity(got.numpy().reshape(-1, synth.DV).astype(np.float64), oracle.attention_problem(p),
                  f"graph ragged attend sparse={sparse}")
