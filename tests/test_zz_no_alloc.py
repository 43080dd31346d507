"""mla_fa_decode_noalloc: decode for callers that cannot allocate, with the split partials
in the library's per-GPU scratch array instead of a caller workspace.  Its output must
equal mla_fa_decode's bit for bit (same kernels, same plan) on consecutive calls, the
second smaller than the first; calls past the scratch's size are refused before anything
is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import binding as B
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, to_dev

BF16, Q8 = synth.TYPE_BF16, synth.TYPE_Q8_0
SCRATCH = 48 << 20          # MLA_FA_NOALLOC_SCRATCH_BYTES in include/mla_fa.h
FAKE = 1 << 20


def test_automatic_plans_fit_the_scratch():
    """Every automatic split plan's partials fit the scratch (CPU: sizes only)."""
    worst = max(B.mla_fa_workspace_size(r, h, 1 << 20, t, 0)
                for h in range(16, 129, 16) for r in range(1, 600) for t in (1, 2, 3))
    assert worst <= SCRATCH


def test_too_large_is_refused_before_any_hip_call():
    """Partials past the scratch: MLA_FA_ERR_WORKSPACE from the host checks (CPU: the
    pointers are never used)."""
    L = B.lib()
    f = lambda n_seq, n_split: L.mla_fa_decode_noalloc(FAKE, BF16, FAKE, BF16, 1152, 1152 * 4096, n_seq, 128,
                                                       4096, None, 0, None, None, 0, ctypes.c_float(0.1), FAKE,
                                                       n_split, None)
    assert B.mla_fa_workspace_size(300, 128, 4096, BF16, 64) > SCRATCH
    assert f(300, 64) == B.MLA_FA_ERR_WORKSPACE
    assert f(0, 0) == B.MLA_FA_ERR_INVALID


def _inputs(p):
    q = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK))
    kv = to_dev(p.kv)
    mask = None if p.mask is None else to_dev(p.mask.reshape(p.n_seq, p.n_kv))
    return q, kv, mask


@pytest.mark.gpu
def test_noalloc_matches_decode_on_consecutive_calls():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    # call 1: 4 sequences x 128 heads x 8192 bf16 cells (automatic split count);
    # call 2: a smaller sparse Q8_0 problem through compacted index lists
    p1 = synth.make_problem(kind="decode", n_seq=4, n_head=128, n_kv=8192, seed=301)
    p2 = synth.make_problem(kind="sparse", n_seq=2, n_head=64, n_kv=3000, kv_type=Q8, seed=302)
    for p in (p1, p2):
        q, kv, mask = _inputs(p)
        idx = cnt = None
        if p.kind == "sparse":
            idx = torch.empty((p.n_seq, p.n_kv), dtype=torch.int32, device="cuda")
            cnt = torch.empty((p.n_seq,), dtype=torch.int32, device="cuda")
            B.fa_mask_compact(mask, idx, cnt)
        ref_out = torch.full((p.n_seq, p.n_head, synth.DV), float("nan"), dtype=torch.float32, device="cuda")
        ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, 0)
        assert ws is not None                       # a split plan: the scratch is used
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, ref_out, mask=mask, kv_idx=idx, kv_idx_count=cnt,
                        workspace=ws)
        out = torch.full_like(ref_out, float("nan"))
        B.mla_fa_decode_noalloc(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, kv_idx=idx,
                                kv_idx_count=cnt)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref_out.cpu().numpy()
        assert np.array_equal(a, b), f"{p.name}: noalloc differs from mla_fa_decode"
        assert_parity(a.reshape(-1, synth.DV).astype(np.float64), oracle.attention_problem(p), p.name)


@pytest.mark.gpu
def test_noalloc_refuses_oversized_calls_without_writing():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    p = synth.make_problem(kind="decode", n_seq=300, n_head=128, n_kv=64, seed=303)
    q, kv, _ = _inputs(p)
    out = torch.full((p.n_seq, p.n_head, synth.DV), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(B.MlaFaError) as e:
        B.mla_fa_decode_noalloc(q, p.q_type, kv, p.kv_type, p.scale, out, n_split=64)
    assert e.value.status == B.MLA_FA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
