"""Helpers for the GPU parity tests: upload a synthetic problem, run it through the
C ABI (binding), and measure agreement with the oracle.  Imports torch lazily."""
from __future__ import annotations

import numpy as np

from mla_flash_attention_amd import synth

REL_L2_TOL = 5e-3      # whole-tensor relative L2 error bound for attention outputs
MAX_ABS_TOL = 2e-2     # whole-tensor max |error| bound


def to_dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint8:
        t = torch.from_numpy(a)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def parity(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    return float(rel), float(np.abs(diff).max()) if diff.size else 0.0


def assert_parity(got, ref, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel, mx = parity(got, ref)
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_TOL, f"{what}: rel-L2 {rel:.3e} max-abs {mx:.3e}"
    return rel, mx


def run_decode(p, n_split=0, out=None, ws=None, via_compaction=None, chunked=False):
    """Run decode (dense, masked, or sparse through fa_mask_compact, or through
    fa_mask_compact_ws when `chunked`) for problem p.
    Returns (out fp32 numpy [n_seq*n_head][512], extras dict)."""
    import torch
    from mla_flash_attention_amd import binding as B
    assert p.n_tok == 1
    q = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK))
    kv = to_dev(p.kv)
    out = out if out is not None else torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    mask = None if p.mask is None else to_dev(p.mask.reshape(p.n_seq, p.n_kv))
    extras = {}
    kv_idx = kv_cnt = None
    sparse = p.kind == "sparse" if via_compaction is None else via_compaction
    if sparse:
        assert mask is not None
        kv_idx = torch.full((p.n_seq, p.n_kv), -7, dtype=torch.int32, device="cuda")
        kv_cnt = torch.full((p.n_seq,), -7, dtype=torch.int32, device="cuda")
        if chunked:
            need = B.fa_mask_compact_workspace_size(p.n_seq, p.n_kv)
            cws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            B.fa_mask_compact_ws(mask, kv_idx, kv_cnt, cws)
        else:
            B.fa_mask_compact(mask, kv_idx, kv_cnt)
        extras["idx"], extras["count"] = kv_idx, kv_cnt
    if ws is None:
        ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, n_split)
    B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, kv_idx=kv_idx,
                    kv_idx_count=kv_cnt, n_split=n_split, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64), extras


def run_prefill(p, n_split=0, causal=None):
    import torch
    from mla_flash_attention_amd import binding as B
    assert p.n_seq == 1
    q = to_dev(p.q.reshape(p.n_tok, p.n_head, synth.DK))
    kv = to_dev(p.kv.reshape(p.n_kv, -1))
    out = torch.empty((p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    mask = None if p.mask is None else to_dev(p.mask.reshape(p.n_tok, p.n_kv))
    ws = B.workspace_for(p.n_tok, p.n_head, p.n_kv, p.kv_type, n_split)
    B.mla_fa_prefill(q, p.q_type, kv, p.kv_type, p.scale, out, causal=p.causal if causal is None else causal,
                     mask=mask, n_split=n_split, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64)
