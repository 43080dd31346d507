"""The library's calls are reentrant: host threads may call it at the same time, each
on its own stream with its own workspace.  Five threads run a mix of calls (split
decode, sparse step with chunked compaction, absorbed decode, per-head prefill, ragged
multi-token attend) ten times each on their own streams; every result must equal the
same call made alone, bit for bit (the kernels are deterministic), and the lone results
meet the oracle bar."""
import threading

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


def _decode_job(seed):
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=3, n_head=128, n_kv=4000, q_type=BF16, kv_type=Q8, seed=seed,
                           mask_kind="runs_bias")
    q, kv, mask = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK)), to_dev(p.kv), to_dev(p.mask.reshape(p.n_seq, -1))
    out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ns = B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)

    def run():
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, n_split=ns, workspace=ws)
        return [out]
    return run, lambda got: assert_parity(got[0].cpu().numpy().astype(np.float64), oracle.attention_problem(p),
                                          "threads decode")


def _sparse_job(seed):
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="sparse", n_seq=1, n_head=128, n_kv=20000, q_type=BF16, kv_type=BF16, seed=seed)
    q, kv, mask = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK)), to_dev(p.kv), to_dev(p.mask.reshape(p.n_seq, -1))
    out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    idx = torch.zeros((p.n_seq, p.n_kv), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((p.n_seq,), dtype=torch.int32, device="cuda")
    cws = torch.empty(max(B.fa_mask_compact_workspace_size(p.n_seq, p.n_kv), 1), dtype=torch.uint8, device="cuda")
    ns = B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)

    def run():
        B.fa_mask_compact_ws(mask, idx, cnt, cws)
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, kv_idx=idx, kv_idx_count=cnt,
                        n_split=ns, workspace=ws)
        return [out, cnt]
    return run, lambda got: assert_parity(got[0].cpu().numpy().astype(np.float64), oracle.attention_problem(p),
                                          "threads sparse")


def _absorbed_job(seed):
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_absorbed_problem(n_seq=2, n_tok=1, n_head=64, n_kv=2500, q_type=F16, kv_type=F16, seed=seed)
    args = [to_dev(a) for a in (p.q_nope, p.q_pe)] + [p.q_type] + [to_dev(a) for a in (p.w_uk, p.w_uv, p.kv)]
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, 128), dtype=torch.float32, device="cuda")
    ws = B.absorbed_workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, 0)

    def run():
        B.mla_fa_absorbed(*args, p.kv_type, p.scale, out, workspace=ws)
        return [out]
    ref = lambda: oracle.absorbed_attention(p.q_nope, p.q_pe, p.q_type, p.w_uk, p.w_uv, p.kv, p.kv_type, p.n_seq,
                                           p.n_tok, p.n_head, p.n_kv, p.scale)
    return run, lambda got: assert_parity(got[0].cpu().numpy().reshape(-1, 128).astype(np.float64), ref(),
                                          "threads absorbed")


def _mha_job(seed):
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_mha_problem(300, 32, 700, BF16, BF16, seed=seed, causal=True)
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    out = torch.empty((p.n_tok, p.n_head, synth.MHA_DV), dtype=torch.float32, device="cuda")

    def run():
        B.mla_fa_prefill_mha(q, p.q_type, k, v, p.kv_type, p.scale, out, causal=True)
        return [out]
    ref = lambda: oracle.mha_attention(p.q, p.q_type, p.k, p.v, p.kv_type, p.scale, causal=True)
    return run, lambda got: assert_parity(got[0].cpu().numpy().reshape(-1, synth.MHA_DV).astype(np.float64), ref(),
                                          "threads mha")


def _ragged_job(seed):
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=4, n_tok=2, n_head=128, n_kv=6000, q_type=BF16, kv_type=BF16,
                           seed=seed, ragged=True, causal=True)
    q, kv = to_dev(p.q), to_dev(p.kv)
    kvl = torch.from_numpy(np.ascontiguousarray(p.kv_len)).cuda()
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ws = B.workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, 0)

    def run():
        B.mla_fa_attend(q, p.q_type, kv, p.kv_type, p.scale, out, kv_len=kvl, causal=True, n_split=0, workspace=ws)
        return [out]
    return run, lambda got: assert_parity(got[0].cpu().numpy().reshape(-1, synth.DV).astype(np.float64),
                                          oracle.attention_problem(p), "threads ragged")


def test_concurrent_host_threads():
    import torch
    jobs = [_decode_job(111), _sparse_job(112), _absorbed_job(113), _mha_job(114), _ragged_job(115)]
    alone = []
    for run, check in jobs:                            # each call alone, on the default stream
        got = [t.clone() for t in run()]
        torch.cuda.synchronize()
        check(got)
        alone.append([t.cpu() for t in got])
    errors = []
    barrier = threading.Barrier(len(jobs))

    def worker(j):
        try:
            run, _ = jobs[j]
            s = torch.cuda.Stream()
            barrier.wait()
            with torch.cuda.stream(s):
                for it in range(10):
                    got = run()
                    s.synchronize()
                    for t, ref in zip(got, alone[j]):
                        if not torch.equal(t.cpu(), ref):
                            errors.append(f"job {j} iteration {it}")
                            return
        except Exception as e:                          # reported below, in the main thread
            errors.append(f"job {j}: {e!r}")
    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
