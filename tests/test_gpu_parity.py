"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs.  Attention outputs must satisfy, over the whole output tensor, relative L2 error
<= 5e-3 and max |error| <= 2e-2; compacted index lists and counts must be bit-exact."""
import numpy as np
import pytest

import oracle
from mla_flash_attention_amd import synth
from tests.gpu_common import assert_parity, run_decode, run_prefill, to_dev

pytestmark = pytest.mark.gpu

BF16, F16, Q8 = synth.TYPE_BF16, synth.TYPE_F16, synth.TYPE_Q8_0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from mla_flash_attention_amd import binding
    binding.lib()


def _decode_case(n_seq, n_head, n_kv, q_type, kv_type, seed, n_split=0, mask_kind=None, q_gain=1.0):
    p = synth.make_problem(kind="decode", n_seq=n_seq, n_head=n_head, n_kv=n_kv, q_type=q_type,
                           kv_type=kv_type, seed=seed, mask_kind=mask_kind, q_gain=q_gain)
    got, _ = run_decode(p, n_split=n_split)
    ref = oracle.attention_problem(p)
    return assert_parity(got, ref, f"decode s{n_seq} h{n_head} kv{n_kv} t{q_type}/{kv_type} split{n_split}")


# ---------------------------------------------------------------- workloads at full size
def test_plan_fills_the_devices_compute_units():
    """The automatic split plan sizes itself to the device's compute units: on the
    4 x 128-head decode (two 64-head workgroups per key range) one workgroup per CU."""
    import torch
    from mla_flash_attention_amd import binding as B
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert B.mla_fa_auto_splits(4, 128, 32768, BF16) == -(-cus // 8)


def test_c1_full():
    p = synth.make_config(1)
    for n_split in (0, 1):
        got, _ = run_decode(p, n_split=n_split)
        assert_parity(got, oracle.attention_problem(p), f"C1 split{n_split}")


def test_c2_full():
    p = synth.make_config(2)
    got, _ = run_decode(p)
    assert_parity(got, oracle.attention_problem(p), "C2")


def test_c4_full():
    p = synth.make_config(4)
    got, _ = run_decode(p)
    assert_parity(got, oracle.attention_problem(p), "C4")


@pytest.mark.parametrize("chunked", [False, True])
def test_c5_full_sparse(chunked):
    """The full sparse workload through either compaction entry point (the benchmark
    times the chunked one)."""
    p = synth.make_config(5)
    got, ex = run_decode(p, chunked=chunked)
    idx_ref, cnt_ref = oracle.mask_compact(p.mask.reshape(1, -1))
    cnt = int(ex["count"].cpu()[0])
    assert cnt == int(cnt_ref[0])
    assert np.array_equal(ex["idx"].cpu().numpy()[0, :cnt], idx_ref[0, :cnt])
    assert_parity(got, oracle.attention_problem(p), "C5")


def test_c3_full():
    """The full causal prefill (2048 tokens x 128 heads over 4096 cells, the benched launch):
    every output row against the oracle."""
    p = synth.make_config(3)
    got = run_prefill(p)
    assert_parity(got, oracle.attention_problem(p), "C3")


# ---------------------------------------------------------------- reduced-size sweeps
@pytest.mark.parametrize("n_kv", [1, 2, 31, 32, 33, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("n_head", [16, 128])
def test_decode_kv_sweep(n_kv, n_head):
    _decode_case(2, n_head, n_kv, BF16, BF16, seed=n_kv + n_head)


@pytest.mark.parametrize("n_head", [16, 32, 48, 64, 80, 96, 112, 128])
@pytest.mark.parametrize("kv_type", [BF16, F16])
def test_decode_head_counts(n_head, kv_type):
    _decode_case(2, n_head, 777, kv_type, kv_type, seed=n_head)


@pytest.mark.parametrize("n_split", [1, 2, 3, 0, 1024])
def test_decode_split_sweep(n_split):
    _decode_case(3, 128, 5000, BF16, BF16, seed=40 + n_split, n_split=n_split)


@pytest.mark.parametrize("q_type", [BF16, F16])
@pytest.mark.parametrize("n_kv", [1, 65, 3000])
def test_decode_q8_0(q_type, n_kv):
    _decode_case(2, 128, n_kv, q_type, Q8, seed=7 + n_kv)


@pytest.mark.parametrize("mask_kind", ["random", "runs_bias"])
@pytest.mark.parametrize("kv_type", [BF16, Q8])
def test_decode_masked_dense(mask_kind, kv_type):
    q_type = BF16
    _decode_case(3, 64, 2500, q_type, kv_type, seed=11, mask_kind=mask_kind)


@pytest.mark.parametrize("kv_type", [BF16, F16, Q8])
@pytest.mark.parametrize("mask_kind", ["runs", "runs_bias", "random"])
def test_decode_sparse_reduced(kv_type, mask_kind):
    q_type = F16 if kv_type == F16 else BF16
    p = synth.make_problem(kind="sparse", n_seq=2, n_head=128, n_kv=20000, q_type=q_type,
                           kv_type=kv_type, seed=3, mask_kind=mask_kind)
    got, ex = run_decode(p)
    idx_ref, cnt_ref = oracle.mask_compact(p.mask.reshape(2, -1))
    cnt = ex["count"].cpu().numpy()
    assert np.array_equal(cnt, cnt_ref)
    idx = ex["idx"].cpu().numpy()
    for s in range(2):
        assert np.array_equal(idx[s, :cnt[s]], idx_ref[s, :cnt[s]])
    assert_parity(got, oracle.attention_problem(p), f"sparse {kv_type} {mask_kind}")


@pytest.mark.parametrize("n_tok,n_kv", [(1, 1), (5, 7), (64, 64), (70, 300), (128, 1000)])
def test_prefill_causal_reduced(n_tok, n_kv):
    p = synth.make_problem(kind="prefill", n_tok=n_tok, n_head=128, n_kv=n_kv, seed=n_kv, causal=True)
    assert_parity(run_prefill(p), oracle.attention_problem(p), f"prefill {n_tok}x{n_kv}")


def test_prefill_split_and_mask():
    p = synth.make_problem(kind="prefill", n_tok=6, n_head=16, n_kv=3000, seed=8, causal=True,
                           mask_kind="random")
    for n_split in (0, 1, 5):
        assert_parity(run_prefill(p, n_split=n_split), oracle.attention_problem(p), f"prefill split{n_split}")


def test_prefill_noncausal_q8():
    p = synth.make_problem(kind="prefill", n_tok=33, n_head=32, n_kv=500, seed=9, causal=False,
                           kv_type=Q8, q_type=F16)
    assert_parity(run_prefill(p), oracle.attention_problem(p), "prefill non-causal q8_0")


# ---------------------------------------------------------------- adversarial softmax
def _bf(x):
    return synth.round_bits(np.asarray(x, np.float32), BF16)


def test_scores_rise_every_tile():
    """Each 64-key tile raises the running max by ~14 (~20 in log2 units), so every tile
    rescales.  The rising component sits in a RoPE column (575), outside V, so outputs
    keep the N(0,1) scale the absolute tolerance is meant for."""
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=700, seed=50)
    p.q[..., 575] = _bf(60.0)
    p.kv[0, :, 575] = _bf(0.05 * np.arange(700))
    assert_parity(run_decode(p, n_split=1)[0], oracle.attention_problem(p), "rising")


def test_planted_peak_last_key():
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=1000, seed=51, q_gain=3.0)
    p.kv[0, -1] = p.q[0, 0, 3]                   # the last key equals head 3's query
    assert_parity(run_decode(p, n_split=2)[0], oracle.attention_problem(p), "peak")


def test_all_keys_equal():
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=300, seed=52)
    p.kv[0, :] = p.kv[0, 0]
    got = run_decode(p)[0]
    assert_parity(got, oracle.attention_problem(p), "equal keys")


def test_all_masked_but_one_and_fully_masked():
    p = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=900, seed=53, mask_kind="none_kept")
    p.mask[0, 0, 417] = 0                        # sequence 0 keeps one cell, sequence 1 none
    for sparse in (False, True):
        got, _ = run_decode(p, via_compaction=sparse)
        ref = oracle.attention_problem(p)
        assert np.all(got[16:] == 0.0)           # fully masked row -> zeros, not NaN
        assert_parity(got, ref, f"one kept (sparse={sparse})")


# ---------------------------------------------------------------- determinism and redzones
def test_bitwise_determinism():
    p = synth.make_config(2, n_kv=9000)
    a, _ = run_decode(p)
    b, _ = run_decode(p)
    assert np.array_equal(a, b)


def test_redzones_untouched():
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=2, n_head=128, n_kv=3000, seed=60)
    pad = 4096
    buf = torch.full((2 * 128 * 512 + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + 2 * 128 * 512].view(2, 128, 512)
    nsplit = 6
    ws_bytes = B.mla_fa_workspace_size(2, 128, 3000, BF16, nsplit)
    wbuf = torch.full((ws_bytes + 2 * pad,), 77, dtype=torch.uint8, device="cuda")
    ws = wbuf[pad:pad + ws_bytes]
    got, _ = run_decode(p, n_split=nsplit, out=out, ws=ws)
    assert_parity(got, oracle.attention_problem(p), "redzone run")
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[-pad:] == 12345.0)
    assert torch.all(wbuf[:pad] == 77) and torch.all(wbuf[-pad:] == 77)


def _scale_bits(bits, shift, type_id):
    """Multiply 16-bit floats (bits) by 2^shift exactly, by moving the exponent field of
    every normal value (zeros stay zero); asserts nothing leaves the normal range."""
    mant = 7 if type_id == BF16 else 10
    emax = 255 if type_id == BF16 else 31
    v = bits.astype(np.int64)
    e = (v >> mant) & emax
    ok = (e > 0) & (e < emax)
    e2 = e + shift
    assert np.all((e2[ok] > 0) & (e2[ok] < emax))
    v = np.where(ok, (v & ~(emax << mant)) | (e2 << mant), v)
    return v.astype(np.uint16)


@pytest.mark.parametrize("t,shift", [(BF16, 90), (BF16, -90), (BF16, 40)])
def test_split_partials_value_range(t, shift):
    """Split partials hold O in f16 under a power-of-two scale per half: outputs far from
    1 in magnitude must keep their precision.  The cache's latent dims (K and V) are
    scaled by 2^shift and Q's latent dims by 2^-shift, which leaves every score exactly
    as it was and scales the output by exactly 2^shift (bf16 only: f16's exponent range
    cannot move N(0,1) values this far)."""
    p = synth.make_problem(kind="decode", n_seq=2, n_head=128, n_kv=3000, q_type=t, kv_type=t, seed=77)
    ref = oracle.attention_problem(p)
    kv = p.kv.copy()
    kv[..., :512] = _scale_bits(kv[..., :512], shift, t)
    q = p.q.copy()
    q[..., :512] = _scale_bits(q[..., :512], -shift, t)
    p.kv, p.q = kv, q
    got, _ = run_decode(p, n_split=8)
    assert np.all(np.isfinite(got))
    assert_parity(got * 2.0 ** -shift, ref, f"value range 2^{shift}")


# ---------------------------------------------------------------- compaction
def compact(mask, idx, cnt, entry):
    """Run one compaction entry point; the chunked one gets a workspace between two
    redzones, which must come back untouched."""
    import torch
    from mla_flash_attention_amd import binding as B
    if entry == "one":
        B.fa_mask_compact(mask, idx, cnt)
        return
    n_rows, n_kv = mask.shape
    need = B.fa_mask_compact_workspace_size(n_rows, n_kv)
    pad = 1024
    wbuf = torch.full((need + 2 * pad,), 77, dtype=torch.uint8, device="cuda")
    B.fa_mask_compact_ws(mask, idx, cnt, wbuf[pad:pad + need] if need else None)
    torch.cuda.synchronize()
    assert torch.all(wbuf[:pad] == 77) and torch.all(wbuf[pad + need:] == 77)


@pytest.mark.parametrize("entry", ["one", "chunked"])
@pytest.mark.parametrize("case", ["empty", "full", "first", "last", "alternating", "runs", "tiny"])
@pytest.mark.parametrize("aligned", [True, False])
def test_compaction_cases(case, aligned, entry):
    import torch
    from mla_flash_attention_amd import binding as B
    n = 3 if case == "tiny" else 70001
    g = np.random.default_rng(5)
    rows = []
    for r in range(3):
        bits = np.full(n, synth.F16_NEG_INF, np.uint16)
        if case == "full":
            bits[:] = 0
        elif case == "first":
            bits[0] = 0
        elif case == "last":
            bits[-1] = 0
        elif case == "alternating":
            bits[r % 2::2] = 0x3C00
        elif case in ("runs", "tiny"):
            bits = synth.sparse_runs_mask(n, g, max_gap=700 if n > 3 else 1, max_run=600 if n > 3 else 1)
        rows.append(bits)
    m = np.stack(rows)
    # aligned: rows start on 16-byte boundaries (vector path); unaligned: the buffer is
    # offset by one element and rows are n + 3 apart (one-cell-per-lane path)
    stride = n + 8 - n % 8 if aligned else n + 3
    lead = 0 if aligned else 1
    host = np.full(lead + 3 * stride, 0x1234, np.uint16)
    host[lead:].reshape(3, stride)[:, :n] = m
    mask = to_dev(host)[lead:].view(3, stride)[:, :n]
    idx = torch.full((3, n + 5), -9, dtype=torch.int32, device="cuda")
    cnt = torch.full((3,), -9, dtype=torch.int32, device="cuda")
    compact(mask, idx, cnt, entry)
    torch.cuda.synchronize()
    idx_ref, cnt_ref = oracle.mask_compact(m)
    ci, ii = cnt.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(ci, cnt_ref)
    for r in range(3):
        assert np.array_equal(ii[r, :ci[r]], idx_ref[r, :ci[r]])
        assert np.all(ii[r, ci[r]:] == -9)        # untouched past the count


@pytest.mark.parametrize("n", [(1 << 20) - 5, 1 << 20, (1 << 20) + 517])
def test_compaction_long_rows(n):
    """Rows of up to 2^20 cells keep their kept bits in LDS between the two passes; longer
    rows read the mask twice.  Both sides of that limit, bit-exact."""
    import torch
    from mla_flash_attention_amd import binding as B
    g = np.random.default_rng(n)
    m = np.stack([synth.sparse_runs_mask(n, g, max_gap=2312, max_run=256) for _ in range(2)])
    stride = n + 8 - n % 8
    host = np.full(2 * stride, 0x1234, np.uint16)
    host.reshape(2, stride)[:, :n] = m
    mask = to_dev(host).view(2, stride)[:, :n]
    idx = torch.full((2, n), -9, dtype=torch.int32, device="cuda")
    cnt = torch.full((2,), -9, dtype=torch.int32, device="cuda")
    B.fa_mask_compact(mask, idx, cnt)
    torch.cuda.synchronize()
    idx_ref, cnt_ref = oracle.mask_compact(m)
    ci, ii = cnt.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(ci, cnt_ref)
    for r in range(2):
        assert np.array_equal(ii[r, :ci[r]], idx_ref[r, :ci[r]])
        assert np.all(ii[r, ci[r]:] == -9)


@pytest.mark.parametrize("n", [1, 7, 4095, 4096, 4097, 8191, 131072, 131073, 1 << 22, (1 << 22) + 1])
def test_compaction_chunked_sizes(n):
    """The chunked compaction at and around its 4096-cell chunk boundaries, and on both
    sides of its 2^22-cell limit (past it the one-workgroup kernel runs and the workspace
    stays untouched); two rows of runs plus one fully kept row, bit-exact."""
    import torch
    g = np.random.default_rng(n + 11)
    m = np.stack([synth.sparse_runs_mask(n, g, max_gap=900, max_run=300) for _ in range(2)]
                 + [np.zeros(n, np.uint16)])
    stride = n + 8 - n % 8
    host = np.full(3 * stride, 0x1234, np.uint16)
    host.reshape(3, stride)[:, :n] = m
    mask = to_dev(host).view(3, stride)[:, :n]
    idx = torch.full((3, n), -9, dtype=torch.int32, device="cuda")
    cnt = torch.full((3,), -9, dtype=torch.int32, device="cuda")
    compact(mask, idx, cnt, "chunked")
    idx_ref, cnt_ref = oracle.mask_compact(m)
    ci, ii = cnt.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(ci, cnt_ref)
    for r in range(3):
        assert np.array_equal(ii[r, :ci[r]], idx_ref[r, :ci[r]])
        assert np.all(ii[r, ci[r]:] == -9)


# ---------------------------------------------------------------- rows past one launch
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_rows_past_the_grid_limit(kind):
    """More query rows than one launch's grid holds (65535): 70,000 rows whose inputs repeat
    every 1000 rows.  Every row must equal its twin among the first 1000 bitwise, and
    those match the oracle."""
    import torch
    from mla_flash_attention_amd import binding as B
    reps = 70
    if kind == "decode":
        p = synth.make_problem(kind="decode", n_seq=1000, n_head=16, n_kv=40, seed=77)
        q = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK)).repeat(reps, 1, 1)
        kv = to_dev(p.kv).repeat(reps, 1, 1)
        out = torch.empty((reps * p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, n_split=1)
    else:
        p = synth.make_problem(kind="prefill", n_tok=1000, n_head=16, n_kv=40, seed=78, causal=False)
        q = to_dev(p.q.reshape(p.n_tok, p.n_head, synth.DK)).repeat(reps, 1, 1)
        kv = to_dev(p.kv.reshape(p.n_kv, -1))
        out = torch.empty((reps * p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
        B.mla_fa_prefill(q, p.q_type, kv, p.kv_type, p.scale, out, causal=False, n_split=1)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(reps, -1, p.n_head, synth.DV)
    assert np.array_equal(got, np.broadcast_to(got[:1], got.shape)), "rows past 65535 differ from their twins"
    assert_parity(got[0].reshape(-1, synth.DV).astype(np.float64), oracle.attention_problem(p), f"{kind} first rows")


def test_sparse_index_out_of_range_is_clamped():
    """Index-list entries outside [0, n_kv) are clamped in the kernel (documented: the
    result is then unspecified, but every read stays inside the cache).  A list with such
    entries gives exactly the output of the same list clamped on the host."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=2, n_head=16, n_kv=3000, seed=79)
    g = np.random.default_rng(79)
    good = np.stack([np.sort(g.choice(p.n_kv, 900, replace=False)) for _ in range(2)]).astype(np.int64)
    bad = good.copy()
    bad[0, [0, 100, 899]] = [-3, p.n_kv + 5, 1 << 30]
    bad[1, [1, 64, 65]] = [-(1 << 30), p.n_kv, -1]
    outs = []
    for lst in (bad, np.clip(bad, 0, p.n_kv - 1)):
        q = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK))
        kv = to_dev(p.kv)
        full = np.zeros((2, p.n_kv), np.int32)          # index rows are n_kv apart
        full[:, :900] = lst
        idx = torch.from_numpy(full).cuda()
        cnt = torch.full((2,), 900, dtype=torch.int32, device="cuda")
        out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
        ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, 3)
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, kv_idx=idx, kv_idx_count=cnt, n_split=3,
                        workspace=ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1])


def test_decode_cache_past_2gib():
    """One sequence over a 2,000,003-row bf16 cache (2.3 GB: row offsets past 2^31 bytes),
    automatic split count; the whole output against the oracle."""
    p = synth.make_problem(kind="decode", n_seq=1, n_head=16, n_kv=2_000_003, seed=80)
    assert p.n_kv * 1152 > (1 << 31)
    got, _ = run_decode(p)
    assert_parity(got, oracle.attention_problem(p), "decode 2.3 GB cache")


@pytest.mark.parametrize("kv_type", [Q8, BF16])
def test_decode_padded_cache_rows(kv_type):
    """Cache rows stored at a padded stride (Q8_0: 640 B for 612, bf16: 1280 B for 1152),
    so no tile is one contiguous block; sizes with full and ragged tiles."""
    import torch
    from mla_flash_attention_amd import binding as B
    p = synth.make_problem(kind="decode", n_seq=2, n_head=128, n_kv=3000, kv_type=kv_type, seed=81)
    row = p.kv.shape[-1]
    pad = 640 if kv_type == Q8 else 1280 // 2        # bytes for Q8_0 rows; elements for 16-bit
    padded = np.zeros(p.kv.shape[:-1] + (pad,), dtype=p.kv.dtype)
    padded[..., :row] = p.kv
    kv = to_dev(padded)[..., :row]                   # strided view: row stride = the padded row
    q = to_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK))
    out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, 0)
    B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy().reshape(-1, synth.DV).astype(np.float64), oracle.attention_problem(p),
                  f"padded rows {kv_type}")
