"""The achievable-peak micro-benchmarks (include/mla_peaks.h) do the work they claim:
every byte read, every MFMA issued, every LDS word read shows up in the sinks, whose
values the host predicts exactly.  They are measurement support for bench.py, not part
of the attention path."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def P():
    from mla_flash_attention_amd import peaks
    peaks.lib()
    return peaks


def _xor_all(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.astype(np.uint32).ravel()))


@pytest.mark.parametrize("n_wg", [1, 37, 1024])
def test_hbm_read_sees_every_word(P, n_wg):
    # 64 MiB + 48 bytes: not a multiple of the grid's stride, so the tail loop runs
    n = (64 << 20) // 4 + 12
    buf = torch.zeros(n, dtype=torch.int32, device="cuda")
    marks = {5: 0x12345678, 1000003: 0x0F0F0F0F, n - 1: 0x7EADBEEF}
    for i, v in marks.items():
        buf[i] = v
    sink = torch.zeros(n_wg, dtype=torch.int32, device="cuda")
    P.hbm_read(buf, sink, n_wg)
    torch.cuda.synchronize()
    want = 0
    for v in marks.values():
        want ^= v
    assert _xor_all(sink.cpu().numpy()) == want


def test_mfma_chains_accumulate_exactly(P):
    n_wg, iters = 3, 100
    sink = torch.full((n_wg * P.THREADS,), -1.0, dtype=torch.float32, device="cuda")
    P.mfma_bf16(iters, 2.0 ** -10, sink, n_wg)
    torch.cuda.synchronize()
    # 8 chains x 4 values x (32 * 2^-10 per MFMA) x iters
    assert torch.all(sink.cpu() == float(iters)), sink[:8]


def _lds_word(w: np.ndarray) -> np.ndarray:
    h = (w.astype(np.uint64) * 40503) & 0xFFFF
    return (h * 0x10001).astype(np.uint32)


@pytest.mark.parametrize("iters", [1, 2, 5])
def test_lds_b128_reads_every_slot(P, iters):
    # step `it` of wave v reads the 8 KiB slot s = 4 (it mod 2) + v; the sink folds the
    # first word of every 16-byte read: words 4 l + 256 i of the slot
    n_wg = 5
    sink = torch.zeros(n_wg, dtype=torch.int32, device="cuda")
    P.lds_read(iters, False, sink, n_wg)
    torch.cuda.synchronize()
    words = _lds_word(np.arange(16384))
    want = 0
    for it in range(iters):
        for v in range(4):
            s = 4 * (it % 2) + v
            want ^= _xor_all(words[2048 * s:2048 * (s + 1):4])
    assert want != 0
    got = sink.cpu().numpy().astype(np.uint32)
    assert np.all(got == want), (got, want)


def test_lds_transpose_reads_run(P):
    # the transpose read permutes 16-bit halves across lanes, so only invariants are
    # checked: every workgroup sees the same data, and (both halves of every word being
    # equal) the XOR of the low halves equals the XOR of the high halves
    n_wg = 4
    sink = torch.zeros(n_wg, dtype=torch.int32, device="cuda")
    P.lds_read(3, True, sink, n_wg)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().astype(np.uint32)
    assert np.all(got == got[0])
    assert (int(got[0]) & 0xFFFF) == (int(got[0]) >> 16)
