"""The C-ABI library: it loads, exports every symbol include/mla_fa.h declares, and its
host-side validation rejects bad arguments before any HIP call (CPU only: every call
here returns from the validation layer, no kernel is launched)."""
import ctypes
import os
import re

import pytest

from mla_flash_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="mla_fa.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"^(?:const char \*|int |size_t )\s*(\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmlafa.so is not built")
    return B.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_peaks_library_exports_and_validates():
    """libmlapeaks.so (include/mla_peaks.h) loads, exports what its header declares, and
    rejects bad arguments before launching anything."""
    from mla_flash_attention_amd import peaks as P
    if not os.path.exists(P.LIB_PATH):
        pytest.fail("libmlapeaks.so is not built")
    names = _declared("mla_peaks.h")
    assert set(names) == set(P.EXPORTS), names
    Lp = P.lib()
    for n in names:
        assert hasattr(Lp, n), n
    sink = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation
    assert Lp.mla_peak_hbm_read(None, 1024, sink, 1, None) == -1
    assert Lp.mla_peak_hbm_read(ctypes.c_void_p(16), 1000, sink, 1, None) == -1     # not a multiple of 16
    assert Lp.mla_peak_hbm_read(ctypes.c_void_p(8), 1024, sink, 1, None) == -1      # misaligned
    assert Lp.mla_peak_hbm_read(ctypes.c_void_p(16), 1024, sink, 0, None) == -1     # no workgroups
    assert Lp.mla_peak_mfma_bf16(0, 1.0, sink, 1, None) == -1
    assert Lp.mla_peak_mfma_bf16(1, 1.0, None, 1, None) == -1
    assert Lp.mla_peak_lds_read(0, 0, sink, 1, None) == -1
    assert Lp.mla_peak_lds_read(1, 1, sink, 0, None) == -1


def test_version_and_strerror(L):
    assert B.mla_fa_version() >= 10000
    for s in (0, -1, -2, -3, -4):
        assert B.strerror(s)
    assert B.strerror(-99) == "unknown status"


def test_workspace_and_splits(L):
    assert B.mla_fa_auto_splits(2048, 128, 4096, B.MLA_FA_BF16) == 1
    s = B.mla_fa_auto_splits(4, 128, 32768, B.MLA_FA_BF16)
    assert 1 < s <= 1024
    assert B.mla_fa_workspace_size(4, 128, 32768, B.MLA_FA_BF16, 1) == 0
    # per split, row and head: m, l and two scales (fp32) and 512 f16 values; then a 1 KiB tail
    assert B.mla_fa_workspace_size(4, 128, 32768, B.MLA_FA_BF16, 8) == 8 * 4 * 128 * (4 * 4 + 512 * 2) + 1024
    assert B.mla_fa_workspace_size(4, 128, 32768, B.MLA_FA_BF16, 0) == s * 4 * 128 * (4 * 4 + 512 * 2) + 1024
    assert B.mla_fa_workspace_size(4, 100, 32768, B.MLA_FA_BF16, 8) == 0     # unsupported heads


FAKE = 1 << 20    # a 16-byte-aligned non-null address; never dereferenced on these paths


def _decode(L, **kw):
    a = dict(q=FAKE, qt=B.MLA_FA_BF16, kv=FAKE, kvt=B.MLA_FA_BF16, rs=1152, ss=1152 * 64, n_seq=1,
             H=128, n_kv=64, mask=None, ms=0, idx=None, cnt=None, iss=0, scale=0.1, out=FAKE,
             n_split=1, ws=None, wsb=0)
    a.update(kw)
    return L.mla_fa_decode(a["q"], a["qt"], a["kv"], a["kvt"], a["rs"], a["ss"], a["n_seq"], a["H"],
                           a["n_kv"], a["mask"], a["ms"], a["idx"], a["cnt"], a["iss"],
                           ctypes.c_float(a["scale"]), a["out"], a["n_split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.MLA_FA_ERR_INVALID),
    (dict(kv=None), B.MLA_FA_ERR_INVALID),
    (dict(out=None), B.MLA_FA_ERR_INVALID),
    (dict(n_kv=0), B.MLA_FA_ERR_INVALID),
    (dict(n_kv=1 << 31), B.MLA_FA_ERR_INVALID),
    (dict(n_seq=0), B.MLA_FA_ERR_INVALID),
    (dict(H=100), B.MLA_FA_ERR_UNSUPPORTED),
    (dict(H=144), B.MLA_FA_ERR_UNSUPPORTED),
    (dict(H=0), B.MLA_FA_ERR_INVALID),
    (dict(qt=B.MLA_FA_F16), B.MLA_FA_ERR_UNSUPPORTED),        # f16 q with bf16 cache
    (dict(qt=7), B.MLA_FA_ERR_INVALID),
    (dict(kvt=9), B.MLA_FA_ERR_INVALID),
    (dict(q=FAKE + 8), B.MLA_FA_ERR_INVALID),                   # misaligned q
    (dict(rs=1000), B.MLA_FA_ERR_INVALID),                      # row stride < row bytes
    (dict(rs=1160), B.MLA_FA_ERR_INVALID),                      # not a multiple of 16
    (dict(ss=-16), B.MLA_FA_ERR_INVALID),
    (dict(scale=float("inf")), B.MLA_FA_ERR_INVALID),
    (dict(scale=float("nan")), B.MLA_FA_ERR_INVALID),
    (dict(idx=FAKE), B.MLA_FA_ERR_INVALID),                     # index list without count
    (dict(n_split=-1), B.MLA_FA_ERR_INVALID),
    (dict(n_split=1025), B.MLA_FA_ERR_INVALID),
    (dict(n_split=4), B.MLA_FA_ERR_WORKSPACE),                  # split without a workspace
    (dict(n_split=4, ws=FAKE, wsb=16), B.MLA_FA_ERR_WORKSPACE), # workspace too small
    (dict(n_seq=2, mask=FAKE, ms=10), B.MLA_FA_ERR_INVALID),    # mask rows overlap
    (dict(kvt=B.MLA_FA_Q8_0, rs=600), B.MLA_FA_ERR_INVALID),    # Q8_0 row is 612 bytes
    (dict(kvt=B.MLA_FA_Q8_0, rs=614), B.MLA_FA_ERR_INVALID),    # Q8_0 stride not 4-aligned
    (dict(kvt=B.MLA_FA_Q8_0, rs=(1 << 26) + 4), B.MLA_FA_ERR_INVALID),  # Q8_0 stride past 2^26 B
    (dict(n_seq=1 << 24), B.MLA_FA_ERR_INVALID),                # rows x heads past the merge grid
])
def test_decode_validation(L, kw, status):
    assert _decode(L, **kw) == status


def test_prefill_validation(L):
    f = lambda **kw: L.mla_fa_prefill(kw.get("q", FAKE), B.MLA_FA_BF16, FAKE, B.MLA_FA_BF16, 1152,
                                      kw.get("n_tok", 8), 128, kw.get("n_kv", 16), kw.get("causal", 1),
                                      None, 0, ctypes.c_float(0.1), FAKE, 1, None, 0, None)
    assert f(n_tok=17, n_kv=16) == B.MLA_FA_ERR_INVALID            # causal chunk longer than cache
    assert f(q=None) == B.MLA_FA_ERR_INVALID
    assert f(n_tok=0) == B.MLA_FA_ERR_INVALID


def test_merge_grid_limit(L):
    """One merge workgroup per (row, head): rows x heads beyond 2^31 - 1 is rejected before
    any launch."""
    assert L.mla_fa_merge_partials(1 << 24, 128, 4, FAKE, FAKE, 1 << 62, None) == B.MLA_FA_ERR_INVALID


def test_compact_validation(L):
    f = lambda m=FAKE, ms=100, rows=1, n=100, idx=FAKE, istr=100, cnt=FAKE: L.fa_mask_compact(
        m, ms, rows, n, idx, istr, cnt, None)
    assert f(m=None) == B.MLA_FA_ERR_INVALID
    assert f(idx=None) == B.MLA_FA_ERR_INVALID
    assert f(cnt=None) == B.MLA_FA_ERR_INVALID
    assert f(istr=99) == B.MLA_FA_ERR_INVALID
    assert f(rows=2, ms=50) == B.MLA_FA_ERR_INVALID
    assert f(n=0) == B.MLA_FA_ERR_INVALID
    assert f(m=FAKE + 1) == B.MLA_FA_ERR_INVALID


def test_compact_ws_validation(L):
    """The chunked compaction's argument checks (none of these launch anything)."""
    assert B.fa_mask_compact_workspace_size(1, 131072) == 32 * 4
    assert B.fa_mask_compact_workspace_size(3, 4097) == 3 * 2 * 4
    assert B.fa_mask_compact_workspace_size(1, (1 << 22) + 1) == 0     # past the chunked limit
    assert B.fa_mask_compact_workspace_size(0, 100) == 0
    assert B.fa_mask_compact_workspace_size(70000, 100) == 0           # past the grid's y limit
    f = lambda m=FAKE, ms=4096, rows=1, n=4096, idx=FAKE, istr=4096, cnt=FAKE, ws=FAKE, wsb=1 << 20: \
        L.fa_mask_compact_ws(m, ms, rows, n, idx, istr, cnt, ws, wsb, None)
    assert f(m=None) == B.MLA_FA_ERR_INVALID
    assert f(idx=None) == B.MLA_FA_ERR_INVALID
    assert f(cnt=None) == B.MLA_FA_ERR_INVALID
    assert f(istr=4095) == B.MLA_FA_ERR_INVALID
    assert f(rows=2, ms=100) == B.MLA_FA_ERR_INVALID
    assert f(n=0) == B.MLA_FA_ERR_INVALID
    assert f(m=FAKE + 1) == B.MLA_FA_ERR_INVALID
    assert f(ws=None, wsb=0) == B.MLA_FA_ERR_WORKSPACE                  # the chunked form applies
    assert f(wsb=3) == B.MLA_FA_ERR_WORKSPACE
    assert f(ws=FAKE + 2) == B.MLA_FA_ERR_WORKSPACE                     # not 4-byte aligned


def test_merge_validation(L):
    assert L.mla_fa_merge_partials(4, 128, 8, FAKE, None, 0, None) == B.MLA_FA_ERR_WORKSPACE
    assert L.mla_fa_merge_partials(4, 100, 8, FAKE, FAKE, 1 << 30, None) == B.MLA_FA_ERR_UNSUPPORTED
    assert L.mla_fa_merge_partials(0, 128, 8, FAKE, FAKE, 1 << 30, None) == B.MLA_FA_ERR_INVALID
    # n_split == 1 has nothing to merge
    assert L.mla_fa_merge_partials(4, 128, 1, FAKE, None, 0, None) == B.MLA_FA_OK


def _attend(L, **kw):
    a = dict(q=FAKE, qt=B.MLA_FA_BF16, kv=FAKE, kvt=B.MLA_FA_BF16, rs=1152, ss=1152 * 64, n_seq=2, n_tok=2,
             H=128, n_kv=64, kv_len=None, causal=0, mask=None, ms=0, mt=0, idx=None, cnt=None, iss=0, its=0,
             alibi=None, sinks=None, softcap=0.0, scale=0.1, out=FAKE, n_split=1, ws=None, wsb=0)
    a.update(kw)
    return L.mla_fa_attend(a["q"], a["qt"], a["kv"], a["kvt"], a["rs"], a["ss"], a["n_seq"], a["n_tok"],
                           a["H"], a["n_kv"], a["kv_len"], a["causal"], a["mask"], a["ms"], a["mt"],
                           a["idx"], a["cnt"], a["iss"], a["its"], a["alibi"], a["sinks"],
                           ctypes.c_float(a["softcap"]), ctypes.c_float(a["scale"]), a["out"], a["n_split"],
                           a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(softcap=-1.0), B.MLA_FA_ERR_INVALID),                      # negative softcap
    (dict(softcap=float("inf")), B.MLA_FA_ERR_INVALID),              # non-finite softcap
    (dict(kv_len=FAKE + 2), B.MLA_FA_ERR_INVALID),                   # misaligned lengths
    (dict(alibi=FAKE + 1), B.MLA_FA_ERR_INVALID),                    # misaligned slopes
    (dict(sinks=FAKE + 2), B.MLA_FA_ERR_INVALID),                    # misaligned sinks
    (dict(causal=1, n_tok=65), B.MLA_FA_ERR_INVALID),                # causal, no lengths, n_tok > n_kv
    (dict(n_tok=0), B.MLA_FA_ERR_INVALID),                           # no query token
    (dict(H=120), B.MLA_FA_ERR_UNSUPPORTED),                         # heads not a multiple of 16
    (dict(qt=B.MLA_FA_F16, kvt=B.MLA_FA_BF16), B.MLA_FA_ERR_UNSUPPORTED),
    (dict(n_split=4, ws=FAKE, wsb=16), B.MLA_FA_ERR_WORKSPACE),      # workspace too small
    (dict(idx=FAKE), B.MLA_FA_ERR_INVALID),                          # index lists without counts
    (dict(cnt=FAKE), B.MLA_FA_ERR_INVALID),                          # counts without index lists
    (dict(idx=FAKE, cnt=FAKE, iss=128, its=64, causal=1), B.MLA_FA_ERR_INVALID),   # sparse + causal
    (dict(idx=FAKE, cnt=FAKE, iss=128, its=64, kv_len=FAKE), B.MLA_FA_ERR_INVALID),  # sparse + lengths
    (dict(idx=FAKE + 2, cnt=FAKE, iss=128, its=64), B.MLA_FA_ERR_INVALID),  # misaligned lists
    (dict(idx=FAKE, cnt=FAKE, iss=128, its=63), B.MLA_FA_ERR_INVALID),     # token rows overlap
    (dict(idx=FAKE, cnt=FAKE, iss=63, its=64), B.MLA_FA_ERR_INVALID),      # sequence rows overlap
    (dict(idx=FAKE, cnt=FAKE, iss=-128, its=64), B.MLA_FA_ERR_INVALID),
])
def test_attend_validation(L, kw, status):
    assert _attend(L, **kw) == status


def _mha(L, **kw):
    a = dict(q=FAKE, qt=B.MLA_FA_BF16, k=FAKE, v=FAKE, kvt=B.MLA_FA_BF16, ks=128 * 384, vs=128 * 256, n_tok=8,
             H=128, n_kv=16, causal=1, mask=None, ms=0, scale=0.1, out=FAKE)
    a.update(kw)
    return L.mla_fa_prefill_mha(a["q"], a["qt"], a["k"], a["v"], a["kvt"], a["ks"], a["vs"], a["n_tok"], a["H"],
                                a["n_kv"], a["causal"], a["mask"], a["ms"], ctypes.c_float(a["scale"]), a["out"],
                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.MLA_FA_ERR_INVALID),
    (dict(v=None), B.MLA_FA_ERR_INVALID),
    (dict(n_tok=17), B.MLA_FA_ERR_INVALID),                          # causal chunk longer than the cache
    (dict(n_tok=0), B.MLA_FA_ERR_INVALID),
    (dict(n_kv=0), B.MLA_FA_ERR_INVALID),
    (dict(H=0), B.MLA_FA_ERR_INVALID),
    (dict(ks=128 * 384 - 16), B.MLA_FA_ERR_INVALID),                 # key rows overlap
    (dict(vs=128 * 256 + 8), B.MLA_FA_ERR_INVALID),                  # value stride not a multiple of 16
    (dict(k=FAKE + 8), B.MLA_FA_ERR_INVALID),                        # misaligned keys
    (dict(mask=FAKE + 8, ms=16), B.MLA_FA_ERR_INVALID),              # mask not 16-byte aligned
    (dict(mask=FAKE, ms=20), B.MLA_FA_ERR_INVALID),                  # mask stride not a multiple of 8
    (dict(mask=FAKE, ms=8), B.MLA_FA_ERR_INVALID),                   # mask rows shorter than n_kv
    (dict(scale=float("nan")), B.MLA_FA_ERR_INVALID),
    (dict(qt=B.MLA_FA_F16), B.MLA_FA_ERR_UNSUPPORTED),               # q and cache types differ
    (dict(qt=B.MLA_FA_Q8_0, kvt=B.MLA_FA_Q8_0), B.MLA_FA_ERR_INVALID),
    (dict(kvt=B.MLA_FA_Q8_0), B.MLA_FA_ERR_UNSUPPORTED),
])
def test_prefill_mha_validation(L, kw, status):
    assert _mha(L, **kw) == status


def _absorbed(L, **kw):
    a = dict(qn=FAKE, qp=FAKE, qt=B.MLA_FA_BF16, wk=FAKE, wv=FAKE, kv=FAKE, kvt=B.MLA_FA_BF16, rs=1152, ss=1152 * 64,
             n_seq=2, n_tok=1, H=128, n_kv=64, kv_len=None, causal=0, mask=None, ms=0, mt=0, scale=0.1, out=FAKE,
             n_split=1, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.mla_fa_absorbed(a["qn"], a["qp"], a["qt"], a["wk"], a["wv"], a["kv"], a["kvt"], a["rs"], a["ss"],
                             a["n_seq"], a["n_tok"], a["H"], a["n_kv"], a["kv_len"], a["causal"], a["mask"], a["ms"],
                             a["mt"], ctypes.c_float(a["scale"]), a["out"], a["n_split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qn=None), B.MLA_FA_ERR_INVALID),
    (dict(qp=None), B.MLA_FA_ERR_INVALID),
    (dict(wk=None), B.MLA_FA_ERR_INVALID),
    (dict(wv=FAKE + 8), B.MLA_FA_ERR_INVALID),                       # misaligned weights
    (dict(ws=FAKE + 16), B.MLA_FA_ERR_INVALID),                      # workspace not 256-byte aligned
    (dict(n_tok=0), B.MLA_FA_ERR_INVALID),
    (dict(H=120), B.MLA_FA_ERR_UNSUPPORTED),
    (dict(qt=B.MLA_FA_F16), B.MLA_FA_ERR_UNSUPPORTED),               # query and cache types differ
    (dict(causal=1, n_tok=65), B.MLA_FA_ERR_INVALID),
    (dict(ws=None, wsb=0), B.MLA_FA_ERR_WORKSPACE),
    (dict(wsb=1024), B.MLA_FA_ERR_WORKSPACE),
    (dict(ws=None, wsb=0, qn=None), B.MLA_FA_ERR_INVALID),           # argument errors come first
])
def test_absorbed_validation(L, kw, status):
    assert _absorbed(L, **kw) == status


def test_absorbed_workspace_size(L):
    n = L.mla_fa_absorbed_workspace_size(4, 128, 32768, B.MLA_FA_BF16, 1)
    assert n >= 4 * 128 * (576 * 2 + 512 * 4)
    assert L.mla_fa_absorbed_workspace_size(4, 128, 32768, B.MLA_FA_BF16, 8) > n    # plus the partials
    assert L.mla_fa_absorbed_workspace_size(0, 128, 32768, B.MLA_FA_BF16, 1) == 0


# ---------------------------------------------------------------- launch failures
# MLA_FA_FAIL_LAUNCH=k: the call launches nothing and reports its k-th launch as failed,
# so every MLA_FA_ERR_HIP return is reached here without a GPU.
@pytest.mark.parametrize("k,status", [(1, B.MLA_FA_ERR_HIP), (2, B.MLA_FA_ERR_HIP), (3, B.MLA_FA_OK)])
def test_decode_launch_failure(L, monkeypatch, k, status):
    """Decode with splits is two launches: the attention, then the merge."""
    monkeypatch.setenv("MLA_FA_FAIL_LAUNCH", str(k))
    assert _decode(L, n_split=4, ws=FAKE, wsb=1 << 30) == status
    assert _decode(L, n_split=1) == (B.MLA_FA_ERR_HIP if k == 1 else B.MLA_FA_OK)   # one launch


@pytest.mark.parametrize("k", [1, 2])
def test_two_phase_and_prefill_launch_failures(L, monkeypatch, k):
    monkeypatch.setenv("MLA_FA_FAIL_LAUNCH", str(k))
    exp = B.MLA_FA_ERR_HIP if k == 1 else B.MLA_FA_OK
    assert L.mla_fa_decode_partials(FAKE, B.MLA_FA_BF16, FAKE, B.MLA_FA_BF16, 1152, 1152 * 64, 1, 128, 64, None, 0,
                                    None, None, 0, ctypes.c_float(0.1), FAKE, 4, FAKE, 1 << 30, None) == exp
    assert L.mla_fa_merge_partials(4, 128, 8, FAKE, FAKE, 1 << 30, None) == exp
    pre = L.mla_fa_prefill(FAKE, B.MLA_FA_BF16, FAKE, B.MLA_FA_BF16, 1152, 8, 128, 16, 1, None, 0,
                           ctypes.c_float(0.1), FAKE, 2, FAKE, 1 << 30, None)
    assert pre == B.MLA_FA_ERR_HIP
    assert _attend(L, n_split=2, ws=FAKE, wsb=1 << 30) == B.MLA_FA_ERR_HIP
    assert _mha(L) == exp
    assert L.fa_mask_compact(FAKE, 100, 1, 100, FAKE, 100, FAKE, None) == exp
    assert L.fa_mask_compact_ws(FAKE, 4096, 1, 4096, FAKE, 4096, FAKE, FAKE, 1 << 20, None) == exp   # chunked
    assert L.fa_mask_compact_ws(FAKE + 2, 100, 1, 100, FAKE, 100, FAKE, None, 0, None) == exp        # one-WG (unaligned)


@pytest.mark.parametrize("n_split", [1, 4])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_absorbed_launch_failures(L, monkeypatch, k, n_split):
    """Absorbed decode: three launches, query projection, attention, then the output
    projection (fused with the merge of a split plan)."""
    monkeypatch.setenv("MLA_FA_FAIL_LAUNCH", str(k))
    assert _absorbed(L, n_split=n_split) == (B.MLA_FA_ERR_HIP if k <= 3 else B.MLA_FA_OK)


def test_header_is_plain_c(tmp_path):
    """include/mla_fa.h needs no HIP header and compiles as strict C99 and as C++ (the
    boundary takes plain pointers, sizes and a void * stream)."""
    import shutil
    import subprocess
    inc = os.path.join(ROOT, "include")
    src = tmp_path / "use.c"
    src.write_text('#include "mla_fa.h"\nint main(void) { return mla_fa_version() > 0 ? 0 : 1; }\n')
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++11")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        args = [cc, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-I", inc]
        if cc == "g++":
            args += ["-x", "c++"]
        r = subprocess.run(args + [str(src)], capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, r.stderr
