"""CPU oracle for MLA flash attention (fp64, plain definition).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by the
CPU-baseline leg of bench.py, never by the product package.  It shares no code with
the HIP path; both receive the same bytes from the seeded generators.

What each function follows is documented in mla_oracle.c and in the docstrings here.
Every function is pinned (tests/test_oracle_pins.py, test_oracle_ext_pins.py,
test_oracle_mha_pins.py, test_oracle_absorbed_pins.py); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16, Q8_0 = 1, 2, 3
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_mla_attention.restype = ctypes.c_int64
        lib.oracle_mla_attention.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_mla_attention_ext.restype = ctypes.c_int64
        lib.oracle_mla_attention_ext.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.oracle_mla_attention_q64.restype = ctypes.c_int64
        lib.oracle_mla_attention_q64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_mha_attention.restype = ctypes.c_int64
        lib.oracle_mha_attention.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_mask_compact.restype = None
        lib.oracle_mask_compact.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p]
        _LIB = lib
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_lib().oracle_num_threads())


def decode(bits: np.ndarray, type_id: int) -> np.ndarray:
    """Decode f16/bf16 bits (uint16) or Q8_0 bytes (uint8, one row) to float64."""
    a = np.ascontiguousarray(bits)
    if type_id == Q8_0:
        n = a.size // 34 * 32
    else:
        assert a.dtype == np.uint16
        n = a.size
    out = np.empty(n, dtype=np.float64)
    rc = _lib().oracle_decode(_ptr(a), type_id, n, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode failed")
    return out.reshape(a.shape if type_id != Q8_0 else (n,))


def decode_q8_0_rows(rows: np.ndarray, dk: int) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1, dk // 32 * 34)
    return np.stack([decode(r, Q8_0) for r in rows]).reshape(*rows.shape[:-1], dk)


def attention(q, q_type, kv, kv_type, n_seq, n_tok, n_head, n_kv, scale, *, causal=False,
              mask=None, rows=None, dk=576, dv=512, kv_shared=False, return_stats=False,
              kv_len=None, alibi=None, sinks=None, softcap=0.0):
    """fp64 attention outputs [len(rows) or n_seq*n_tok*n_head][dv].

    q: uint16 [n_seq][n_tok][n_head][dk]; kv: [n_seq or 1][n_kv][row] (uint16 rows of
    dk elements, or uint8 Q8_0 rows); mask: uint16 [n_seq][n_tok][n_kv] or None;
    scale: the fp32 value passed to the GPU (widened here); rows: flat row ids
    (s*n_tok + t)*n_head + h.  kv_len: int [n_seq] valid cells per sequence (None = all
    n_kv); alibi / sinks: float [n_head] slopes / sink logits (the fp32 values passed to
    the GPU, widened); softcap: 0 = off.
    """
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv = np.ascontiguousarray(kv)
    assert q.size == n_seq * n_tok * n_head * dk
    row_bytes = kv.shape[-1] * kv.itemsize
    assert kv.shape[-2] == n_kv
    seq_stride = 0 if (kv_shared or kv.shape[0] == 1 and n_seq > 1) else n_kv * row_bytes
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.uint16).reshape(n_seq, n_tok, n_kv)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.size
    else:
        n_rows = n_seq * n_tok * n_head
    if kv_len is not None:
        kv_len = np.ascontiguousarray(kv_len, dtype=np.int32).reshape(n_seq)
    if alibi is not None:
        alibi = np.ascontiguousarray(np.asarray(alibi, dtype=np.float32), dtype=np.float64).reshape(n_head)
    if sinks is not None:
        sinks = np.ascontiguousarray(np.asarray(sinks, dtype=np.float32), dtype=np.float64).reshape(n_head)
    out = np.zeros((n_rows, dv), dtype=np.float64)
    rmax = np.zeros(n_rows, dtype=np.float64)
    rsum = np.zeros(n_rows, dtype=np.float64)
    rc = _lib().oracle_mla_attention_ext(
        _ptr(q), q_type, _ptr(kv), kv_type, row_bytes, seq_stride, n_seq, n_tok, n_head,
        n_kv, dk, dv, _ptr(kv_len), 1 if causal else 0, _ptr(mask), n_kv, n_tok * n_kv,
        _ptr(alibi), _ptr(sinks), float(np.float32(softcap)), float(np.float32(scale)),
        _ptr(rows), n_rows, _ptr(out), _ptr(rmax), _ptr(rsum))
    if rc < 0:
        raise ValueError(f"oracle_mla_attention_ext failed ({rc})")
    if return_stats:
        return out, rmax, rsum
    return out


def attention_problem(p, rows=None, return_stats=False):
    """Oracle outputs for a synthetic problem object (duck-typed: q, kv, mask, ...;
    optional kv_len, alibi, sinks, softcap)."""
    return attention(p.q, p.q_type, p.kv, p.kv_type, p.n_seq, p.n_tok, p.n_head, p.n_kv,
                     p.scale, causal=p.causal, mask=p.mask, rows=rows,
                     dk=p.q.shape[-1], dv=512 if p.q.shape[-1] == 576 else p.q.shape[-1],
                     return_stats=return_stats, kv_len=getattr(p, "kv_len", None),
                     alibi=getattr(p, "alibi", None), sinks=getattr(p, "sinks", None),
                     softcap=getattr(p, "softcap", 0.0))


def absorbed_attention(q_nope, q_pe, q_type, w_uk, w_uv, kv, kv_type, n_seq, n_tok, n_head, n_kv, scale, *,
                       causal=False, mask=None, rows=None, kv_len=None, return_latent=False):
    """fp64 MLA attention with the absorbed projections either side, [len(rows) or
    n_seq*n_tok*n_head][128].

    The per-head up-projection of the latent cache is split into W_UK (128 key dims from
    the 512 latent) and W_UV (128 value dims from the 512 latent); instead of
    decompressing every cached row, W_UK is folded into the query and W_UV applied to
    the attention output ("ik_llama.cpp -mla flag deep-dive": wkv_b split per head into
    wk_b / wv_b, "128 x 512 x 128"; "Vulkan backend fused Flash Attention: DeepSeek MLA
    local inference", sections 3.2-3.3 and 6.1: the fused path is logically the
    step-by-step one).  In order:
        q_lat[h] = W_UK[h] q_nope[h]                    (512)
        q[h]     = [q_lat[h], q_pe[h]]                  (576, not rounded)
        O_lat    = latent attention of q over the cache (512; `attention` above, in fp64)
        out[h]   = W_UV[h] O_lat[h]                     (128)
    q_nope uint16 [n_seq][n_tok][n_head][128], q_pe uint16 [..][64] (type q_type);
    w_uk uint16 [n_head][512][128], w_uv uint16 [n_head][128][512] (type q_type, weights
    stored output-major like a linear layer); kv as for `attention`.
    """
    qn = decode(np.ascontiguousarray(q_nope, dtype=np.uint16), q_type).reshape(n_seq, n_tok, n_head, 128)
    qp = decode(np.ascontiguousarray(q_pe, dtype=np.uint16), q_type).reshape(n_seq, n_tok, n_head, 64)
    wk = decode(np.ascontiguousarray(w_uk, dtype=np.uint16), q_type).reshape(n_head, 512, 128)
    wv = decode(np.ascontiguousarray(w_uv, dtype=np.uint16), q_type).reshape(n_head, 128, 512)
    q_lat = np.einsum("sthd,hcd->sthc", qn, wk)
    q64 = np.ascontiguousarray(np.concatenate([q_lat, qp], axis=-1), dtype=np.float64)
    kv = np.ascontiguousarray(kv)
    row_bytes = kv.shape[-1] * kv.itemsize
    assert kv.shape[-2] == n_kv
    seq_stride = 0 if (kv.shape[0] == 1 and n_seq > 1) else n_kv * row_bytes
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.uint16).reshape(n_seq, n_tok, n_kv)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.size
    else:
        n_rows = n_seq * n_tok * n_head
    if kv_len is not None:
        kv_len = np.ascontiguousarray(kv_len, dtype=np.int32).reshape(n_seq)
    o_lat = np.zeros((n_rows, 512), dtype=np.float64)
    rc = _lib().oracle_mla_attention_q64(
        _ptr(q64), _ptr(kv), kv_type, row_bytes, seq_stride, n_seq, n_tok, n_head, n_kv, 576, 512,
        _ptr(kv_len), 1 if causal else 0, _ptr(mask), n_kv, n_tok * n_kv, float(np.float32(scale)),
        _ptr(rows), n_rows, _ptr(o_lat))
    if rc < 0:
        raise ValueError(f"oracle_mla_attention_q64 failed ({rc})")
    heads = (rows if rows is not None else np.arange(n_rows)) % n_head
    out = np.einsum("iec,ic->ie", wv[heads], o_lat)
    return (out, o_lat) if return_latent else out


def mha_attention(q, q_type, k, v, kv_type, scale, *, causal=False, mask=None, rows=None):
    """fp64 per-head attention with separate K and V: q uint16 [n_tok][n_head][dk],
    k uint16 [n_kv][n_head][dk], v uint16 [n_kv][n_head][dv], mask uint16 [n_tok][n_kv] or
    None -> [len(rows) or n_tok*n_head][dv] (rows: flat ids t*n_head + h)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    n_tok, n_head, dk = q.shape
    n_kv, dv = k.shape[0], v.shape[-1]
    assert k.shape == (n_kv, n_head, dk) and v.shape == (n_kv, n_head, dv)
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.uint16).reshape(n_tok, n_kv)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.size
    else:
        n_rows = n_tok * n_head
    out = np.zeros((n_rows, dv), dtype=np.float64)
    rc = _lib().oracle_mha_attention(
        _ptr(q), q_type, _ptr(k), _ptr(v), kv_type, n_head * dk, n_head * dv, n_tok, n_head, n_kv, dk, dv,
        1 if causal else 0, _ptr(mask), n_kv, float(np.float32(scale)), _ptr(rows), n_rows, _ptr(out))
    if rc < 0:
        raise ValueError(f"oracle_mha_attention failed ({rc})")
    return out


def mask_compact(mask2d: np.ndarray):
    """Ascending kept-index lists of each row of an f16-bits mask [rows][n_kv]."""
    m = np.ascontiguousarray(mask2d, dtype=np.uint16)
    if m.ndim == 1:
        m = m[None]
    n_rows, n_kv = m.shape
    idx = np.full((n_rows, n_kv), -1, dtype=np.int32)
    cnt = np.zeros(n_rows, dtype=np.int32)
    _lib().oracle_mask_compact(_ptr(m), n_kv, n_rows, n_kv, _ptr(idx), n_kv, _ptr(cnt))
    return idx, cnt
