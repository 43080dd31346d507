"""ctypes binding of libmlafa (include/mla_fa.h), with the same entry-point names.

Argument marshalling only: tensors are passed as device pointers plus sizes and byte
strides, the current torch stream as the hipStream_t.  Every step of the computation
runs in the library's HIP kernels; there is no fallback of any kind, and importing a
function when the library is missing raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmlafa.so")

MLA_FA_F16, MLA_FA_BF16, MLA_FA_Q8_0 = synth.TYPE_F16, synth.TYPE_BF16, synth.TYPE_Q8_0
MLA_FA_OK, MLA_FA_ERR_INVALID, MLA_FA_ERR_UNSUPPORTED, MLA_FA_ERR_WORKSPACE, MLA_FA_ERR_HIP = 0, -1, -2, -3, -4

EXPORTS = ("mla_fa_strerror", "mla_fa_version", "mla_fa_auto_splits", "mla_fa_workspace_size",
           "mla_fa_decode", "mla_fa_decode_noalloc", "mla_fa_decode_partials", "mla_fa_merge_partials",
           "mla_fa_prefill",
           "mla_fa_attend", "mla_fa_prefill_mha", "mla_fa_absorbed_workspace_size", "mla_fa_absorbed",
           "fa_mask_compact", "fa_mask_compact_workspace_size", "fa_mask_compact_ws")

_LIB = None
_p, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class MlaFaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmlafa.so not built ({LIB_PATH}); run mla_flash_attention_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.mla_fa_strerror.restype = ctypes.c_char_p
        L.mla_fa_strerror.argtypes = [_i]
        L.mla_fa_version.restype = _i
        L.mla_fa_version.argtypes = []
        L.mla_fa_auto_splits.restype = _i
        L.mla_fa_auto_splits.argtypes = [_i, _i, _i64, _i]
        L.mla_fa_workspace_size.restype = _sz
        L.mla_fa_workspace_size.argtypes = [_i, _i, _i64, _i, _i]
        dec = [_p, _i, _p, _i, _i64, _i64, _i, _i, _i64, _p, _i64, _p, _p, _i64, _f, _p, _i, _p, _sz, _p]
        L.mla_fa_decode.restype = _i
        L.mla_fa_decode.argtypes = dec
        L.mla_fa_decode_noalloc.restype = _i
        L.mla_fa_decode_noalloc.argtypes = dec[:-3] + [_p]
        L.mla_fa_decode_partials.restype = _i
        L.mla_fa_decode_partials.argtypes = dec
        L.mla_fa_merge_partials.restype = _i
        L.mla_fa_merge_partials.argtypes = [_i, _i, _i, _p, _p, _sz, _p]
        L.mla_fa_prefill.restype = _i
        L.mla_fa_prefill.argtypes = [_p, _i, _p, _i, _i64, _i, _i, _i64, _i, _p, _i64, _f, _p, _i, _p, _sz, _p]
        L.fa_mask_compact.restype = _i
        L.fa_mask_compact.argtypes = [_p, _i64, _i, _i64, _p, _i64, _p, _p]
        L.fa_mask_compact_workspace_size.restype = _sz
        L.fa_mask_compact_workspace_size.argtypes = [_i, _i64]
        L.fa_mask_compact_ws.restype = _i
        L.fa_mask_compact_ws.argtypes = [_p, _i64, _i, _i64, _p, _i64, _p, _p, _sz, _p]
        L.mla_fa_attend.restype = _i
        L.mla_fa_attend.argtypes = [_p, _i, _p, _i, _i64, _i64, _i, _i, _i, _i64, _p, _i, _p, _i64, _i64,
                                    _p, _p, _i64, _i64, _p, _p, _f, _f, _p, _i, _p, _sz, _p]
        L.mla_fa_absorbed_workspace_size.restype = _sz
        L.mla_fa_absorbed_workspace_size.argtypes = [_i, _i, _i64, _i, _i]
        L.mla_fa_absorbed.restype = _i
        L.mla_fa_absorbed.argtypes = [_p, _p, _i, _p, _p, _p, _i, _i64, _i64, _i, _i, _i, _i64, _p, _i, _p, _i64,
                                      _i64, _f, _p, _i, _p, _sz, _p]
        L.mla_fa_prefill_mha.restype = _i
        L.mla_fa_prefill_mha.argtypes = [_p, _i, _p, _p, _i, _i64, _i64, _i, _i, _i64, _i, _p, _i64, _f, _p, _p]
        _LIB = L
    return _LIB


def strerror(status: int) -> str:
    return lib().mla_fa_strerror(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != MLA_FA_OK:
        raise MlaFaError(status, where)


def _row_stride_bytes(kv: torch.Tensor) -> int:
    return kv.stride(-2) * kv.element_size()


def _seq_stride_bytes(kv: torch.Tensor, n_seq: int) -> int:
    """Bytes between sequences' caches; 0 when one cache serves every sequence."""
    return kv.stride(0) * kv.element_size() if kv.dim() == 3 and kv.shape[0] > 1 else 0


def mla_fa_version() -> int:
    return int(lib().mla_fa_version())


def mla_fa_auto_splits(n_rows: int, n_head: int, n_kv: int, kv_type: int) -> int:
    return int(lib().mla_fa_auto_splits(n_rows, n_head, n_kv, kv_type))


def mla_fa_workspace_size(n_rows: int, n_head: int, n_kv: int, kv_type: int, n_split: int = 0) -> int:
    return int(lib().mla_fa_workspace_size(n_rows, n_head, n_kv, kv_type, n_split))


def workspace_for(n_rows, n_head, n_kv, kv_type, n_split=0, device="cuda"):
    """A device workspace of the size the call needs (None when it needs none)."""
    nbytes = mla_fa_workspace_size(n_rows, n_head, n_kv, kv_type, n_split)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device) if nbytes else None


def _decode_args(q, q_type, kv, kv_type, scale, out, mask, kv_idx, kv_idx_count, n_split,
                 workspace, stream):
    n_seq, n_head = q.shape[0], q.shape[-2]
    n_kv = kv.shape[-2]
    kv_seq_stride = _seq_stride_bytes(kv, n_seq)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(q), q_type, _ptr(kv), kv_type, _row_stride_bytes(kv), kv_seq_stride, n_seq, n_head,
            n_kv, _ptr(mask), 0 if mask is None else mask.stride(0), _ptr(kv_idx), _ptr(kv_idx_count),
            0 if kv_idx is None else kv_idx.stride(0), float(scale), _ptr(out), n_split,
            _ptr(workspace), ws_bytes, _stream(stream))


def mla_fa_decode(q, q_type, kv, kv_type, scale, out, *, mask=None, kv_idx=None, kv_idx_count=None,
                  n_split=0, workspace=None, stream=None):
    """q [n_seq][n_head][576] (int16/uint16 bits), kv [n_seq][n_kv][576 | 612 bytes],
    out fp32 [n_seq][n_head][512]; mask [n_seq][>=n_kv] f16 bits; kv_idx [n_seq][>=n_kv]
    int32 + kv_idx_count [n_seq] int32 for the sparse path."""
    _check(lib().mla_fa_decode(*_decode_args(q, q_type, kv, kv_type, scale, out, mask, kv_idx,
                                             kv_idx_count, n_split, workspace, stream)),
           "mla_fa_decode")
    return out


def mla_fa_decode_noalloc(q, q_type, kv, kv_type, scale, out, *, mask=None, kv_idx=None, kv_idx_count=None,
                          n_split=0, stream=None):
    """mla_fa_decode without a workspace: the split partials live in the library's
    per-GPU scratch (include/mla_fa.h); same arguments otherwise."""
    a = _decode_args(q, q_type, kv, kv_type, scale, out, mask, kv_idx, kv_idx_count, n_split, None, stream)
    _check(lib().mla_fa_decode_noalloc(*(a[:-3] + (a[-1],))), "mla_fa_decode_noalloc")
    return out


def mla_fa_decode_partials(q, q_type, kv, kv_type, scale, out, *, mask=None, kv_idx=None,
                           kv_idx_count=None, n_split=0, workspace=None, stream=None):
    _check(lib().mla_fa_decode_partials(*_decode_args(q, q_type, kv, kv_type, scale, out, mask, kv_idx,
                                                      kv_idx_count, n_split, workspace, stream)),
           "mla_fa_decode_partials")


def mla_fa_merge_partials(n_rows, n_head, n_split, out, workspace, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_fa_merge_partials(n_rows, n_head, n_split, _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "mla_fa_merge_partials")


def mla_fa_prefill(q, q_type, kv, kv_type, scale, out, *, causal=True, mask=None, n_split=0,
                   workspace=None, stream=None):
    """q [n_tok][n_head][576], kv [n_kv][row] (or [1][n_kv][row]), out fp32
    [n_tok][n_head][512]; mask [n_tok][>=n_kv] f16 bits."""
    n_tok, n_head = q.shape[-3], q.shape[-2]
    n_kv = kv.shape[-2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_fa_prefill(_ptr(q), q_type, _ptr(kv), kv_type, _row_stride_bytes(kv), n_tok,
                                n_head, n_kv, 1 if causal else 0, _ptr(mask),
                                0 if mask is None else mask.stride(-2), float(scale), _ptr(out),
                                n_split, _ptr(workspace), ws_bytes, _stream(stream)),
           "mla_fa_prefill")
    return out


def mla_fa_attend(q, q_type, kv, kv_type, scale, out, *, kv_len=None, causal=False, mask=None,
                  kv_idx=None, kv_idx_count=None, alibi=None, sinks=None, softcap=0.0, n_split=0,
                  workspace=None, stream=None):
    """q [n_seq][n_tok][n_head][576], kv [n_seq][n_kv][row] (n_kv = capacity), out fp32
    [n_seq][n_tok][n_head][512]; kv_len int32 [n_seq]; mask [n_seq][n_tok][>=n_kv] f16
    bits; kv_idx int32 [n_seq][n_tok][>=n_kv] + kv_idx_count int32 [n_seq][n_tok] for the
    sparse path; alibi / sinks fp32 [n_head]; softcap 0 = off."""
    n_seq, n_tok, n_head = q.shape[0], q.shape[1], q.shape[2]
    n_kv = kv.shape[-2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    mseq = 0 if mask is None else mask.stride(0)
    mtok = 0 if mask is None else mask.stride(1)
    iseq = 0 if kv_idx is None else kv_idx.stride(0)
    itok = 0 if kv_idx is None else kv_idx.stride(1)
    _check(lib().mla_fa_attend(_ptr(q), q_type, _ptr(kv), kv_type, _row_stride_bytes(kv),
                               _seq_stride_bytes(kv, n_seq), n_seq, n_tok, n_head, n_kv, _ptr(kv_len),
                               1 if causal else 0, _ptr(mask), mseq, mtok, _ptr(kv_idx), _ptr(kv_idx_count),
                               iseq, itok, _ptr(alibi), _ptr(sinks), float(softcap), float(scale), _ptr(out),
                               n_split, _ptr(workspace), ws_bytes, _stream(stream)),
           "mla_fa_attend")
    return out


def mla_fa_prefill_mha(q, q_type, k, v, kv_type, scale, out, *, causal=True, mask=None, stream=None):
    """q [n_tok][n_head][192], k [n_kv][n_head][192], v [n_kv][n_head][128] (16-bit bits;
    k and v rows may be strided), out fp32 [n_tok][n_head][128]; mask [n_tok][>=n_kv] f16
    bits, 16-byte aligned, with a row stride that is a multiple of 8."""
    n_tok, n_head = q.shape[0], q.shape[1]
    n_kv = k.shape[0]
    _check(lib().mla_fa_prefill_mha(_ptr(q), q_type, _ptr(k), _ptr(v), kv_type, k.stride(0) * k.element_size(),
                                    v.stride(0) * v.element_size(), n_tok, n_head, n_kv, 1 if causal else 0,
                                    _ptr(mask), 0 if mask is None else mask.stride(0), float(scale), _ptr(out),
                                    _stream(stream)),
           "mla_fa_prefill_mha")
    return out


def mla_fa_absorbed_workspace_size(n_rows: int, n_head: int, n_kv: int, kv_type: int, n_split: int = 0) -> int:
    return int(lib().mla_fa_absorbed_workspace_size(n_rows, n_head, n_kv, kv_type, n_split))


def absorbed_workspace_for(n_rows, n_head, n_kv, kv_type, n_split=0, device="cuda"):
    nbytes = mla_fa_absorbed_workspace_size(n_rows, n_head, n_kv, kv_type, n_split)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def mla_fa_absorbed(q_nope, q_pe, q_type, w_uk, w_uv, kv, kv_type, scale, out, *, kv_len=None, causal=False,
                    mask=None, n_split=0, workspace=None, stream=None):
    """q_nope [n_seq][n_tok][n_head][128], q_pe [..][64] (16-bit bits), w_uk [n_head][512][128],
    w_uv [n_head][128][512] (same type), kv [n_seq][n_kv][row], out fp32 [n_seq][n_tok][n_head][128];
    kv_len int32 [n_seq]; mask [n_seq][n_tok][>=n_kv] f16 bits."""
    n_seq, n_tok, n_head = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
    n_kv = kv.shape[-2]
    if workspace is None:
        workspace = absorbed_workspace_for(n_seq * n_tok, n_head, n_kv, kv_type, n_split, device=q_nope.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    mseq = 0 if mask is None else mask.stride(0)
    mtok = 0 if mask is None else mask.stride(1)
    _check(lib().mla_fa_absorbed(_ptr(q_nope), _ptr(q_pe), q_type, _ptr(w_uk), _ptr(w_uv), _ptr(kv), kv_type,
                                 _row_stride_bytes(kv), _seq_stride_bytes(kv, n_seq), n_seq, n_tok, n_head, n_kv,
                                 _ptr(kv_len), 1 if causal else 0, _ptr(mask), mseq, mtok, float(scale), _ptr(out),
                                 n_split, _ptr(workspace), ws_bytes, _stream(stream)),
           "mla_fa_absorbed")
    return out


def fa_mask_compact(mask, idx, count, stream=None):
    """mask [n_rows][n_kv] f16 bits -> idx [n_rows][>=n_kv] int32 (ascending kept
    cells), count [n_rows] int32."""
    n_rows, n_kv = mask.shape
    _check(lib().fa_mask_compact(_ptr(mask), mask.stride(0), n_rows, n_kv, _ptr(idx), idx.stride(0),
                                 _ptr(count), _stream(stream)), "fa_mask_compact")


def fa_mask_compact_workspace_size(n_rows, n_kv):
    return lib().fa_mask_compact_workspace_size(n_rows, n_kv)


def fa_mask_compact_ws(mask, idx, count, workspace, stream=None):
    """fa_mask_compact over many workgroups per row; `workspace` is a device tensor of at
    least fa_mask_compact_workspace_size(n_rows, n_kv) bytes (or None where that is 0)."""
    n_rows, n_kv = mask.shape
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fa_mask_compact_ws(_ptr(mask), mask.stride(0), n_rows, n_kv, _ptr(idx), idx.stride(0),
                                    _ptr(count), _ptr(workspace), wsb, _stream(stream)), "fa_mask_compact_ws")
