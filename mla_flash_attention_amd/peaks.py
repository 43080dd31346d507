"""ctypes binding of libmlapeaks (include/mla_peaks.h): achievable-peak micro-benchmarks.

Measurement support for benchmarks, not part of the attention path.  Argument
marshalling only: device tensors are passed as pointers, the current torch stream as
the hipStream_t; the caller times the launches.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmlapeaks.so")
EXPORTS = ("mla_peak_hbm_read", "mla_peak_mfma_bf16", "mla_peak_lds_read")
THREADS = 256                     # threads per workgroup of every peak kernel
MFMA_FLOPS = 16 * 16 * 32 * 2     # one v_mfma_f32_16x16x32_bf16
LDS_STEP_BYTES = 8192             # bytes one wave reads per LDS step

_LIB = None
_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmlapeaks.so not built ({LIB_PATH}); run mla_flash_attention_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.mla_peak_hbm_read.restype = _i
        L.mla_peak_hbm_read.argtypes = [_p, _sz, _p, _i, _p]
        L.mla_peak_mfma_bf16.restype = _i
        L.mla_peak_mfma_bf16.argtypes = [_i, _f, _p, _i, _p]
        L.mla_peak_lds_read.restype = _i
        L.mla_peak_lds_read.argtypes = [_i, _i, _p, _i, _p]
        _LIB = L
    return _LIB


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{where} failed (status {rc})")


def hbm_read(buf: torch.Tensor, sink: torch.Tensor, n_wg: int) -> None:
    """Read every byte of `buf` once; sink: int32 [n_wg] (per-workgroup XOR)."""
    assert buf.is_cuda and buf.is_contiguous() and sink.dtype == torch.int32 and sink.numel() >= n_wg
    _check(lib().mla_peak_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), n_wg,
                                   _stream()), "mla_peak_hbm_read")


def mfma_bf16(iters: int, b_val: float, sink: torch.Tensor, n_wg: int) -> None:
    """n_wg * 4 waves x iters x 8 dense bf16 MFMAs; sink: float32 [n_wg * 256]."""
    assert sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= n_wg * THREADS
    _check(lib().mla_peak_mfma_bf16(iters, b_val, sink.data_ptr(), n_wg, _stream()), "mla_peak_mfma_bf16")


def lds_read(iters: int, transpose: bool, sink: torch.Tensor, n_wg: int) -> None:
    """n_wg * 4 waves x iters x 8 KiB of LDS reads; sink: int32 [n_wg]."""
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= n_wg
    _check(lib().mla_peak_lds_read(iters, int(bool(transpose)), sink.data_ptr(), n_wg, _stream()),
           "mla_peak_lds_read")
