"""ctypes binding of libkvarn_probe.so: a plain streaming-read kernel, the
measurement aid whose timing gives the achievable read bandwidth reported
beside the HBM peak.  It does no KVarN computation and is not part of the
KVarN C ABI."""
from __future__ import annotations

import ctypes
import os

import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvarn_probe.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build it with `python -m kv_cache_quantization_seal_amd.build`")
        L = ctypes.CDLL(_PATH)
        L.kvarn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.kvarn_probe_read.restype = ctypes.c_int
        _lib = L
    return _lib


def read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream every byte of `buf` (device, contiguous, 16-byte aligned);
    `sink` is a device tensor of at least 4 bytes that is, in practice, never
    written."""
    if not (buf.is_cuda and sink.is_cuda and buf.is_contiguous()):
        raise ValueError("buf and sink must be contiguous device tensors")
    if stream is None:
        stream = torch.cuda.current_stream()
    st = lib().kvarn_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                int(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"kvarn_probe_read failed with status {st}")
