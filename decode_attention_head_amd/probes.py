"""Tensor-level wrappers of the benchmark's memory probes (include/dah_probe.h).

The byte counts are taken from the tensors themselves, so a probe can never be
asked to touch more memory than the tensors own.
"""
from __future__ import annotations

import ctypes

from ._native import check, probe_lib


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(t, stream):
    import torch
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def probe_copy(src, dst, stream=None) -> int:
    """dst <- src with 16-byte vector loads/stores; both contiguous, same byte
    size (a positive multiple of 16).  Returns the bytes copied."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("probe_copy needs contiguous GPU tensors")
    n = _nbytes(src)
    if n != _nbytes(dst):
        raise ValueError(f"probe_copy: src has {n} bytes, dst {_nbytes(dst)}")
    check(probe_lib().dah_probe_copy(src.data_ptr(), dst.data_ptr(), n, _stream(src, stream)),
          "dah_probe_copy")
    return n


def probe_read(src, sink, blocks: int, stream=None) -> int:
    """Stream all of src through non-temporal 16-byte loads with `blocks`
    workgroups; sink is an int32 tensor with at least `blocks` elements.
    Returns the bytes read."""
    import torch
    if not (src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32):
        raise ValueError("probe_read needs a contiguous GPU tensor and an int32 GPU sink")
    if not 1 <= blocks <= min(sink.numel(), 65536):
        raise ValueError(f"blocks must be in [1, min(sink size, 65536)], got {blocks}")
    n = _nbytes(src)
    check(probe_lib().dah_probe_read(src.data_ptr(), n, sink.data_ptr(), blocks,
                                     _stream(src, stream)), "dah_probe_read")
    return n
