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


def probe_paged_read(k_cache, v_cache, block_table, seq_lens, max_seq_len: int, sink,
                     stream=None) -> None:
    """Read the batch's cached pages through the block table in the decode
    kernel's arrangement (include/dah_probe.h) without its arithmetic.  Pools
    [num_pages, 8, 16, 128] (float32 or bfloat16), int32 block_table [B, P] and
    seq_lens [B] on the GPU; sink an int32 GPU tensor of at least B * 8
    elements.  Only launches (no synchronisation), so that it can be timed
    back to back."""
    import torch
    if not all(t.is_cuda and t.is_contiguous() for t in (k_cache, v_cache, block_table, seq_lens,
                                                          sink)):
        raise ValueError("probe_paged_read needs contiguous GPU tensors")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or \
            k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (8, 16, 128):
        raise ValueError("probe_paged_read: pools of shape [num_pages, 8, 16, 128] expected")
    if k_cache.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("probe_paged_read: float32 or bfloat16 pools")
    B = block_table.shape[0]
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or \
            seq_lens.shape != (B,) or sink.dtype != torch.int32 or sink.numel() < 8 * B:
        raise ValueError("probe_paged_read: int32 block_table [B, P], seq_lens [B], sink >= 8 B")
    dtype = 1 if k_cache.dtype == torch.bfloat16 else 0
    check(probe_lib().dah_probe_paged_read(
        k_cache.data_ptr(), v_cache.data_ptr(), dtype, k_cache.shape[0], block_table.data_ptr(),
        block_table.shape[1], seq_lens.data_ptr(), B, int(max_seq_len), sink.data_ptr(),
        _stream(k_cache, stream)), "dah_probe_paged_read")
