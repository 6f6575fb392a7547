"""Qwen3-0.6B decode-attention block on AMD MI355X (gfx950): thin Python binding.

The three calls mirror the C ABI in include/dah.h and only marshal arguments:
they check torch dtypes, shapes, devices and contiguity, then pass raw device
pointers and the current HIP stream to libdah.so.  Every step of the
computation runs in the library's HIP kernels.

    qk_norm_rope_append  nodes attn.qk_norm + attn.rope and the cache store
    paged_decode_gqa     node attn.core (decodeGQA) over the paged cache
    decode_attn_step     both, in order, on one stream
    chunk_attn_step      the same for several new tokens per sequence (causal)
    decoder_layer_step   a whole layer around the block (norms, residuals, SwiGLU MLP)
    qkv_proj, o_proj     nodes attn.qkv_proj and attn.o_proj around them
    linear               the product both use (float32 x, bfloat16 weights)
    linear_ws, o_proj_ws the same with k split over workgroups (a workspace)

(Node names from the "Qwen3-0.6B" Model Spec page, "Compute-graph nodes".)

Cache layout: k_cache / v_cache are [num_pages, 8, 16, 128] tensors of
float32 or bfloat16 (page, KV head, slot, dim); block_table is int32
[B, max_pages_per_seq]; seq_lens is int32 [B] and counts the new token.

q, q_out and o are [B, H, 128] with H = 16 (Qwen3-0.6B, the C calls without
suffix) or another of the family's head counts 32, 40, 64 over the same 8 KV
heads (the *_ex C calls, chosen from q's shape).
"""
from __future__ import annotations

import ctypes

from ._native import DAH_BF16, DAH_F32, DahError, LIB_PATH, check, lib

__all__ = [
    "qk_norm_rope_append", "paged_decode_gqa", "decode_attn_step", "plan_decode",
    "workspace_bytes", "DahError", "LIB_PATH", "NUM_HEADS", "NUM_KV_HEADS", "HEAD_DIM",
    "PAGE_SIZE", "HEAD_COUNTS", "linear", "linear_ws", "linear_kernel", "linear_ws_kernel",
    "linear_workspace_bytes", "qkv_proj", "o_proj", "o_proj_ws", "chunk_attn_step", "rmsnorm",
    "silu_mul", "decoder_layer_step", "layer_workspace_bytes", "LAYER_WEIGHTS",
]

NUM_HEADS = 16
HEAD_COUNTS = (16, 32, 40, 64)  # query heads over 8 KV heads: group sizes 2, 4, 5, 8
NUM_KV_HEADS = 8
HEAD_DIM = 128
PAGE_SIZE = 16


def _torch():
    import torch
    return torch


def _ptr(t) -> int:
    return t.data_ptr()


def _require(t, name, dtype, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _cache_dtype(k_cache, v_cache) -> int:
    torch = _torch()
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must share a dtype")
    if k_cache.dtype == torch.bfloat16:
        return DAH_BF16
    if k_cache.dtype == torch.float32:
        return DAH_F32
    raise TypeError(f"cache dtype must be float32 or bfloat16, got {k_cache.dtype}")


def _check_cache(k_cache, v_cache, block_table, seq_lens, B, device):
    torch = _torch()
    dt = _cache_dtype(k_cache, v_cache)
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM):
        raise ValueError(f"k_cache must be [num_pages, 8, 16, 128], got {tuple(k_cache.shape)}")
    _require(k_cache, "k_cache", k_cache.dtype, device=device)
    _require(v_cache, "v_cache", k_cache.dtype, tuple(k_cache.shape), device)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq]")
    _require(block_table, "block_table", torch.int32, device=device)
    _require(seq_lens, "seq_lens", torch.int32, (B,), device)
    return dt


def _stream(device, stream):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(cache_dtype) -> int:
    """DAH_BF16 / DAH_F32 from "bf16" / "f32" or a torch dtype."""
    if cache_dtype in ("bf16", DAH_BF16):
        return DAH_BF16
    if cache_dtype in ("f32", DAH_F32):
        return DAH_F32
    torch = _torch()
    if cache_dtype == torch.bfloat16:
        return DAH_BF16
    if cache_dtype == torch.float32:
        return DAH_F32
    raise TypeError(f"cache dtype must be bfloat16 or float32, got {cache_dtype}")


def plan_decode(B: int, max_seq_len: int, num_splits: int = 0, num_cus: int | None = None,
                num_heads: int = NUM_HEADS, cache_dtype="bf16") -> dict:
    """How the decode will cut the work (dah_plan_decode_ex): a dict with mode
    ("per_sequence", "split" or "balanced"), splits, pages_per_split,
    workgroups, workspace_bytes and kernel ("valu" or "mfma").  num_cus
    defaults to the current device's compute-unit count; the plan depends on
    the head count and the cache dtype through the kernel they select."""
    from ._native import PLAN_MODES, DecodePlan
    if num_cus is None:
        torch = _torch()
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    p = DecodePlan()
    st = lib().dah_plan_decode_ex(B, num_heads, _dtype_code(cache_dtype), max_seq_len,
                                  num_splits, num_cus, ctypes.byref(p))
    check(st, "dah_plan_decode_ex")
    return {"mode": PLAN_MODES[p.mode], "splits": p.splits, "pages_per_split": p.pages_per_split,
            "workgroups": p.workgroups, "workspace_bytes": int(p.workspace_bytes),
            "kernel": "mfma" if p.kernel == 1 else "valu"}


def workspace_bytes(B: int, max_seq_len: int, num_splits: int = 0,
                    num_cus: int | None = None, num_heads: int = NUM_HEADS,
                    cache_dtype="bf16") -> int:
    """Bytes of device workspace paged_decode_gqa / decode_attn_step need for
    these arguments: the partial results of cut sequences (and, under the
    balanced plan, the batch's page prefix sums); 0 when no sequence is cut.
    The contents need no initialisation.  num_cus: plan for that many compute
    units instead of the current device's."""
    if num_heads != NUM_HEADS or _dtype_code(cache_dtype) != DAH_BF16:
        if num_cus is None:
            return int(lib().dah_workspace_bytes_ex(B, num_heads, _dtype_code(cache_dtype),
                                                    max_seq_len, num_splits))
        return plan_decode(B, max_seq_len, num_splits, num_cus, num_heads,
                           cache_dtype)["workspace_bytes"]
    if num_cus is None:
        return int(lib().dah_workspace_bytes(B, max_seq_len, num_splits))
    return int(lib().dah_workspace_bytes_for(B, max_seq_len, num_splits, num_cus))


def _heads(q) -> int:
    if q.dim() != 3 or q.shape[1] not in HEAD_COUNTS or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [B, H, 128] with H in {HEAD_COUNTS}, got {tuple(q.shape)}")
    return int(q.shape[1])


def _workspace(workspace, B, H, dt, max_seq_len, num_splits, device):
    torch = _torch()
    need = workspace_bytes(B, max_seq_len, num_splits, num_heads=H, cache_dtype=dt)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _require(workspace, "workspace", workspace.dtype, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def qk_norm_rope_append(q, k_new, v_new, q_gain, k_gain, k_cache, v_cache, block_table,
                        seq_lens, *, eps: float = 1e-6, rope_theta: float = 1e6, q_out=None,
                        stream=None):
    """Norm and rotate q and the new k at pos = seq_lens - 1, store k and v
    in the cache.  Returns q_out [B,H,128] float32 (q_out may be q)."""
    torch = _torch()
    B, H = q.shape[0], _heads(q)
    dev = q.device
    _require(q, "q", torch.float32, (B, H, HEAD_DIM))
    _require(k_new, "k_new", torch.float32, (B, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(v_new, "v_new", torch.float32, (B, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(q_gain, "q_gain", torch.float32, (HEAD_DIM,), dev)
    _require(k_gain, "k_gain", torch.float32, (HEAD_DIM,), dev)
    dt = _check_cache(k_cache, v_cache, block_table, seq_lens, B, dev)
    if q_out is None:
        q_out = torch.empty_like(q)
    _require(q_out, "q_out", torch.float32, (B, H, HEAD_DIM), dev)
    head = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(q_gain), _ptr(k_gain), eps, rope_theta,
            _ptr(k_cache), _ptr(v_cache), dt, k_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), B)
    tail = (_ptr(q_out), _stream(dev, stream))
    if H == NUM_HEADS:
        st = lib().qk_norm_rope_append(*head, *tail)
    else:
        st = lib().qk_norm_rope_append_ex(*head, H, *tail)
    check(st, "qk_norm_rope_append")
    return q_out


def paged_decode_gqa(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, *,
                     num_splits: int = 0, o=None, workspace=None, stream=None):
    """decodeGQA over the paged cache.  q is already normed and roped.
    max_seq_len bounds every seq_lens[b] (host value, for the planner).
    Returns o [B,H,128] float32."""
    torch = _torch()
    B, H = q.shape[0], _heads(q)
    dev = q.device
    _require(q, "q", torch.float32, (B, H, HEAD_DIM))
    dt = _check_cache(k_cache, v_cache, block_table, seq_lens, B, dev)
    if o is None:
        o = torch.empty_like(q)
    _require(o, "o", torch.float32, (B, H, HEAD_DIM), dev)
    ws, ws_bytes = _workspace(workspace, B, H, dt, max_seq_len, num_splits, dev)
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), dt, k_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), B)
    tail = (int(max_seq_len), int(num_splits), _ptr(o), None if ws is None else _ptr(ws),
            ws_bytes, _stream(dev, stream))
    if H == NUM_HEADS:
        st = lib().paged_decode_gqa(*head, *tail)
    else:
        st = lib().paged_decode_gqa_ex(*head, H, *tail)
    check(st, "paged_decode_gqa")
    return o


def decode_attn_step(q, k_new, v_new, q_gain, k_gain, k_cache, v_cache, block_table, seq_lens,
                     max_seq_len: int, *, eps: float = 1e-6, rope_theta: float = 1e6,
                     num_splits: int = 0, q_out=None, o=None, workspace=None, stream=None):
    """One decode step of one layer: norm, RoPE, cache append, decodeGQA.
    Returns (q_out, o).  q_out=False skips the q_out store (the C call gets
    NULL) and returns (None, o)."""
    torch = _torch()
    B, H = q.shape[0], _heads(q)
    dev = q.device
    _require(q, "q", torch.float32, (B, H, HEAD_DIM))
    _require(k_new, "k_new", torch.float32, (B, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(v_new, "v_new", torch.float32, (B, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(q_gain, "q_gain", torch.float32, (HEAD_DIM,), dev)
    _require(k_gain, "k_gain", torch.float32, (HEAD_DIM,), dev)
    dt = _check_cache(k_cache, v_cache, block_table, seq_lens, B, dev)
    if q_out is None:
        q_out = torch.empty_like(q)
    if o is None:
        o = torch.empty_like(q)
    if q_out is not False:
        _require(q_out, "q_out", torch.float32, (B, H, HEAD_DIM), dev)
    _require(o, "o", torch.float32, (B, H, HEAD_DIM), dev)
    ws, ws_bytes = _workspace(workspace, B, H, dt, max_seq_len, num_splits, dev)
    head = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(q_gain), _ptr(k_gain), eps, rope_theta,
            _ptr(k_cache), _ptr(v_cache), dt, k_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), B)
    tail = (int(max_seq_len), int(num_splits), None if q_out is False else _ptr(q_out), _ptr(o),
            None if ws is None else _ptr(ws), ws_bytes, _stream(dev, stream))
    if H == NUM_HEADS:
        st = lib().decode_attn_step(*head, *tail)
    else:
        st = lib().decode_attn_step_ex(*head, H, *tail)
    check(st, "decode_attn_step")
    return (None if q_out is False else q_out), o


def decode_attn_step_noalloc(q, k_new, v_new, q_gain, k_gain, k_cache, v_cache, block_table,
                             seq_lens, max_seq_len: int, *, eps: float = 1e-6,
                             rope_theta: float = 1e6, num_splits: int = 0, q_out=None, o=None,
                             stream=None):
    """decode_attn_step through decode_attn_step_noalloc: the split partials
    live in the library's static device scratch (DAH_SCRATCH_BYTES), so the
    C call allocates nothing.  q_out and o must then be given by a caller
    that cannot allocate (here they are allocated when omitted); q_out=False
    passes NULL.  Returns (q_out, o)."""
    torch = _torch()
    B, H = q.shape[0], _heads(q)
    dev = q.device
    _require(q, "q", torch.float32, (B, H, HEAD_DIM))
    _require(k_new, "k_new", torch.float32, (B, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(v_new, "v_new", torch.float32, (B, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(q_gain, "q_gain", torch.float32, (HEAD_DIM,), dev)
    _require(k_gain, "k_gain", torch.float32, (HEAD_DIM,), dev)
    dt = _check_cache(k_cache, v_cache, block_table, seq_lens, B, dev)
    if q_out is None:
        q_out = torch.empty_like(q)
    if o is None:
        o = torch.empty_like(q)
    if q_out is not False:
        _require(q_out, "q_out", torch.float32, (B, H, HEAD_DIM), dev)
    _require(o, "o", torch.float32, (B, H, HEAD_DIM), dev)
    st = lib().decode_attn_step_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(q_gain), _ptr(k_gain), eps, rope_theta,
        _ptr(k_cache), _ptr(v_cache), dt, k_cache.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, H, int(max_seq_len), int(num_splits),
        None if q_out is False else _ptr(q_out), _ptr(o), _stream(dev, stream))
    check(st, "decode_attn_step_noalloc")
    return (None if q_out is False else q_out), o


SCRATCH_BYTES = 16 << 20   # DAH_SCRATCH_BYTES (include/dah.h)


# ---------------------------------------------------------------- projections

def _require_weights(w, name, shape, device):
    torch = _torch()
    _require(w, name, torch.bfloat16, shape, device)


def linear(x, w, *, y=None, stream=None):
    """y [T,N] = x [T,K] . w^T with x float32, w bfloat16 [N,K] (dah_linear)."""
    torch = _torch()
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("linear: x must be [T,K] and w [N,K]")
    T, K = x.shape
    N = w.shape[0]
    _require(x, "x", torch.float32, (T, K))
    _require_weights(w, "w", (N, K), x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.float32, device=x.device)
    _require(y, "y", torch.float32, (T, N), x.device)
    check(lib().dah_linear(_ptr(x), _ptr(w), T, N, K, _ptr(y), _stream(x.device, stream)),
          "dah_linear")
    return y


def linear_kernel(T: int, N: int, K: int) -> int:
    """Which kernel dah_linear launches for a T x N x K product (host only):
    0 split-k, 1..5 the LDS tile shapes, -1 for an invalid shape."""
    return int(lib().dah_linear_kernel(int(T), int(N), int(K)))


def linear_workspace_bytes(T: int, N: int, K: int) -> int:
    """Workspace bytes dah_linear_ws needs for a T x N x K product (0 when it
    does not split k)."""
    return int(lib().dah_linear_workspace_bytes(int(T), int(N), int(K)))


def linear_ws_kernel(T: int, N: int, K: int):
    """(kernel, k slices) dah_linear_ws launches for a T x N x K product
    (host only; kernel ids as linear_kernel)."""
    ks = ctypes.c_int(0)
    kernel = int(lib().dah_linear_ws_kernel(int(T), int(N), int(K), ctypes.byref(ks)))
    return kernel, int(ks.value)


def _linear_workspace(workspace, T, N, K, device):
    torch = _torch()
    need = linear_workspace_bytes(T, N, K)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _require(workspace, "workspace", workspace.dtype, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def linear_ws(x, w, *, residual=None, y=None, workspace=None, stream=None):
    """y [T,N] = x [T,K] . w^T (+ residual [T,N]) with k split over
    workgroups into a workspace (dah_linear_ws); the workspace (uint8, at
    least linear_workspace_bytes) is allocated when not given."""
    torch = _torch()
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("linear_ws: x must be [T,K] and w [N,K]")
    T, K = x.shape
    N = w.shape[0]
    _require(x, "x", torch.float32, (T, K))
    _require_weights(w, "w", (N, K), x.device)
    if residual is not None:
        _require(residual, "residual", torch.float32, (T, N), x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.float32, device=x.device)
    _require(y, "y", torch.float32, (T, N), x.device)
    ws, ws_bytes = _linear_workspace(workspace, T, N, K, x.device)
    check(lib().dah_linear_ws(_ptr(x), _ptr(w), None if residual is None else _ptr(residual), T, N,
                              K, _ptr(y), None if ws is None else _ptr(ws), ws_bytes,
                              _stream(x.device, stream)), "dah_linear_ws")
    return y


def qkv_proj(x, w_qkv, num_heads: int = NUM_HEADS, *, q=None, k=None, v=None, stream=None):
    """attn.qkv_proj: x [T,hidden] float32, w_qkv [H*128 + 2048, hidden] bfloat16
    (q_proj, k_proj, v_proj rows stacked) -> (q [T,H,128], k [T,8,128],
    v [T,8,128]) float32, the layouts decode_attn_step takes."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("qkv_proj: x must be [T,hidden]")
    T, hidden = x.shape
    H = int(num_heads)
    _require(x, "x", torch.float32, (T, hidden))
    _require_weights(w_qkv, "w_qkv", ((H + 2 * NUM_KV_HEADS) * HEAD_DIM, hidden), x.device)
    dev = x.device
    q = torch.empty((T, H, HEAD_DIM), dtype=torch.float32, device=dev) if q is None else q
    k = torch.empty((T, NUM_KV_HEADS, HEAD_DIM), dtype=torch.float32, device=dev) if k is None else k
    v = torch.empty((T, NUM_KV_HEADS, HEAD_DIM), dtype=torch.float32, device=dev) if v is None else v
    _require(q, "q", torch.float32, (T, H, HEAD_DIM), dev)
    _require(k, "k", torch.float32, (T, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(v, "v", torch.float32, (T, NUM_KV_HEADS, HEAD_DIM), dev)
    check(lib().attn_qkv_proj(_ptr(x), _ptr(w_qkv), T, hidden, H, _ptr(q), _ptr(k), _ptr(v),
                              _stream(dev, stream)), "attn_qkv_proj")
    return q, k, v


def o_proj(o, w_o, *, y=None, stream=None):
    """attn.o_proj: o [T,H,128] float32 (heads side by side), w_o [hidden, H*128]
    bfloat16 -> y [T,hidden] float32."""
    torch = _torch()
    if o.dim() != 3:
        raise ValueError("o_proj: o must be [T,H,128]")
    T, H = o.shape[0], _heads(o)
    hidden = w_o.shape[0]
    _require(o, "o", torch.float32, (T, H, HEAD_DIM))
    _require_weights(w_o, "w_o", (hidden, H * HEAD_DIM), o.device)
    if y is None:
        y = torch.empty((T, hidden), dtype=torch.float32, device=o.device)
    _require(y, "y", torch.float32, (T, hidden), o.device)
    check(lib().attn_o_proj(_ptr(o), _ptr(w_o), T, H, hidden, _ptr(y), _stream(o.device, stream)),
          "attn_o_proj")
    return y


def o_proj_ws(o, w_o, *, y=None, workspace=None, stream=None):
    """o_proj with k split over workgroups into a workspace (attn_o_proj_ws;
    linear_workspace_bytes(T, hidden, H*128) bytes, allocated when not
    given)."""
    torch = _torch()
    if o.dim() != 3:
        raise ValueError("o_proj_ws: o must be [T,H,128]")
    T, H = o.shape[0], _heads(o)
    hidden = w_o.shape[0]
    _require(o, "o", torch.float32, (T, H, HEAD_DIM))
    _require_weights(w_o, "w_o", (hidden, H * HEAD_DIM), o.device)
    if y is None:
        y = torch.empty((T, hidden), dtype=torch.float32, device=o.device)
    _require(y, "y", torch.float32, (T, hidden), o.device)
    ws, ws_bytes = _linear_workspace(workspace, T, hidden, H * HEAD_DIM, o.device)
    check(lib().attn_o_proj_ws(_ptr(o), _ptr(w_o), T, H, hidden, _ptr(y),
                               None if ws is None else _ptr(ws), ws_bytes,
                               _stream(o.device, stream)), "attn_o_proj_ws")
    return y


# ---------------------------------------------------------------- chunks

def chunk_attn_step(q, k_new, v_new, q_gain, k_gain, k_cache, v_cache, block_table, seq_lens,
                    cu_tokens, max_chunk: int, max_seq_len: int, *, eps: float = 1e-6,
                    rope_theta: float = 1e6, q_out=None, o=None, stream=None):
    """Several new tokens per sequence (chunk_attn_step): token i of sequence
    b's chunk (rows cu_tokens[b] .. cu_tokens[b+1]-1) sits at position
    seq_lens[b] - n_b + i; norm, RoPE, append, then causal decodeGQA.
    q [N,H,128], k_new/v_new [N,8,128] float32, cu_tokens int32 [B+1];
    bfloat16 or float32 cache.  Returns (q_out, o), both [N,H,128] float32."""
    torch = _torch()
    N, H = q.shape[0], _heads(q)
    B = seq_lens.shape[0]
    dev = q.device
    _require(q, "q", torch.float32, (N, H, HEAD_DIM))
    _require(k_new, "k_new", torch.float32, (N, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(v_new, "v_new", torch.float32, (N, NUM_KV_HEADS, HEAD_DIM), dev)
    _require(q_gain, "q_gain", torch.float32, (HEAD_DIM,), dev)
    _require(k_gain, "k_gain", torch.float32, (HEAD_DIM,), dev)
    _require(cu_tokens, "cu_tokens", torch.int32, (B + 1,), dev)
    dt = _check_cache(k_cache, v_cache, block_table, seq_lens, B, dev)
    q_out = torch.empty_like(q) if q_out is None else q_out
    o = torch.empty_like(q) if o is None else o
    _require(q_out, "q_out", torch.float32, (N, H, HEAD_DIM), dev)
    _require(o, "o", torch.float32, (N, H, HEAD_DIM), dev)
    st = lib().chunk_attn_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(q_gain), _ptr(k_gain), eps, rope_theta,
        _ptr(k_cache), _ptr(v_cache), dt, k_cache.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), _ptr(cu_tokens), B, N, int(max_chunk),
        int(max_seq_len), H, _ptr(q_out), _ptr(o), _stream(dev, stream))
    check(st, "chunk_attn_step")
    return q_out, o


# ---------------------------------------------------------------- decoder layer

def rmsnorm(x, w, *, eps: float = 1e-6, y=None, stream=None):
    """Rows of a hidden-size RMSNorm (dah_rmsnorm): x [T,H] float32, w [H]."""
    torch = _torch()
    T, width = x.shape
    _require(x, "x", torch.float32, (T, width))
    _require(w, "w", torch.float32, (width,), x.device)
    y = torch.empty_like(x) if y is None else y
    _require(y, "y", torch.float32, (T, width), x.device)
    check(lib().dah_rmsnorm(_ptr(x), _ptr(w), eps, T, width, _ptr(y), _stream(x.device, stream)),
          "dah_rmsnorm")
    return y


def silu_mul(gate_up, *, act=None, stream=None):
    """mlp.act (dah_silu_mul): gate_up [T, 2I] float32 -> [T, I]."""
    torch = _torch()
    T, two_i = gate_up.shape
    _require(gate_up, "gate_up", torch.float32, (T, two_i))
    act = torch.empty((T, two_i // 2), dtype=torch.float32, device=gate_up.device) \
        if act is None else act
    _require(act, "act", torch.float32, (T, two_i // 2), gate_up.device)
    check(lib().dah_silu_mul(_ptr(gate_up), T, two_i // 2, _ptr(act),
                             _stream(gate_up.device, stream)), "dah_silu_mul")
    return act


def rmsnorm_swiglu(x, x_gain, w_gate_up, *, eps: float = 1e-6, act=None, stream=None):
    """post_attn_norm + gate_up + mlp.act in one launch (dah_rmsnorm_swiglu):
    x [T,K] float32, x_gain [K] float32 or None (no norm), w_gate_up
    [2I,K] bfloat16 (gate rows, then up rows) -> act [T,I] float32."""
    torch = _torch()
    T, K = x.shape
    two_i = w_gate_up.shape[0]
    _require(x, "x", torch.float32, (T, K))
    _require_weights(w_gate_up, "w_gate_up", (two_i, K), x.device)
    if x_gain is not None:
        _require(x_gain, "x_gain", torch.float32, (K,), x.device)
    act = torch.empty((T, two_i // 2), dtype=torch.float32, device=x.device) \
        if act is None else act
    _require(act, "act", torch.float32, (T, two_i // 2), x.device)
    check(lib().dah_rmsnorm_swiglu(_ptr(x), None if x_gain is None else _ptr(x_gain), eps,
                                   _ptr(w_gate_up), T, two_i // 2, K, _ptr(act),
                                   _stream(x.device, stream)), "dah_rmsnorm_swiglu")
    return act


LAYER_WEIGHTS = ("w_in", "w_qkv", "q_gain", "k_gain", "w_o", "w_post", "w_gate_up", "w_down")


def layer_workspace_bytes(B: int, hidden: int, inter: int, max_seq_len: int, num_splits: int = 0,
                          num_heads: int = NUM_HEADS, cache_dtype="bf16") -> int:
    return int(lib().dah_layer_workspace_bytes(B, hidden, inter, num_heads,
                                               _dtype_code(cache_dtype), max_seq_len, num_splits))


def decoder_layer_step(x, weights: dict, k_cache, v_cache, block_table, seq_lens,
                       max_seq_len: int, *, eps: float = 1e-6, rope_theta: float = 1e6,
                       num_splits: int = 0, y=None, workspace=None, stream=None):
    """One decoder layer's decode step (decoder_layer_step): x [B, hidden]
    float32 (one new token per sequence) -> y [B, hidden].  weights holds
    the tensors named in LAYER_WEIGHTS (bf16 matrices, float32 gains)."""
    import ctypes as _ct
    from ._native import LayerWeights
    torch = _torch()
    B, hidden = x.shape
    dev = x.device
    _require(x, "x", torch.float32, (B, hidden))
    w_o, w_down = weights["w_o"], weights["w_down"]
    H = w_o.shape[1] // HEAD_DIM
    inter = w_down.shape[1]
    if H not in HEAD_COUNTS:
        raise ValueError(f"w_o must be [hidden, H*128] with H in {HEAD_COUNTS}")
    shapes = {"w_in": (hidden,), "w_qkv": ((H + 2 * NUM_KV_HEADS) * HEAD_DIM, hidden),
              "q_gain": (HEAD_DIM,), "k_gain": (HEAD_DIM,), "w_o": (hidden, H * HEAD_DIM),
              "w_post": (hidden,), "w_gate_up": (2 * inter, hidden), "w_down": (hidden, inter)}
    for name in LAYER_WEIGHTS:
        dtype = torch.float32 if shapes[name] == (hidden,) or name in ("q_gain", "k_gain") \
            else torch.bfloat16
        _require(weights[name], name, dtype, shapes[name], dev)
    dt = _check_cache(k_cache, v_cache, block_table, seq_lens, B, dev)
    y = torch.empty_like(x) if y is None else y
    _require(y, "y", torch.float32, (B, hidden), dev)
    need = layer_workspace_bytes(B, hidden, inter, max_seq_len, num_splits, H, k_cache.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    lw = LayerWeights(*[_ptr(weights[n]) for n in LAYER_WEIGHTS])
    st = lib().decoder_layer_step(
        _ptr(x), _ct.byref(lw), hidden, inter, H, eps, rope_theta, _ptr(k_cache), _ptr(v_cache),
        dt, k_cache.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B,
        int(max_seq_len), int(num_splits), _ptr(y), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev, stream))
    check(st, "decoder_layer_step")
    return y
