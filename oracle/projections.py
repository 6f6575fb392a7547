"""Plain CPU float64 oracle for the linear layers on either side of the
decode-attention block.

TEST INFRASTRUCTURE ONLY, like ``oracle.decode_attention``: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it,
and it imports nothing from the library.

Nodes (the "Qwen3-0.6B" Model Spec page, "Compute-graph nodes" and "Tensors
of the main nodes"):

  * ``attn.qkv_proj``  linear, y[t,n] = sum_k x[t,k] w[n,k], K = 1024,
    N = 4096: x [T,1024] -> y [T,4096]
  * ``attn.o_proj``    linear, same formula, K = 2048, N = 1024:
    the attention output flattened [T,16*128] -> [T,1024]

Readings (each is listed with its reason in the design notes):

  * The fused projection's 4096 outputs are q (16 heads x 128), then k
    (8 x 128), then v (8 x 128): the nnterp qwen3 page's module listing has
    q_proj (1024 -> 2048), k_proj (1024 -> 1024) and v_proj (1024 -> 1024),
    and the Model Spec page's tensor table gives q [T,16,128] and k [T,8,128].
    For the family's larger members the q block is H x 128 wide.
  * o_proj takes the head outputs side by side, [T, H*128] with head h at
    columns h*128 .. h*128+127 (nnterp page: attention_premix holds every
    head's output side by side, as the output projection takes it).
  * Weights are bfloat16, the checkpoints' dtype (nnterp page, configuration
    table: dtype bfloat16); activations are float32.  Both widen exactly to
    float64 here.

Every function is the plain definition evaluated in float64 (a matrix
product is the one library primitive used); no blocking, no splitting.
"""
from __future__ import annotations

import numpy as np

from oracle.decode_attention import (HEAD_DIM, NUM_KV_HEADS, RMS_EPS, ROPE_THETA,
                                     bf16_bits_to_f64, decode_step)


def weights_to_f64(w: np.ndarray, w_dtype: str) -> np.ndarray:
    """Weights as float64: bfloat16 bit patterns (uint16) or float32/float64 values."""
    if w_dtype == "bf16":
        return bf16_bits_to_f64(np.asarray(w, dtype=np.uint16))
    return np.asarray(w, dtype=np.float64)


def linear(x: np.ndarray, w: np.ndarray, w_dtype: str = "bf16") -> np.ndarray:
    """y[t,n] = sum_k x[t,k] * w[n,k]  (Model Spec page, the `linear` rows).

    x [T,K] (any float dtype), w [N,K] -> y [T,N] in float64."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = weights_to_f64(w, w_dtype)
    if x64.ndim != 2 or w64.ndim != 2 or x64.shape[1] != w64.shape[1]:
        raise ValueError(f"linear: x {x64.shape} and w {w64.shape} do not contract over K")
    return x64 @ w64.T


def qkv_proj(x: np.ndarray, w_qkv: np.ndarray, num_heads: int = 16, w_dtype: str = "bf16"):
    """attn.qkv_proj and the split of its output: x [T,hidden] ->
    (q [T,H,128], k [T,8,128], v [T,8,128]) in float64."""
    y = linear(x, w_qkv, w_dtype)
    nq, nkv = num_heads * HEAD_DIM, NUM_KV_HEADS * HEAD_DIM
    if y.shape[1] != nq + 2 * nkv:
        raise ValueError(f"qkv_proj: {y.shape[1]} outputs, expected {nq + 2 * nkv}")
    T = y.shape[0]
    q = y[:, :nq].reshape(T, num_heads, HEAD_DIM)
    k = y[:, nq:nq + nkv].reshape(T, NUM_KV_HEADS, HEAD_DIM)
    v = y[:, nq + nkv:].reshape(T, NUM_KV_HEADS, HEAD_DIM)
    return q, k, v


def o_proj(o: np.ndarray, w_o: np.ndarray, w_dtype: str = "bf16") -> np.ndarray:
    """attn.o_proj: o [T,H,128] (or [T,H*128]) -> y [T,hidden] in float64."""
    o64 = np.asarray(o, dtype=np.float64)
    return linear(o64.reshape(o64.shape[0], -1), w_o, w_dtype)


def attention_block(x, w_qkv, w_o, q_gain, k_gain, k_pool, v_pool, block_table, seq_lens,
                    cache_dtype: str, num_heads: int = 16, eps: float = RMS_EPS,
                    theta: float = ROPE_THETA, batch_indices=None):
    """x -> qkv_proj -> (qk_norm, rope, append, decodeGQA) -> o_proj, for the
    selected sequences (token t of x is sequence t's new token).

    The projections' outputs enter the decode step exactly (float64); a
    device that keeps them in float32 differs from this by their rounding.
    Returns the decode step's dict plus q, k, v (the projections) and y."""
    idx = range(np.asarray(x).shape[0]) if batch_indices is None else list(batch_indices)
    xs = np.asarray(x)[list(idx)]
    q, k, v = qkv_proj(xs, w_qkv, num_heads)
    sel_lens = np.asarray(seq_lens)[list(idx)]
    sel_table = np.asarray(block_table)[list(idx)]
    step = decode_step(q, k, v, q_gain, k_gain, k_pool, v_pool, sel_table, sel_lens,
                       cache_dtype, eps=eps, theta=theta)
    step.update(q=q, k=k, v=v, y=o_proj(step["o"], w_o))
    return step
