"""Plain CPU float64 oracle for one whole decoder layer's decode step.

TEST INFRASTRUCTURE ONLY, like the other oracle modules: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it,
and it imports nothing from the library.

The layer, node by node (the "Qwen3-0.6B" Model Spec page, "Compute-graph
nodes", per-layer rows, in order):

    h   = input_norm(x)                 rmsnorm over H = 1024, eps 1e-6
    q, k, v = attn.qkv_proj(h)          (oracle.projections)
    o   = attn.qk_norm, attn.rope, append, attn.core   (oracle.decode_attention)
    x1  = attn_residual: x + attn.o_proj(o)
    h2  = post_attn_norm(x1)            rmsnorm over H, eps 1e-6
    gu  = mlp.gate_up(h2)               linear K = 1024, N = 6144
    a   = mlp.act: silu(gu[:, i]) * gu[:, 3072 + i],  i < 3072
    y   = mlp_residual: x1 + mlp.down(a)   linear K = 3072, N = 1024

Weights are bfloat16 (the checkpoints' dtype), norm gains float32, the
residual stream float32; everything is evaluated in float64 from the exact
stored values.  silu(z) = z / (1 + exp(-z)).
"""
from __future__ import annotations

import numpy as np

from oracle.decode_attention import RMS_EPS, ROPE_THETA, decode_step
from oracle.projections import linear, o_proj, qkv_proj

INTERMEDIATE = 3072   # Qwen3-0.6B (Model Spec page: mlp.act I = 3072, gate_up N = 6144)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """y[t,i] = x[t,i] / sqrt(sum_j x[t,j]^2 / H + eps) * w[i] over the last axis
    (the rmsnorm rows input_norm, post_attn_norm, final_norm)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    H = x.shape[-1]
    ms = np.sum(x * x, axis=-1, keepdims=True) / H
    return x / np.sqrt(ms + eps) * w


def silu_mul(gate_up: np.ndarray) -> np.ndarray:
    """mlp.act: y[t,i] = silu(gate_up[t,i]) * gate_up[t, I + i], I = half the width."""
    g = np.asarray(gate_up, dtype=np.float64)
    inter = g.shape[-1] // 2
    gate, up = g[..., :inter], g[..., inter:]
    return gate / (1.0 + np.exp(-gate)) * up


def decoder_layer(x, weights: dict, k_pool, v_pool, block_table, seq_lens, cache_dtype: str,
                  num_heads: int = 16, eps: float = RMS_EPS, theta: float = ROPE_THETA,
                  batch_indices=None):
    """One decode step of one decoder layer for the selected sequences
    (token t of x is sequence t's new token).  weights: w_in (float32
    [hidden]), w_qkv, q_gain, k_gain, w_o, w_post, w_gate_up ([2I, hidden]),
    w_down ([hidden, I]); the matrices as bfloat16 bit patterns.  Returns a
    dict of the intermediates (h, q, k, v, q_out, o, x1, h2, gu, act) and
    the output y, all float64, over the selected tokens."""
    idx = range(np.asarray(x).shape[0]) if batch_indices is None else list(batch_indices)
    x = np.asarray(x, dtype=np.float64)[list(idx)]
    h = rmsnorm(x, weights["w_in"], eps)
    q, k, v = qkv_proj(h, weights["w_qkv"], num_heads)
    step = decode_step(q, k, v, weights["q_gain"], weights["k_gain"], k_pool, v_pool,
                       np.asarray(block_table)[list(idx)], np.asarray(seq_lens)[list(idx)],
                       cache_dtype, eps=eps, theta=theta)
    x1 = x + o_proj(step["o"], weights["w_o"])
    h2 = rmsnorm(x1, weights["w_post"], eps)
    gu = linear(h2, weights["w_gate_up"])
    act = silu_mul(gu)
    y = x1 + linear(act, weights["w_down"])
    out = dict(step)
    out.update(h=h, q=q, k=k, v=v, x1=x1, h2=h2, gu=gu, act=act, y=y)
    return out
