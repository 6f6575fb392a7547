"""Pins of the projection oracle (oracle/projections.py) against closed forms,
exact selections and a correctly rounded brute force -- none re-types the
matrix product it checks.

Nodes: attn.qkv_proj and attn.o_proj, `linear` rows of the "Qwen3-0.6B"
Model Spec page ("Compute-graph nodes"): y[t,n] = sum_k x[t,k] w[n,k].
"""
import math

import numpy as np
import pytest

from oracle import decode_attention as O
from oracle import projections as P


def _bf16_bits(x):
    """Exact bf16 bit patterns of values that are bf16-representable."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "test values must be exact in bf16"
    return (b >> 16).astype(np.uint16)


def _rand_bf16(rng, shape, scale=1.0):
    return O.round_to_bf16(rng.standard_normal(shape) * scale)


def test_identity_input_reads_out_the_weights():
    # x = I (T = K): y[t, n] = w[n, t], i.e. the widened weights transposed.
    rng = np.random.default_rng(1)
    w = _rand_bf16(rng, (24, 16))
    bits = _bf16_bits(w)
    y = P.linear(np.eye(16), bits)
    assert np.array_equal(y, w.T)
    assert np.array_equal(y, O.bf16_bits_to_f64(bits).T)


def test_one_hot_weights_select_input_columns():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 32)).astype(np.float32)
    perm = rng.permutation(32)
    w = np.zeros((32, 32))
    w[np.arange(32), perm] = 1.0
    y = P.linear(x, _bf16_bits(w))
    assert np.array_equal(y, x[:, perm].astype(np.float64))


def test_constant_operands_closed_form():
    # every x = 0.75, every w = -1.5 (exact in bf16): y = K * 0.75 * -1.5 exactly
    for K in (1, 64, 1024, 2048):
        y = P.linear(np.full((3, K), 0.75, np.float32), _bf16_bits(np.full((7, K), -1.5)))
        assert np.all(y == K * 0.75 * -1.5)


def test_correctly_rounded_brute_force():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 40)).astype(np.float32)
    w = _rand_bf16(rng, (6, 40))
    y = P.linear(x, _bf16_bits(w))
    for t in range(4):
        for n in range(6):
            exact = math.fsum(float(x[t, k]) * float(w[n, k]) for k in range(40))
            assert abs(y[t, n] - exact) <= 1e-14 * max(1.0, sum(abs(float(x[t, k]) * float(w[n, k]))
                                                                for k in range(40)))


def test_float_weights_are_taken_as_values():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 8))
    w = rng.standard_normal((3, 8)).astype(np.float32)
    assert np.allclose(P.linear(x, w, "f32"), P.linear(x, _bf16_bits(O.round_to_bf16(w))), atol=0.1)
    assert np.array_equal(P.linear(np.eye(8), w, "f32"), w.T.astype(np.float64))


def test_contraction_mismatch_rejected():
    with pytest.raises(ValueError):
        P.linear(np.zeros((2, 8)), np.zeros((3, 9), np.uint16))


@pytest.mark.parametrize("H", [16, 32, 40, 64])
def test_qkv_split_order_q_then_k_then_v(H):
    # Rows of w_qkv that are one-hot on distinct input coordinates tag every
    # output column, so the split positions and reshapes are checked exactly.
    nq, nkv = H * 128, 8 * 128
    N = nq + 2 * nkv
    hidden = N  # big enough for one distinct input coordinate per output
    x = np.arange(1, hidden + 1, dtype=np.float64)[None, :] / 4.0   # exact small values
    w = np.zeros((N, hidden))
    w[np.arange(N), np.arange(N)] = 1.0
    q, k, v = P.qkv_proj(x, _bf16_bits(w), num_heads=H)
    assert q.shape == (1, H, 128) and k.shape == (1, 8, 128) and v.shape == (1, 8, 128)
    col = (x[0] * 4.0 - 1).astype(np.int64)           # output column n carries value (n+1)/4
    assert np.array_equal(q[0].ravel() * 4 - 1, col[:nq])
    assert np.array_equal(k[0].ravel() * 4 - 1, col[nq:nq + nkv])
    assert np.array_equal(v[0].ravel() * 4 - 1, col[nq + nkv:])
    # q head h, dim d is output column h*128 + d
    assert q[0, 3, 5] * 4 - 1 == 3 * 128 + 5


def test_qkv_rejects_wrong_width():
    with pytest.raises(ValueError):
        P.qkv_proj(np.zeros((1, 8)), np.zeros((4000, 8), np.uint16))


@pytest.mark.parametrize("H", [16, 64])
def test_o_proj_reads_heads_side_by_side(H):
    # o one-hot at (head h, dim d): y = column h*128 + d of w_o
    rng = np.random.default_rng(5)
    w_o = _rand_bf16(rng, (32, H * 128))
    bits = _bf16_bits(w_o)
    for h, d in [(0, 0), (1, 0), (H - 1, 127), (H // 2, 77)]:
        o = np.zeros((1, H, 128))
        o[0, h, d] = 1.0
        assert np.array_equal(P.o_proj(o, bits)[0], w_o[:, h * 128 + d])


def test_attention_block_single_position_closed_form():
    """One cached position (the new token): o[h] = v_new[h // 2] exactly, so
    y[t] = sum_h W_o[:, h-block] v[t, h // 2] with v = the v rows of w_qkv
    applied to x; checked through a one-hot v block that makes v = x[:1024]."""
    rng = np.random.default_rng(6)
    hidden, H = 1024, 16
    nq, nkv = H * 128, 8 * 128
    w_qkv = np.zeros((nq + 2 * nkv, hidden))
    w_qkv[:nq] = _rand_bf16(rng, (nq, hidden), 0.03)
    w_qkv[nq:nq + nkv] = _rand_bf16(rng, (nkv, hidden), 0.03)
    w_qkv[nq + nkv + np.arange(nkv), np.arange(nkv)] = 1.0     # v = x[:, :1024]
    w_o = _rand_bf16(rng, (hidden, nq), 0.03)
    x = O.round_to_bf16(rng.standard_normal((2, hidden))).astype(np.float32)  # exact in the bf16 cache
    pools = np.zeros((4, 8, 16, 128), np.float32)
    table = np.array([[0], [1]], np.int32)
    lens = np.array([1, 1])
    res = P.attention_block(x, _bf16_bits(w_qkv), _bf16_bits(w_o), np.ones(128), np.ones(128),
                            pools, pools, table, lens, "f32")
    v = x[:, :nkv].astype(np.float64).reshape(2, 8, 128)
    assert np.array_equal(res["v"], v)
    assert np.array_equal(res["o"], np.repeat(v, 2, axis=1))       # head h reads KV head h // 2
    want = np.stack([sum(w_o[:, h * 128:(h + 1) * 128] @ v[t, h // 2] for h in range(H))
                     for t in range(2)])
    assert np.allclose(res["y"], want, rtol=1e-13, atol=1e-13)
