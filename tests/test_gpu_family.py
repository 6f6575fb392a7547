"""GPU parity for the Qwen3 family's other group sizes: 32, 40 and 64 query
heads over the same 8 KV heads of 128 dims (nnterp qwen3 page, "Grouped-query
attention, with 128-wide heads on every size"), and RoPE base 5e6 (the
4B-2507 pair, "What loads as this family").  The calls go through the
*_ex entry points of the C ABI, chosen by the binding from q's shape.

Gates as for the 16-head path: 1e-5 max abs for the float32 cache, 2e-2 for
the bfloat16 cache, relative-to-max <= 1e-4, and (full-size cases) an error
under 1% of the distance to uniform attention.  With a bfloat16 cache and 4
or more query heads per KV head the decode runs on the matrix cores (query
and weights as sums of bfloat16 terms), so the bfloat16 cases here are that
kernel's parity tests.
"""
import dataclasses

import numpy as np
import pytest

from dah_testlib import (build_layer, check_rounded, cuda_available, distance_to_uniform, gates,
                         host_snapshot, oracle_decode, oracle_step, read_slots)
from inputs import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]

HEADS = [32, 40, 64]


def _dah():
    import decode_attention_head_amd as dah
    return dah


def _print(*a):
    print(*a, flush=True)


def _with_heads(name, H, theta=W.ROPE_THETA, **kw):
    return dataclasses.replace(W.WORKLOADS[name], num_heads=H, rope_theta=theta, **kw)


TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("theta", [1e6, 5e6])
@pytest.mark.parametrize("num_splits", [0, 1, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_step_every_element(H, theta, num_splits, dtype):
    """Every output of a ragged batch (1 position, a full page, a page plus
    one, longer ragged tails) against the oracle, in the three launch shapes
    (automatic plan, one workgroup per sequence, three splits)."""
    import torch
    dah = _dah()
    w = _with_heads("ragged_f32_b6", H, theta, cache_dtype=dtype)
    _print(f"[family step] {dtype} H={H} theta={theta:g} num_splits={num_splits}")
    t, seq_lens, table, _ = build_layer(w)
    everything = list(range(w.batch))
    snap = host_snapshot(t, seq_lens, table, everything)
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    int(seq_lens.max()), rope_theta=theta,
                                    num_splits=num_splits)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (w.batch, H, 128)
    ref = oracle_step(snap, dtype, theta=theta)
    e_q = float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"])))
    assert e_q <= 1e-5, f"q_out max abs err {e_q:.3g}"
    k_slot, v_slot = read_slots(t, seq_lens, table, everything)
    if dtype == "f32":
        assert np.max(np.abs(k_slot - ref["k_slot"])) <= 1e-5
    else:
        from oracle import decode_attention as O
        _, k_exact = O.norm_rope(snap["q"], snap["k_new"], snap["q_gain"], snap["k_gain"],
                                 snap["seq_lens"], theta=theta)
        check_rounded(k_slot, k_exact)
    assert np.array_equal(v_slot, ref["v_slot"])
    e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], None, TOL[dtype],
                         label=f"H={H}")
    _print(f"  q_out {e_q:.3g}  o max abs {e_abs:.3g}  rel-to-max {e_rel:.3g}")


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_decode_and_append(H, dtype):
    """The two separate calls (append, then decode on q_out) for every head count."""
    import torch
    dah = _dah()
    w = _with_heads("ragged_f32_b6", H, 5e6, cache_dtype=dtype)
    _print(f"[family two calls] {dtype} H={H}")
    t, seq_lens, table, _ = build_layer(w)
    everything = list(range(w.batch))
    snap = host_snapshot(t, seq_lens, table, everything)
    q_out = dah.qk_norm_rope_append(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    rope_theta=5e6)
    o = dah.paged_decode_gqa(q_out, t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                             int(seq_lens.max()))
    torch.cuda.synchronize()
    ref = oracle_step(snap, dtype, theta=5e6)
    assert float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"]))) <= 1e-5
    gates(o.cpu().numpy().astype(np.float64), ref["o"], None, TOL[dtype], label=f"H={H}")


@pytest.mark.parametrize("H", HEADS)
def test_full_size_step(H):
    """B=256, S=2048 (the benchmark's cache) with H query heads, every sequence."""
    import torch
    dah = _dah()
    w = W.WORKLOADS[f"b256_s2048_h{H}"]
    _print(f"[family step] {w.name}")
    t, seq_lens, table, _ = build_layer(w)
    every = range(w.batch)
    snap = host_snapshot(t, seq_lens, table, every)
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    int(seq_lens.max()), rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16", theta=w.rope_theta)
    e_q = float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"])))
    assert e_q <= 1e-5
    k_slot, v_slot = read_slots(t, seq_lens, table, every)
    from oracle import decode_attention as O
    _, k_exact = O.norm_rope(snap["q"], snap["k_new"], snap["q_gain"], snap["k_gain"],
                             snap["seq_lens"], theta=w.rope_theta)
    check_rounded(k_slot, k_exact)
    assert np.array_equal(v_slot, ref["v_slot"])
    dist = distance_to_uniform(ref["o"], snap, "bf16")
    e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], dist, 2e-2,
                         label=w.name)
    _print(f"  q_out {e_q:.3g}  o max abs {e_abs:.3g}  rel-to-max {e_rel:.3g}")


@pytest.mark.parametrize("H,name", [(32, "long_b4_s40960"), (64, "long_b4_s40960"),
                                    (40, "stack28_b128"), (64, "stack28_b128"),
                                    (40, "ragged_b32"), (64, "ragged_b32")])
def test_split_and_balanced_decode(H, name):
    """The split plan (4 sequences up to 40,960 positions) and the balanced
    plan (128 log-uniform lengths; 32 ragged lengths, which the matrix-core
    kernel also cuts evenly) with more query heads, every sequence."""
    import torch
    dah = _dah()
    w = _with_heads(name, H)
    plan = dah.plan_decode(w.batch, w.max_seq_len(), num_heads=H, cache_dtype=w.cache_dtype)
    _print(f"[family decode] {name} H={H} plan={plan['mode']}")
    if name != "long_b4_s40960":
        assert plan["mode"] == "balanced"
    t, seq_lens, table, _ = build_layer(w)
    snap = host_snapshot(t, seq_lens, table, range(w.batch))
    o = dah.paged_decode_gqa(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                             int(seq_lens.max()))
    torch.cuda.synchronize()
    o_ref = oracle_decode(snap, "bf16")
    dist = distance_to_uniform(o_ref, snap, "bf16")
    e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), o_ref, dist, 2e-2,
                         label=f"{name} H={H}")
    _print(f"  o max abs {e_abs:.3g}  rel-to-max {e_rel:.3g}")


@pytest.mark.parametrize("H", [32, 64])
def test_balanced_step(H):
    """The fused step under the balanced plan (32 ragged sequences, bf16
    cache: the matrix-core kernel), every sequence, q_out and the stored slot too."""
    import torch
    dah = _dah()
    w = _with_heads("ragged_b32", H, 5e6)
    _print(f"[family balanced step] H={H}")
    t, seq_lens, table, _ = build_layer(w)
    every = range(w.batch)
    snap = host_snapshot(t, seq_lens, table, every)
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    int(seq_lens.max()), rope_theta=5e6)
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16", theta=5e6)
    assert float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"]))) <= 1e-5
    _, v_slot = read_slots(t, seq_lens, table, every)
    assert np.array_equal(v_slot, ref["v_slot"])
    e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                         label=f"H={H}")
    _print(f"  o max abs {e_abs:.3g}  rel-to-max {e_rel:.3g}")


@pytest.mark.parametrize("H", HEADS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_mapping(H, dtype):
    """Doubling the values of KV head j doubles exactly query heads
    jG .. jG+G-1 (G = H/8) and leaves every other head's bits unchanged."""
    import torch
    dah = _dah()
    G = H // 8
    w = _with_heads("ragged_f32_b6", H, cache_dtype=dtype)
    t, seq_lens, table, _ = build_layer(w)
    L = int(seq_lens.max())

    def decode():
        return dah.paged_decode_gqa(t["q"], t["k_pool"], t["v_pool"], t["block_table"],
                                    t["seq_lens"], L, num_splits=1)
    base = decode().clone()
    for j in (0, 5, 7):
        vp = t["v_pool"].clone()
        t["v_pool"][:, j] *= 2.0
        o = decode()
        torch.cuda.synchronize()
        diff = (o != base).any(dim=2).cpu().numpy()
        assert set(np.nonzero(diff.any(axis=0))[0]) == set(range(j * G, (j + 1) * G))
        assert torch.equal(o[:, j * G:(j + 1) * G], 2.0 * base[:, j * G:(j + 1) * G])
        t["v_pool"] = vp


@pytest.mark.parametrize("H", [40, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place_step_with_splits(H, dtype):
    """q_out = q with a cut sequence (the two-launch path) equals the
    out-of-place fused step to float32 rounding (the two paths sum the norm
    in different orders)."""
    import torch
    dah = _dah()
    w = _with_heads("ragged_f32_b6", H, cache_dtype=dtype)
    t, seq_lens, table, _ = build_layer(w)
    L = int(seq_lens.max())
    kp, vp = t["k_pool"].clone(), t["v_pool"].clone()
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    kp, vp, t["block_table"], t["seq_lens"], L, num_splits=3)
    q = t["q"].clone()
    q2, o2 = dah.decode_attn_step(q, t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                  t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], L,
                                  num_splits=3, q_out=q)
    torch.cuda.synchronize()
    assert q2.data_ptr() == q.data_ptr()
    torch.testing.assert_close(q2, q_out, rtol=0, atol=1e-6)
    if dtype == "f32":
        torch.testing.assert_close(t["k_pool"], kp, rtol=0, atol=1e-6)
    else:  # a different norm summation order may flip one bf16 rounding
        bf16_step = 2.0 ** -7 * kp.float().abs().clamp(min=1e-30)
        assert bool(((t["k_pool"].float() - kp.float()).abs() <= bf16_step).all())
    assert torch.equal(t["v_pool"], vp)
    # bf16: the fused launch scores the new token from registers in float32,
    # the two-launch path reads it back from the cache through the matrix
    # cores (and its key may sit one rounding step away), so the two agree to
    # the bf16 tolerance's scale rather than to float32 rounding.
    torch.testing.assert_close(o2, o, rtol=0, atol=1e-6 if dtype == "f32" else 5e-5)
