"""GPU checks of properties the pages state, on the HIP path through the C ABI:

  * flash decoding equals the spec for any split (theorem flashAttn_eq,
    "Supported models" page, "Facts proved about the specs"): results for
    forced split counts agree with each other and with the oracle;
  * causality / locality (forward_causal, attnHead_local): cache entries at or
    past seq_len, and unused pages, never influence o, even as NaN;
  * one cached position gives o = v; identical keys give the mean of v
    (attnWeights_distribution);
  * KV head j reaches only query heads 2j and 2j+1 (nnterp qwen3 page,
    "The Notes");
  * batch independence, idempotent re-append, the defined results for
    out-of-domain device values, and the workspace check;
  * edge shapes: B = 1, seq_len 1, 15, 16, 17, page-aligned and ragged
    tails, and the domain's maximum (B = 256, S = 40,960), every sequence.
"""
import numpy as np
import pytest

from dah_testlib import (build_layer, cuda_available, gates, host_snapshot, oracle_decode,
                         oracle_step)
from inputs import workloads as W
from oracle import decode_attention as O

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _dah():
    import decode_attention_head_amd as dah
    return dah


def _print(*a):
    print(*a, flush=True)


def _custom(batch, lens, dtype="bf16", pool_pages=None, seed=11, outlier=None):
    return W.Workload(f"custom_{seed}", batch=batch, cache_dtype=dtype, seed=seed,
                      lens_kind="list", lens_args=tuple(int(x) for x in lens),
                      pool_pages=pool_pages, key_outlier=outlier)


def _decode(t, L, **kw):
    dah = _dah()
    return dah.paged_decode_gqa(t["q"], t["k_pool"], t["v_pool"], t["block_table"],
                                t["seq_lens"], L, **kw)


def test_split_count_invariance():
    import torch
    lens = [1, 15, 16, 17, 100, 257, 1024, 3000, 4096, 513]
    w = _custom(len(lens), lens, seed=21)
    _print("[splits] building")
    t, seq_lens, table, _ = build_layer(w)
    snap = host_snapshot(t, seq_lens, table, range(len(lens)))
    ref = oracle_decode(snap, "bf16")
    L = int(max(lens))
    outs, kernel = {}, {}
    for n in (1, 0, 2, 3, 7, 16, 64, 256):
        kernel[n] = _dah().plan_decode(len(lens), L, n)["kernel"]
        _print(f"[splits] num_splits={n} kernel={kernel[n]}")
        o = _decode(t, L, num_splits=n)
        torch.cuda.synchronize()
        outs[n] = o.cpu().numpy().astype(np.float64)
        gates(outs[n], ref, None, 2e-2, label=f"splits={n}")
    # Within the VALU kernel the partition changes only the rounding order
    # (flashAttn_eq); the matrix-core kernel (one split here) carries the
    # weights to 2^-18, so against it the bound is that.
    base = outs[1]
    scale = float(np.max(np.abs(base)))
    for n, o in outs.items():
        tol = 1e-6 if kernel[n] == kernel[1] == "valu" else 2.0 ** -16 * scale
        assert np.max(np.abs(o - base)) <= tol, f"splits={n} differs from 1 split"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_poison_outside_prefix(dtype):
    import torch
    lens = [1, 7, 16, 17, 31, 33, 200]
    w = _custom(len(lens), lens, dtype=dtype, pool_pages=64, seed=22)
    t, seq_lens, table, _ = build_layer(w)
    L = int(max(lens))
    clean = {n: _decode(t, L, num_splits=n).clone() for n in (0, 1, 3)}
    W.poison_unused(t, seq_lens, table, value=float("nan"))
    for n in (0, 1, 3):
        poisoned = _decode(t, L, num_splits=n)
        torch.cuda.synchronize()
        assert torch.equal(poisoned, clean[n]), f"poisoned tail changed o (splits={n})"
    W.poison_unused(t, seq_lens, table, value=float("inf"))
    assert torch.equal(_decode(t, L, num_splits=1), clean[1])


def test_step_into_poisoned_slot():
    """The step writes the new token over a NaN slot and reads only what it wrote."""
    import torch
    dah = _dah()
    lens = [1, 2, 16, 17, 40]
    w = _custom(len(lens), lens, dtype="bf16", pool_pages=32, seed=23)
    t, seq_lens, table, _ = build_layer(w)
    snap = host_snapshot(t, seq_lens, table, range(len(lens)))
    W.poison_unused(t, seq_lens, table, include_new_slot=True)
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    int(max(lens)))
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16")
    gates(o.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2, label="poisoned step")


def test_single_position_returns_v_exactly():
    import torch
    lens = [1] * 9
    w = _custom(9, lens, dtype="f32", pool_pages=16, seed=24)
    t, seq_lens, table, _ = build_layer(w)
    o = _decode(t, 1)
    torch.cuda.synchronize()
    for b in range(9):
        page = int(table[b, 0])
        for h in range(16):
            assert torch.equal(o[b, h], t["v_pool"][page, h // 2, 0]), (b, h)


def test_identical_keys_give_mean_of_v():
    import torch
    lens = [100, 2048, 777]
    w = _custom(3, lens, dtype="bf16", seed=25)
    t, seq_lens, table, _ = build_layer(w)
    t["k_pool"][:] = t["k_pool"][0, :, 0:1, :]           # every position holds the same keys
    snap = host_snapshot(t, seq_lens, table, range(3))
    o = _decode(t, max(lens), num_splits=4)
    torch.cuda.synchronize()
    for i in range(3):
        v = O.gather_sequence(snap["v_pool"], snap["block_table"][i], lens[i], "bf16")
        mean = v.mean(axis=0)
        for h in range(16):
            assert np.max(np.abs(o[i, h].cpu().numpy() - mean[h // 2])) <= 2e-6


def test_head_mapping():
    import torch
    lens = [300, 45]
    w = _custom(2, lens, dtype="bf16", seed=26)
    t, seq_lens, table, _ = build_layer(w)
    base = _decode(t, 300).clone()
    for j in (0, 3, 7):
        vp = t["v_pool"].clone()
        t["v_pool"][:, j] *= 2.0
        o = _decode(t, 300)
        torch.cuda.synchronize()
        diff = (o != base).any(dim=2).cpu().numpy()           # [B,16]
        assert set(np.nonzero(diff.any(axis=0))[0]) == {2 * j, 2 * j + 1}
        assert torch.equal(o[:, 2 * j:2 * j + 2], 2.0 * base[:, 2 * j:2 * j + 2])
        t["v_pool"] = vp


def test_batch_permutation():
    import torch
    lens = [5, 600, 1234, 16, 4000, 33]
    w = _custom(len(lens), lens, dtype="bf16", seed=27)
    t, seq_lens, table, _ = build_layer(w)
    L = max(lens)
    o = _decode(t, L, num_splits=1)
    perm = torch.tensor([3, 0, 5, 1, 4, 2], device="cuda")
    t2 = dict(t)
    t2["q"] = t["q"][perm].contiguous()
    t2["block_table"] = t["block_table"][perm].contiguous()
    t2["seq_lens"] = t["seq_lens"][perm].contiguous()
    o2 = _decode(t2, L, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o2, o[perm])


def test_step_is_idempotent():
    import torch
    dah = _dah()
    lens = [9, 64, 65, 1000]
    w = _custom(4, lens, dtype="bf16", seed=28)
    t, seq_lens, table, _ = build_layer(w)
    args = (t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"], t["k_pool"], t["v_pool"],
            t["block_table"], t["seq_lens"], 1000)
    q1, o1 = dah.decode_attn_step(*args)
    k1, v1 = t["k_pool"].clone(), t["v_pool"].clone()
    q2, o2 = dah.decode_attn_step(*args)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(o1, o2)
    assert torch.equal(k1, t["k_pool"]) and torch.equal(v1, t["v_pool"])


def test_append_touches_only_the_new_slot():
    import torch
    dah = _dah()
    lens = [3, 16, 17, 48]
    w = _custom(4, lens, dtype="bf16", pool_pages=16, seed=29)
    t, seq_lens, table, _ = build_layer(w)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    dah.qk_norm_rope_append(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                            t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"])
    torch.cuda.synchronize()
    changed = (t["k_pool"] != k0).any(dim=3) | (t["v_pool"] != v0).any(dim=3)   # [P,8,16]
    want = torch.zeros_like(changed)
    for b, n in enumerate(lens):
        want[int(table[b, (n - 1) // 16]), :, (n - 1) % 16] = True
    assert torch.equal(changed, want)


def test_out_of_domain_device_values():
    """seq_len <= 0: o = 0 and no append; seq_len > max_seq_len or a page id
    outside the pool: o = NaN and no append.  No fault in any case."""
    import torch
    dah = _dah()
    lens = [20, 20, 20, 20, 20]
    w = _custom(5, lens, dtype="bf16", pool_pages=16, seed=30)
    t, seq_lens, table, num_pages = build_layer(w)
    sl = t["seq_lens"]
    sl[1] = 0
    sl[2] = -3
    sl[3] = 33                       # above max_seq_len = 32 below
    t["block_table"][4, 1] = num_pages + 5
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    for n in (1, 2, 0):
        q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                        t["k_pool"], t["v_pool"], t["block_table"], sl, 32,
                                        num_splits=n)
        torch.cuda.synchronize()
        assert torch.isfinite(o[0]).all()
        assert torch.equal(o[1], torch.zeros_like(o[1])) and torch.equal(o[2], torch.zeros_like(o[2]))
        assert torch.isnan(o[3]).all() and torch.isnan(o[4]).all()
    # only sequence 0's slot may have changed
    changed = (t["k_pool"] != k0).any(dim=3) | (t["v_pool"] != v0).any(dim=3)
    assert int(changed.sum()) == 8 and bool(changed[int(table[0, 1]), :, 3].all())


def test_workspace_too_small_is_rejected():
    import torch
    dah = _dah()
    lens = [4096] * 4
    w = _custom(4, lens, dtype="bf16", seed=31)
    t, seq_lens, table, _ = build_layer(w)
    need = dah.workspace_bytes(4, 4096)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(dah.DahError) as e:
        _decode(t, 4096, workspace=small)
    assert e.value.status == 5


def test_large_gain_peaked_softmax():
    """Gains of the trained model's magnitude (k_norm up to 96.5, q_norm up to
    11.8, nnterp qwen3 page) give scores of O(1e3) and a sharply peaked
    softmax; a sink key at position 0 aligned with the query."""
    import torch
    dah = _dah()
    lens = [2048, 517, 40]
    w = _custom(3, lens, dtype="bf16", seed=32)
    t, seq_lens, table, _ = build_layer(w)
    t["q_gain"] *= 11.8
    t["k_gain"] *= 96.5
    # a sink at position 0: the key equals a scaled copy of the (normed) query direction
    for b in range(3):
        p0 = int(table[b, 0])
        t["k_pool"][p0, :, 0, :] = (t["q"][b, ::2, :] * 4.0).to(torch.bfloat16)
    snap = host_snapshot(t, seq_lens, table, range(3))
    for n in (1, 5, 0):
        k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
        q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                        t["k_pool"], t["v_pool"], t["block_table"],
                                        t["seq_lens"], 2048, num_splits=n)
        torch.cuda.synchronize()
        ref = oracle_step(snap, "bf16")
        e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                             tol_rel=5e-4, label=f"large gains splits={n}")
        _print(f"  large gains splits={n}: max abs {e_abs:.3g} rel {e_rel:.3g}")
        t["k_pool"], t["v_pool"] = k0, v0


def test_domain_maximum_every_sequence():
    """B = 256 sequences of S = 40,960 positions (the shape domain's corners,
    "At a glance"): every sequence against the oracle, 32 at a time so that
    the host holds 5 GB of pages at once."""
    import torch
    w = W.Workload("max_b256_s40960", batch=256, cache_dtype="bf16", seed=33,
                   lens_kind="fixed", lens_args=(40960,))
    _print("[max] building 256 x 40960")
    t, seq_lens, table, _ = build_layer(w)
    o = _decode(t, 40960)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    o_host = o.cpu().numpy().astype(np.float64)
    worst_abs = worst_rel = 0.0
    for first in range(0, w.batch, 32):
        rows = list(range(first, first + 32))
        snap = host_snapshot(t, seq_lens, table, rows)
        ref = oracle_decode(snap, "bf16")
        e_abs, e_rel = gates(o_host[rows], ref, None, 2e-2, label=f"max, rows {first}..")
        worst_abs, worst_rel = max(worst_abs, e_abs), max(worst_rel, e_rel)
        del snap
    _print(f"  max shape, all {w.batch} sequences: max abs {worst_abs:.3g} rel {worst_rel:.3g}")


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_step_in_place_query(splits):
    """q_out may be q: the in-place call gives the same q_out, o and cache as
    a call with a separate q_out."""
    import torch
    dah = _dah()
    lens = [1, 16, 17, 250, 1000]
    w = _custom(len(lens), lens, dtype="bf16", seed=34)
    t, seq_lens, table, _ = build_layer(w)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q_sep, o_sep = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                        t["k_pool"], t["v_pool"], t["block_table"],
                                        t["seq_lens"], 1000, num_splits=splits)
    k1, v1 = t["k_pool"].clone(), t["v_pool"].clone()
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    q = t["q"].clone()
    q_in, o_in = dah.decode_attn_step(q, t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                      t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                      1000, num_splits=splits, q_out=q)
    torch.cuda.synchronize()
    assert q_in.data_ptr() == q.data_ptr()
    assert torch.allclose(q_in, q_sep, atol=1e-6, rtol=0)
    assert torch.allclose(o_in, o_sep, atol=1e-6, rtol=0)
    bf16_step = 2.0 ** -7 * t["k_pool"].float().abs().clamp(min=1e-30)
    assert bool(((t["k_pool"].float() - k1.float()).abs() <= bf16_step).all())
    assert torch.equal(t["v_pool"], v1)


@pytest.mark.parametrize("splits", [1, 4, 0])
def test_fused_step_matches_two_calls(splits):
    """decode_attn_step (one fused launch) against qk_norm_rope_append followed
    by paged_decode_gqa: same q_out and o to float32 rounding, same stored v,
    stored k within one bf16 step (the two kernels sum the norm in different
    orders, which may flip a rounding decision)."""
    import torch
    dah = _dah()
    lens = [1, 2, 15, 16, 17, 33, 700, 2048]
    w = _custom(len(lens), lens, dtype="bf16", seed=35)
    t, seq_lens, table, _ = build_layer(w)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q_f, o_f = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    2048, num_splits=splits)
    kf, vf = t["k_pool"].clone(), t["v_pool"].clone()
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    q_2 = dah.qk_norm_rope_append(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                  t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"])
    o_2 = dah.paged_decode_gqa(q_2, t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                               2048, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.allclose(q_f, q_2, atol=2e-6, rtol=0)
    assert torch.allclose(o_f, o_2, atol=2e-5, rtol=0)
    assert torch.equal(vf, t["v_pool"])
    step = 2.0 ** -7 * t["k_pool"].float().abs()
    assert bool(((kf.float() - t["k_pool"].float()).abs() <= step).all())


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_step_touches_only_the_new_slot(splits):
    import torch
    dah = _dah()
    lens = [1, 3, 16, 17, 48, 95]
    w = _custom(len(lens), lens, dtype="bf16", pool_pages=24, seed=36)
    t, seq_lens, table, _ = build_layer(w)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"], t["k_pool"],
                         t["v_pool"], t["block_table"], t["seq_lens"], 95, num_splits=splits)
    torch.cuda.synchronize()
    changed = (t["k_pool"] != k0).any(dim=3) | (t["v_pool"] != v0).any(dim=3)   # [P,8,16]
    want = torch.zeros_like(changed)
    for b, n in enumerate(lens):
        want[int(table[b, (n - 1) // 16]), :, (n - 1) % 16] = True
    assert torch.equal(changed, want)


def test_balanced_plan_with_more_workgroups_than_pages():
    """Balanced decode when the batch has fewer pages than workgroups (some
    workgroups own no page): results match the per-sequence layout."""
    import torch
    dah = _dah()
    lens = list(np.random.default_rng(38).integers(1, 48, 80))
    w = _custom(len(lens), lens, dtype="bf16", seed=37)
    t, seq_lens, table, _ = build_layer(w)
    L = int(max(lens))
    plan = dah.plan_decode(len(lens), L)
    assert plan["mode"] == "balanced" and plan["workgroups"] > sum(-(-n // 16) for n in lens)
    o_bal = _decode(t, L, num_splits=0)
    o_one = _decode(t, L, num_splits=1)
    torch.cuda.synchronize()
    assert torch.isfinite(o_bal).all()
    # The matrix-core kernel's weights depend (at 2^-18) on the softmax
    # reference, which depends on the partition; the VALU kernel's only on
    # the rounding order.
    mfma = plan["kernel"] == "mfma"
    tol = 2.0 ** -16 * float(o_one.abs().max()) if mfma else 1e-6
    assert torch.allclose(o_bal, o_one, atol=tol, rtol=0)
    snap = host_snapshot(t, seq_lens, table, range(len(lens)))
    gates(o_bal.cpu().numpy().astype(np.float64), oracle_decode(snap, "bf16"), None, 2e-2,
          label="balanced, T < G")


@pytest.mark.parametrize("H", [16, 40])
def test_balanced_out_of_domain_device_values(H):
    """The balanced layout (its merge reads the page prefix sums the decode
    leaves in the workspace) with out-of-domain device values: seq_len <= 0
    gives o = 0, seq_len > max_seq_len or a page id outside the pool gives
    o = NaN; every other sequence matches the per-sequence layout."""
    import dataclasses
    import torch
    dah = _dah()
    rng = np.random.default_rng(40)
    lens = [int(x) for x in rng.integers(1, 2000, 80)]
    lens[4] = 2000                   # spread over several workgroups
    w = dataclasses.replace(_custom(len(lens), lens, dtype="bf16", seed=41), num_heads=H)
    t, seq_lens, table, num_pages = build_layer(w)
    L = int(max(lens))
    assert dah.plan_decode(len(lens), L, num_heads=H, cache_dtype="bf16")["mode"] == "balanced"
    sl = t["seq_lens"]
    sl[1] = 0
    sl[2] = -3
    sl[3] = L + 1                    # above max_seq_len
    t["block_table"][4, 3] = num_pages + 5

    def step(n):
        _, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], sl, L,
                                    num_splits=n)
        torch.cuda.synchronize()
        return o

    o_bal = step(0)
    o_one = step(1)                  # the same append again (idempotent), one workgroup each
    for o in (o_bal, o_one):
        assert torch.equal(o[1], torch.zeros_like(o[1])) and torch.equal(o[2], torch.zeros_like(o[2]))
        assert torch.isnan(o[3]).all() and torch.isnan(o[4]).all()
    keep = [b for b in range(len(lens)) if b not in (1, 2, 3, 4)]
    assert torch.isfinite(o_bal[keep]).all()
    tol = 2.0 ** -16 * float(o_one[keep].abs().max())   # the matrix-core kernel's reference
    assert torch.allclose(o_bal[keep], o_one[keep], atol=tol, rtol=0)


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_balanced_ragged_batch_matches_oracle(splits):
    """A ragged batch of 96 sequences (1 .. 6000 positions, some sharing
    workgroups, some spread over many) in every layout, with the fused step."""
    import torch
    dah = _dah()
    rng = np.random.default_rng(39)
    lens = list(np.floor(np.exp(rng.uniform(0, np.log(6000), 96))).astype(int))
    w = _custom(len(lens), lens, dtype="bf16", seed=38)
    t, seq_lens, table, _ = build_layer(w)
    L = int(max(lens))
    if splits == 0:
        assert dah.plan_decode(len(lens), L)["mode"] == "balanced"
    snap = host_snapshot(t, seq_lens, table, range(len(lens)))
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L, num_splits=splits)
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16")
    e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                         label=f"ragged step, splits={splits}")
    assert float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"]))) <= 1e-5
    _print(f"  ragged step splits={splits}: max abs {e_abs:.3g} rel {e_rel:.3g}")


@pytest.mark.parametrize("H,splits", [(16, 0), (40, 0), (16, 5), (16, 1)])
def test_step_under_graph_replay(H, splits):
    """decode_attn_step captured in one HIP graph under the balanced plan
    (the merge reads the prefix sums the decode leaves in the workspace),
    fixed splits and one workgroup per sequence: every replay, with eager
    work and synchronisations between replays, equals the eager result bit
    for bit.  The cache is restored before each run."""
    import dataclasses
    import torch
    dah = _dah()
    rng = np.random.default_rng(42)
    lens = [int(x) for x in rng.integers(1, 1500, 80)]
    w = dataclasses.replace(_custom(len(lens), lens, dtype="bf16", seed=43), num_heads=H)
    t, seq_lens, table, _ = build_layer(w)
    L = int(max(lens))
    plan = dah.plan_decode(len(lens), L, splits, num_heads=H, cache_dtype="bf16")
    assert plan["mode"] == {0: "balanced", 5: "split", 1: "per_sequence"}[splits]
    ws = torch.empty(max(dah.workspace_bytes(len(lens), L, splits, num_heads=H,
                                             cache_dtype="bf16"), 256),
                     dtype=torch.uint8, device="cuda")
    q_out, o = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def step():
        dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                             t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], L,
                             num_splits=splits, q_out=q_out, o=o, workspace=ws)

    def restore():
        t["k_pool"].copy_(k0)
        t["v_pool"].copy_(v0)

    step()
    torch.cuda.synchronize()
    want_o, want_q, want_k = o.clone(), q_out.clone(), t["k_pool"].clone()
    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for i in range(3):
        restore()
        o.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), f"replay {i}: o differs"
        assert torch.equal(q_out, want_q), f"replay {i}: q_out differs"
        assert torch.equal(t["k_pool"], want_k), f"replay {i}: cache differs"
        _ = (t["q"] * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("H", [16, 64])
def test_sorted_page_walk_matches_oracle(H):
    """The matrix-core decode walks a range of 65 .. 129 pages in ascending
    page order, its final (possibly masked) page last, and shorter or longer
    ranges in table order.  Lengths on either side of both bounds, with
    page-aligned and ragged tails, one workgroup per sequence: the fused step
    (the new slot and every slot past the sequence poisoned with NaN first)
    and the decode alone on its q_out, against the oracle."""
    import dataclasses
    import torch
    dah = _dah()
    lens = [1024, 1025, 1040, 1041, 1500, 2048, 2064, 2065, 2080]
    w = dataclasses.replace(_custom(len(lens), lens, dtype="bf16", seed=41), num_heads=H)
    t, seq_lens, table, _ = build_layer(w)
    L = int(max(lens))
    assert dah.plan_decode(len(lens), L, 1, num_heads=H)["kernel"] == "mfma"
    snap = host_snapshot(t, seq_lens, table, range(len(lens)))
    W.poison_unused(t, seq_lens, table, include_new_slot=True, value=float("nan"))
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L, num_splits=1)
    o_dec = dah.paged_decode_gqa(q_out, t["k_pool"], t["v_pool"], t["block_table"],
                                 t["seq_lens"], L, num_splits=1)
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16")
    for got, label in ((o, "step"), (o_dec, "decode")):
        e_abs, e_rel = gates(got.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                             label=f"sorted walk {label} H={H}")
        _print(f"  sorted walk {label} H={H}: max abs {e_abs:.3g} rel {e_rel:.3g}")


def test_sorted_page_walk_with_bad_and_repeated_ids():
    """Ranges the decode sorts (94 pages, one workgroup per sequence): a page
    id outside the pool gives o = NaN for that sequence, as in table order,
    while the new token still lands in its own (valid) page; an id repeated
    within a row counts its page twice, as the oracle reading through the
    same table does."""
    import torch
    dah = _dah()
    lens = [1500, 1500, 1500]
    w = _custom(len(lens), lens, dtype="bf16", seed=43)
    t, seq_lens, table, num_pages = build_layer(w)
    L = int(max(lens))
    table = table.copy()
    table[2, 21] = table[2, 20]                        # sequence 2 reads page 20 twice
    t["block_table"].copy_(torch.from_numpy(table))
    snap = host_snapshot(t, seq_lens, table, [0, 2])
    t["block_table"][1, 10] = num_pages + 7            # sequence 1: outside the pool
    last1 = int(table[1, (lens[1] - 1) // 16])
    slot1 = (lens[1] - 1) % 16
    k1 = t["k_pool"][last1].clone()
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L, num_splits=1)
    torch.cuda.synchronize()
    assert torch.isnan(o[1]).all()
    after = t["k_pool"][last1]
    assert torch.equal(after[:, :slot1], k1[:, :slot1]), "other slots changed"
    assert not torch.equal(after[:, slot1], k1[:, slot1]), "new token not stored"
    ref = oracle_step(snap, "bf16")
    got = o[[0, 2]].cpu().numpy().astype(np.float64)
    e_abs, e_rel = gates(got, ref["o"], None, 2e-2, label="sorted walk, repeated id")
    _print(f"  sorted walk with bad/repeated ids: max abs {e_abs:.3g} rel {e_rel:.3g}")


def _balanced_segments(lens, workgroups):
    """(sequence, first page, pages) of every segment the balanced decode
    walks: the batch's pages in sequence order cut into `workgroups` ranges
    [floor(k T / G), floor((k+1) T / G)), each split at sequence ends."""
    pages = [W.pages_for(n) for n in lens]
    prefix = np.concatenate([[0], np.cumsum(pages)])
    T, G = int(prefix[-1]), int(workgroups)
    segs = []
    for k in range(G):
        s, e = k * T // G, (k + 1) * T // G
        while s < e:
            b = int(np.searchsorted(prefix, s, side="right") - 1)
            end = min(e, int(prefix[b + 1]))
            segs.append((b, s - int(prefix[b]), end - s))
            s = end
    return segs


@pytest.mark.parametrize("H", [16, 64])
def test_balanced_sorted_ranges_with_bad_and_repeated_ids(H):
    """The balanced plan with workgroup ranges of 65 .. 129 pages, which the
    matrix-core decode walks in ascending page order, most of them starting
    in the middle of a sequence and some sharing a workgroup with the end of
    the previous sequence.  Every slot past each sequence (and the new
    token's slot) NaN-poisoned, one page id repeated inside a row (the
    oracle reading through the same table counts that page twice), one id
    outside the pool (that sequence gives NaN, its neighbours in the same
    workgroups are unaffected).  The fused step and the decode alone on its
    q_out, every other sequence against the oracle."""
    import dataclasses
    import torch
    dah = _dah()
    rng = np.random.default_rng(50 + H)
    lens = [int(x) for x in rng.integers(2000, 9000, 64)]
    w = dataclasses.replace(_custom(len(lens), lens, dtype="bf16", seed=51), num_heads=H)
    t, seq_lens, table, num_pages = build_layer(w)
    L = int(max(lens))
    plan = dah.plan_decode(len(lens), L, num_heads=H, cache_dtype="bf16")
    assert plan["mode"] == "balanced" and plan["kernel"] == "mfma"
    segs = _balanced_segments(lens, plan["workgroups"])
    window = [sg for sg in segs if 65 <= sg[2] <= 129]
    assert len(window) >= 0.6 * len(segs), "ranges outside the sorted walk's window"
    assert sum(1 for sg in window if sg[1] > 0) >= 0.5 * len(segs), "few mid-sequence starts"
    rep, bad = 9, 30                                   # the repeated-id and bad-id sequences
    table = table.copy()
    table[rep, 40] = table[rep, 39]                    # page 39 read twice, page 40's dropped
    t["block_table"].copy_(torch.from_numpy(table))
    keep = [b for b in range(len(lens)) if b != bad]
    snap = host_snapshot(t, seq_lens, table, keep)
    W.poison_unused(t, seq_lens, table, include_new_slot=True, value=float("nan"))
    t["block_table"][bad, 50] = num_pages + 7          # after poisoning: the host table stays valid
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L)
    o_dec = dah.paged_decode_gqa(q_out, t["k_pool"], t["v_pool"], t["block_table"],
                                 t["seq_lens"], L)
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16")
    assert float(np.max(np.abs(q_out[keep].cpu().numpy() - ref["q_out"]))) <= 1e-5
    for got, label in ((o, "step"), (o_dec, "decode")):
        assert torch.isnan(got[bad]).all(), f"{label}: the bad id did not give NaN"
        e_abs, e_rel = gates(got[keep].cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                             label=f"balanced sorted {label} H={H}")
        _print(f"  balanced sorted ranges {label} H={H}: {len(window)} of {len(segs)} segments "
               f"in 65..129 pages; max abs {e_abs:.3g} rel {e_rel:.3g}")


def test_split_sorted_ranges_at_64_heads():
    """Fixed splits of 107 pages (the long-context batch, 24 splits of its
    2,560-page sequences) at 64 query heads: the matrix-core decode walks
    every full split, each starting mid-sequence, in ascending page order;
    tails NaN-poisoned, every sequence against the oracle, the fused step
    and the decode alone."""
    import dataclasses
    import torch
    dah = _dah()
    w = dataclasses.replace(W.WORKLOADS["long_b4_s40960"], num_heads=64)
    t, seq_lens, table, _ = build_layer(w)
    L = int(seq_lens.max())
    plan = dah.plan_decode(w.batch, L, 24, num_heads=64, cache_dtype="bf16")
    assert plan["mode"] == "split" and plan["kernel"] == "mfma"
    assert 65 <= plan["pages_per_split"] <= 128
    snap = host_snapshot(t, seq_lens, table, range(w.batch))
    W.poison_unused(t, seq_lens, table, include_new_slot=True, value=float("nan"))
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L, num_splits=24)
    o_dec = dah.paged_decode_gqa(q_out, t["k_pool"], t["v_pool"], t["block_table"],
                                 t["seq_lens"], L, num_splits=24)
    torch.cuda.synchronize()
    ref = oracle_step(snap, "bf16")
    for got, label in ((o, "step"), (o_dec, "decode")):
        e_abs, e_rel = gates(got.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                             label=f"split sorted {label}")
        _print(f"  split sorted ranges ({plan['pages_per_split']} pages) {label}: "
               f"max abs {e_abs:.3g} rel {e_rel:.3g}")


@pytest.mark.parametrize("H,splits", [(16, 1), (16, 0), (16, 3), (64, 1), (64, 0), (40, 5)])
def test_step_without_q_out(H, splits):
    """decode_attn_step with a NULL q_out writes o and the cache exactly as
    the call that also stores q_out (the same launches, minus that store),
    on every plan: one workgroup per sequence, balanced, fixed splits."""
    import dataclasses
    import torch
    dah = _dah()
    rng = np.random.default_rng(60 + H + splits)
    lens = [int(x) for x in rng.integers(1, 3000, 72)] + [1, 16, 17, 2048]
    w = dataclasses.replace(_custom(len(lens), lens, dtype="bf16", seed=61), num_heads=H)
    t, seq_lens, table, _ = build_layer(w)
    L = int(max(lens))
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L, num_splits=splits)
    k1, v1 = t["k_pool"].clone(), t["v_pool"].clone()
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    none, o2 = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    L, num_splits=splits, q_out=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o2, o)
    assert torch.equal(t["k_pool"], k1) and torch.equal(t["v_pool"], v1)
