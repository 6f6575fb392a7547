"""GPU parity: the HIP path against the float64 oracle on the five seeded
workloads, through the C ABI (via the thin binding).

Gates (max abs error): 1e-5 for the float32 cache, 2e-2 for the bfloat16
cache with float32 accumulation; plus the relative-to-max error of the
"Model conformance" page ("How the comparison works", step 4) <= 1e-4 and
an error under 1% of the distance to uniform attention.  Every sequence of
every workload is compared element by element ("Model conformance" page,
"How the comparison works", step 4 compares whole tensors), in the launch
configuration the benchmark times; the 28-layer stack compares every
sequence of its first, middle and last layers.
"""
import numpy as np
import pytest

from dah_testlib import (build_layer, check_rounded, cuda_available, distance_to_uniform, gates,
                         host_snapshot, oracle_decode, oracle_step, read_slots)
from inputs import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _dah():
    import decode_attention_head_amd as dah
    return dah


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", ["tiny_f32_b2", "ragged_b32", "b256_s2048", "long_b4_s40960"])
def test_decode_parity(name):
    import torch
    dah = _dah()
    w = W.WORKLOADS[name]
    _print(f"[decode parity] {name}")
    t, seq_lens, table, _ = build_layer(w)
    every = range(w.batch)
    snap = host_snapshot(t, seq_lens, table, every)
    o = dah.paged_decode_gqa(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                             int(seq_lens.max()))
    torch.cuda.synchronize()
    o_gpu = o.cpu().numpy().astype(np.float64)
    o_ref = oracle_decode(snap, w.cache_dtype)
    dist = distance_to_uniform(o_ref, snap, w.cache_dtype)
    e_abs, e_rel = gates(o_gpu, o_ref, dist, TOL[w.cache_dtype], label=name)
    _print(f"  max abs {e_abs:.3g}  rel-to-max {e_rel:.3g}  dist-to-uniform {dist:.3g}")
    assert torch.isfinite(o).all()


@pytest.mark.parametrize("name", ["tiny_f32_b2", "ragged_b32", "b256_s2048", "long_b4_s40960"])
def test_step_parity(name):
    import torch
    dah = _dah()
    w = W.WORKLOADS[name]
    _print(f"[step parity] {name}")
    t, seq_lens, table, _ = build_layer(w)
    every = range(w.batch)
    snap = host_snapshot(t, seq_lens, table, every)
    q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    int(seq_lens.max()))
    torch.cuda.synchronize()
    ref = oracle_step(snap, w.cache_dtype)
    tol = TOL[w.cache_dtype]
    qo = q_out.cpu().numpy().astype(np.float64)
    e_q = float(np.max(np.abs(qo - ref["q_out"])))
    assert e_q <= min(tol, 1e-5), f"q_out max abs err {e_q:.3g}"
    k_slot, v_slot = read_slots(t, seq_lens, table, every)
    if w.cache_dtype == "bf16":
        from oracle import decode_attention as O
        _, k_exact = O.norm_rope(snap["q"], snap["k_new"], snap["q_gain"], snap["k_gain"],
                                 snap["seq_lens"])
        flips = check_rounded(k_slot, k_exact)
        assert np.array_equal(v_slot, ref["v_slot"]), "v store is not the RNE of v_new"
        _print(f"  k slot: {flips:.2e} of entries took the other rounding neighbour")
    else:
        assert np.max(np.abs(k_slot - ref["k_slot"])) <= 1e-5
        assert np.array_equal(v_slot, ref["v_slot"])
    o_gpu = o.cpu().numpy().astype(np.float64)
    e_abs, e_rel = gates(o_gpu, ref["o"], None, tol, label=name)
    _print(f"  q_out {e_q:.3g}  o max abs {e_abs:.3g}  rel-to-max {e_rel:.3g}")


def test_stack28_layers():
    """28 layers, each with its own cache and gains, one step through all of
    them; every sequence of three layers checked against the oracle."""
    import torch
    dah = _dah()
    w = W.WORKLOADS["stack28_b128"]
    seq_lens = W.make_seq_lens(w)
    table, num_pages = W.make_block_table(w, seq_lens)
    every = range(w.batch)
    L = int(seq_lens.max())
    checked = {0, 13, 27}
    ws = torch.empty(dah.workspace_bytes(w.batch, L), dtype=torch.uint8, device="cuda")
    for layer in range(w.num_layers):
        _print(f"[stack28] layer {layer}")
        t = W.make_layer(w, layer, "cuda", table=table, num_pages=num_pages, seq_lens=seq_lens)
        snap = host_snapshot(t, seq_lens, table, every) if layer in checked else None
        q_out, o = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                        t["k_pool"], t["v_pool"], t["block_table"],
                                        t["seq_lens"], L, workspace=ws)
        if snap is not None:
            torch.cuda.synchronize()
            ref = oracle_step(snap, "bf16")
            e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], None, 2e-2,
                                 label=f"layer {layer}")
            e_q = float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"])))
            assert e_q <= 1e-5
            _print(f"  o max abs {e_abs:.3g} rel-to-max {e_rel:.3g} q_out {e_q:.3g}")
        del t
