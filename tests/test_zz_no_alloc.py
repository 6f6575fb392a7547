"""decode_attn_step_noalloc, the allocation-free variant of decode_attn_step_ex
(its split partials in the library's static device scratch instead of a
caller workspace), through the C ABI: each call gives exactly what
decode_attn_step gives on the same inputs with its own workspace -- the same
plan and kernels -- over two calls in a row (the second smaller, so it runs
over the first one's leftover scratch), at 16 and 64 query heads; a plan
too large for the scratch is refused before anything is launched."""
import dataclasses

import numpy as np
import pytest

from dah_testlib import build_layer, cuda_available
from inputs import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _dah():
    import decode_attention_head_amd as dah
    return dah


def _case(lens, H, seed):
    w = W.Workload(f"noalloc_{seed}", batch=len(lens), cache_dtype="bf16", seed=seed,
                   lens_kind="list", lens_args=tuple(int(x) for x in lens))
    return build_layer(dataclasses.replace(w, num_heads=H))


def _both(t, L, splits, H):
    """(q_out, o, k_pool, v_pool) from decode_attn_step and from the no-alloc
    call, each on its own copy of the cache."""
    import torch
    dah = _dah()
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    ws = torch.empty(max(dah.workspace_bytes(t["q"].shape[0], L, splits, num_heads=H,
                                             cache_dtype="bf16"), 256),
                     dtype=torch.uint8, device="cuda")
    q_ref, o_ref = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                        t["k_pool"], t["v_pool"], t["block_table"],
                                        t["seq_lens"], L, num_splits=splits, workspace=ws)
    k_ref, v_ref = t["k_pool"].clone(), t["v_pool"].clone()
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    q_na, o_na = dah.decode_attn_step_noalloc(t["q"], t["k_new"], t["v_new"], t["q_gain"],
                                              t["k_gain"], t["k_pool"], t["v_pool"],
                                              t["block_table"], t["seq_lens"], L,
                                              num_splits=splits)
    torch.cuda.synchronize()
    return (q_ref, o_ref, k_ref, v_ref), (q_na, o_na, t["k_pool"], t["v_pool"])


@pytest.mark.parametrize("H", [16, 64])
def test_noalloc_matches_the_workspace_call_twice(H):
    import torch
    dah = _dah()
    rng = np.random.default_rng(70 + H)
    first = [int(x) for x in np.floor(np.exp(rng.uniform(np.log(16), np.log(16384), 128)))]
    second = [int(x) for x in rng.integers(512, 4097, 32)]
    for lens, splits in ((first, 0), (second, 0), (second, 5)):
        t, seq_lens, table, _ = _case(lens, H, seed=71 + len(lens) + splits)
        L = int(max(lens))
        plan = dah.plan_decode(len(lens), L, splits, num_heads=H, cache_dtype="bf16")
        assert 0 < plan["workspace_bytes"] <= dah.SCRATCH_BYTES
        ref, got = _both(t, L, splits, H)
        for name, a, b in zip(("q_out", "o", "k_pool", "v_pool"), ref, got):
            assert torch.equal(a, b), f"{name} differs (H={H}, B={len(lens)}, plan {plan['mode']})"
        assert torch.isfinite(got[1]).all()
        print(f"[noalloc] H={H} B={len(lens)} plan={plan['mode']} "
              f"scratch {plan['workspace_bytes']} B: identical", flush=True)
        del t


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    import torch
    dah = _dah()
    lens = [32] * 1024
    t, seq_lens, table, _ = _case(lens, 16, seed=79)
    plan = dah.plan_decode(1024, 32, 2, num_heads=16, cache_dtype="bf16")
    assert plan["workspace_bytes"] > dah.SCRATCH_BYTES
    k0 = t["k_pool"].clone()
    o = torch.full_like(t["q"], 3.0)
    with pytest.raises(dah.DahError) as exc:
        dah.decode_attn_step_noalloc(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                     t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                     32, num_splits=2, o=o)
    assert "scratch" in str(exc.value)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and torch.equal(t["k_pool"], k0)
