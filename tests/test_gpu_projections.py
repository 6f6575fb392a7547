"""GPU parity of the projections around the block (attn.qkv_proj and
attn.o_proj of the "Qwen3-0.6B" Model Spec page, `linear` rows), through the
C ABI, against the float64 oracle (oracle/projections.py).

Gate, elementwise: |y_gpu - y_oracle| <= 2^-16 * sum_k |x[t,k] w[n,k]|.
The kernels feed x to the matrix cores as two bfloat16 terms (2^-18
relative per element) and accumulate in float32 (K <= 5120 terms in chains
of at most a few dozen additions); 2^-16 of the absolute sum covers both with
room, and a wrong index, a dropped k chunk or a missing x term misses it by
orders of magnitude.  Also rel-to-max <= 1e-5 ("Model conformance" page's
metric).
"""
import numpy as np
import pytest

from dah_testlib import (appended_slot_slack, build_layer, cuda_available, host_snapshot,
                         oracle_map, read_slots)
from inputs import workloads as W
from oracle import decode_attention as O
from oracle import projections as P

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _dah():
    import decode_attention_head_amd as dah
    return dah


def _print(*a):
    print(*a, flush=True)


def _bits(w):
    import torch
    return w.cpu().view(torch.int16).numpy().view(np.uint16)


def _check(y_gpu, x, w_bits, label):
    ref = P.linear(x, w_bits)
    bound = 2.0 ** -16 * P.linear(np.abs(x), np.abs(O.bf16_bits_to_f64(w_bits)), "f64") + 1e-30
    err = np.abs(np.asarray(y_gpu, np.float64) - ref)
    worst = float(np.max(err / bound))
    assert np.all(np.isfinite(y_gpu)), label
    assert worst <= 1.0, f"{label}: error {worst:.3g} x the bound"
    rel = O.rel_to_max_err(y_gpu, ref)
    assert rel <= 1e-5, f"{label}: rel-to-max {rel:.3g}"
    return worst, rel


def _rand(shape, seed, scale=1.0, dtype=None):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device="cuda") * scale
    return t if dtype is None else t.to(dtype)


LINEAR_T = [1, 7, 16, 17, 33, 48, 64, 65, 128, 256, 300, 511, 1000]
LINEAR_NK = [(4096, 1024), (1024, 2048), (192, 256)]


@pytest.mark.parametrize("N,K", LINEAR_NK)
@pytest.mark.parametrize("T", LINEAR_T)
def test_linear_parity(T, N, K):
    """Every kernel and tile shape the product picks (the split-k kernel and
    the five LDS tiles: the cases cover all six, see test_abi), ragged row
    tails, three shapes; a guard row after the output stays untouched."""
    import torch
    dah = _dah()
    kernel = dah.linear_kernel(T, N, K)
    x = _rand((T, K), 100 + T)
    w = _rand((N, K), 200 + N, 1.0 / np.sqrt(K), torch.bfloat16)
    y_all = torch.full((T + 1, N), float("nan"), device="cuda")
    y = dah.linear(x, w, y=y_all[:T])
    torch.cuda.synchronize()
    assert torch.isnan(y_all[T]).all(), "wrote past the output"
    worst, rel = _check(y.cpu().numpy(), x.cpu().numpy(), _bits(w), f"T={T} N={N} K={K}")
    _print(f"[linear] T={T} N={N} K={K} kernel {kernel}: {worst:.3f} of bound, "
           f"rel-to-max {rel:.2e}")


# T, N, K for dah_linear_ws: every LDS tile shape over 8 k slices, two over 4,
# ragged row tails, one and seven rows, N not a multiple of 128 (test_abi
# checks the plans these reach).
LINEAR_WS_CASES = [(1, 1024, 2048), (7, 192, 2048), (16, 1024, 8192), (33, 1024, 2048),
                   (64, 1024, 8192), (128, 1024, 2048), (128, 1024, 8192), (256, 1024, 2048),
                   (256, 1024, 3072), (300, 1024, 4096), (512, 1024, 8192)]


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("T,N,K", LINEAR_WS_CASES)
def test_linear_ws_parity(T, N, K, residual):
    """dah_linear_ws, k split over workgroups: against the oracle's product
    (plus the residual, within its add's rounding), the workspace filled with
    NaN beforehand (its contents on entry must not matter), a guard row after
    y untouched; with the residual also in place (residual = y), equal to the
    out-of-place result."""
    import torch
    dah = _dah()
    kernel, slices = dah.linear_ws_kernel(T, N, K)
    x = _rand((T, K), 400 + T)
    w = _rand((N, K), 500 + N + K, 1.0 / np.sqrt(K), torch.bfloat16)
    r = _rand((T, N), 600 + T) if residual else None
    need = dah.linear_workspace_bytes(T, N, K)
    assert need == slices * T * N * 4
    ws = torch.full((need // 4,), float("nan"), device="cuda").view(torch.uint8)
    y_all = torch.full((T + 1, N), float("nan"), device="cuda")
    y = dah.linear_ws(x, w, residual=r, y=y_all[:T], workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(y_all[T]).all(), "wrote past the output"
    xr, wb = x.cpu().numpy(), _bits(w)
    ref = P.linear(xr, wb)
    bound = 2.0 ** -16 * P.linear(np.abs(xr), np.abs(O.bf16_bits_to_f64(wb)), "f64") + 1e-30
    if residual:
        ref = ref + r.cpu().numpy()
        bound = bound + 2.0 ** -23 * np.abs(ref)
        r2 = r.clone()
        dah.linear_ws(x, w, residual=r2, y=r2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(r2, y), "in place differs"
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"error {worst:.3g} x the bound"
    _print(f"[linear_ws] T={T} N={N} K={K} kernel {kernel} x {slices} slices "
           f"residual={residual}: {worst:.3f} of bound")


@pytest.mark.parametrize("H,hidden", [(16, 1024), (32, 2560), (40, 5120), (64, 5120)])
@pytest.mark.parametrize("T", [1, 37, 256])
def test_qkv_and_o_proj_parity(H, hidden, T):
    """attn.qkv_proj split into q, k, v and attn.o_proj, at the family's
    widths (nnterp qwen3 page: hidden 1024 / 2560 / 5120)."""
    import dataclasses
    import torch
    dah = _dah()
    w = dataclasses.replace(W.WORKLOADS["b256_s2048"], batch=T, num_heads=H, hidden=hidden)
    p = W.make_projections(w, 0, "cuda")
    q, k, v = dah.qkv_proj(p["x"], p["w_qkv"], H)
    o = _rand((T, H, 128), 300 + H)
    y = dah.o_proj(o, p["w_o"])
    y_ws = dah.o_proj_ws(o, p["w_o"])
    torch.cuda.synchronize()
    x = p["x"].cpu().numpy()
    y_qkv = np.concatenate([q.cpu().numpy().reshape(T, -1), k.cpu().numpy().reshape(T, -1),
                            v.cpu().numpy().reshape(T, -1)], axis=1)
    wq, rq = _check(y_qkv, x, _bits(p["w_qkv"]), f"qkv H={H}")
    rq_split = P.qkv_proj(x, _bits(p["w_qkv"]), H)
    for got, ref in zip((q, k, v), rq_split):
        assert O.rel_to_max_err(got.cpu().numpy(), ref) <= 1e-5
    wo, ro = _check(y.cpu().numpy(), o.cpu().numpy().reshape(T, -1), _bits(p["w_o"]),
                    f"o_proj H={H}")
    wo2, _ = _check(y_ws.cpu().numpy(), o.cpu().numpy().reshape(T, -1), _bits(p["w_o"]),
                    f"o_proj_ws H={H}")
    _print(f"[proj] H={H} hidden={hidden} T={T}: qkv {wq:.3f} / o {wo:.3f} / o_ws "
           f"{wo2:.3f} ({dah.linear_ws_kernel(T, hidden, H * 128)}) of bound")


@pytest.mark.parametrize("name,H", [("ragged_f32_b6", 16), ("ragged_f32_b6", 64),
                                    ("b256_s2048", 16), ("b256_s2048_h64", 64)])
def test_attention_block_parity(name, H):
    """x -> attn_qkv_proj -> decode_attn_step -> attn_o_proj_ws against the
    oracle's composed block.  The device's q, k, v carry the projection's
    error (x as two bf16 terms: ~2.5e-6 relative, measured) into the norm and
    the attention, so the composed gates are 1e-4 absolute on q_out and, for
    a float32 cache, on o and y (2e-2 for bf16), with rel-to-max <= 1e-4."""
    import dataclasses
    import torch
    dah = _dah()
    w = dataclasses.replace(W.WORKLOADS[name], num_heads=H)
    _print(f"[block] {name} H={H}")
    t, seq_lens, table, _ = build_layer(w)
    p = W.make_projections(w, 0, "cuda")
    snap = host_snapshot(t, seq_lens, table, range(w.batch))
    q, k, v = dah.qkv_proj(p["x"], p["w_qkv"], H)
    q_out, o = dah.decode_attn_step(q, k, v, t["q_gain"], t["k_gain"], t["k_pool"], t["v_pool"],
                                    t["block_table"], t["seq_lens"], int(seq_lens.max()),
                                    rope_theta=w.rope_theta)
    y = dah.o_proj_ws(o, p["w_o"])
    torch.cuda.synchronize()
    x = p["x"].cpu().numpy()
    wq_bits, wo_bits = _bits(p["w_qkv"]), _bits(p["w_o"])
    ref = oracle_map(lambda rows: P.attention_block(
        x, wq_bits, wo_bits, snap["q_gain"], snap["k_gain"], snap["k_pool"], snap["v_pool"],
        snap["block_table"], snap["seq_lens"], w.cache_dtype, num_heads=H, theta=w.rope_theta,
        batch_indices=rows), w.batch, chunk=8)
    tol = 1e-4 if w.cache_dtype == "f32" else 2e-2
    e_q = float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"])))
    assert e_q <= 1e-4, f"q_out {e_q:.3g}"
    assert O.rel_to_max_err(q_out.cpu().numpy(), ref["q_out"]) <= 1e-4
    # The appended slot may hold the other bf16 neighbour wherever the
    # device's float32 projection lies within its error of a rounding
    # midpoint; the slack bounds what that moves (dah_testlib).
    slack, flagged = appended_slot_slack(snap, ref, x, wq_bits, H, w.cache_dtype)
    slack_y = P.linear(slack.reshape(w.batch, -1), np.abs(O.bf16_bits_to_f64(wo_bits)), "f64")
    for name_, got, want, sl in (("o", o, ref["o"], slack), ("y", y, ref["y"], slack_y)):
        got = got.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), name_
        err = np.abs(got - want)
        scale = float(np.max(np.abs(want)))
        assert float(err.max()) <= tol, f"{name_}: max abs {float(err.max()):.3g}"
        over = err > 1e-4 * scale + sl
        assert not over.any(), (f"{name_}: {int(over.sum())} elements exceed 1e-4 x max + slack; "
                                f"worst {float(np.max(err - sl)) / scale:.3g} of max")
        _print(f"  {name_}: rel-to-max {float(err.max()) / scale:.2e}, beyond the slack "
               f"{float(np.max(err - sl)) / scale:.2e} ({flagged} near-midpoint slot elements)")
    _print(f"  q_out {e_q:.2e}")


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("name", ["b256_s2048", "ragged_b32"])
def test_block_under_graph_replay(name, split):
    """The whole block (qkv_proj, decode_attn_step, o_proj or o_proj_ws)
    captured in one HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager result bit for bit
    (the library records no memset, allocation or host synchronisation).
    The cache is restored before each run, since the step appends to it."""
    import torch
    dah = _dah()
    w = W.WORKLOADS[name]
    t, seq_lens, table, _ = build_layer(w)
    p = W.make_projections(w, 0, "cuda")
    L = int(seq_lens.max())
    H = w.num_heads
    ws = torch.empty(max(dah.workspace_bytes(w.batch, L), 256), dtype=torch.uint8, device="cuda")
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q, k, v = dah.qkv_proj(p["x"], p["w_qkv"], H)
    q_out, o = torch.empty_like(q), torch.empty_like(q)
    y = torch.empty((w.batch, w.hidden), device="cuda")
    o_ws = torch.empty(max(dah.linear_workspace_bytes(w.batch, w.hidden, H * 128), 256),
                       dtype=torch.uint8, device="cuda")

    def block():
        dah.qkv_proj(p["x"], p["w_qkv"], H, q=q, k=k, v=v)
        dah.decode_attn_step(q, k, v, t["q_gain"], t["k_gain"], t["k_pool"], t["v_pool"],
                             t["block_table"], t["seq_lens"], L, q_out=q_out, o=o, workspace=ws)
        if split:
            dah.o_proj_ws(o, p["w_o"], y=y, workspace=o_ws)
        else:
            dah.o_proj(o, p["w_o"], y=y)

    def restore():
        t["k_pool"].copy_(k0)
        t["v_pool"].copy_(v0)

    block()
    torch.cuda.synchronize()
    want_y, want_o, want_k = y.clone(), o.clone(), t["k_pool"].clone()
    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            block()
    torch.cuda.synchronize()
    for i in range(3):
        restore()
        y.zero_()
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want_y), f"replay {i}: y differs"
        assert torch.equal(o, want_o), f"replay {i}: o differs"
        assert torch.equal(t["k_pool"], want_k), f"replay {i}: cache differs"
        _ = (p["x"] * 2).sum().item()   # eager work between replays
