"""GPU parity of the decoder layer's pieces and of the whole layer step
(decoder_layer_step) against the float64 oracle (oracle/layer.py): the
standalone RMSNorm and silu*up, the product with the norm folded into its
input (as the layer runs it), the residual product, and the layer.

Gates: the hidden-size RMSNorm and silu*up elementwise within float32
rounding (rel 1e-6 of the row / element); the residual product within the
projection bound plus the add's rounding; the whole layer's x1 and y with
rel-to-max <= 1e-4 (the products feed x as two bf16 terms, the attention its
weights as two) and max abs 1e-4 (float32 cache) or 2e-2 (bf16 cache).
"""
import dataclasses

import numpy as np
import pytest

from dah_testlib import build_layer, cuda_available, gates, host_snapshot, oracle_map
from inputs import workloads as W
from oracle import decode_attention as O
from oracle import layer as L
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


def _rand(shape, seed, scale=1.0):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda") * scale


@pytest.mark.parametrize("T,width", [(1, 1024), (37, 2560), (256, 1024), (5, 5120)])
def test_rmsnorm_parity(T, width):
    import torch
    dah = _dah()
    x = _rand((T, width), T + width, 2.0)
    w = 1.0 + 0.1 * _rand((width,), 7)
    y = dah.rmsnorm(x, w)
    y2 = x.clone()
    dah.rmsnorm(y2, w, y=y2)          # in place
    torch.cuda.synchronize()
    ref = L.rmsnorm(x.cpu().numpy(), w.cpu().numpy())
    err = np.abs(y.cpu().numpy() - ref)
    assert np.all(err <= 1e-6 * np.max(np.abs(ref), axis=1, keepdims=True)), float(err.max())
    assert torch.equal(y2, y)


@pytest.mark.parametrize("T,inter", [(1, 3072), (64, 3072), (256, 9728 // 4 * 4)])
def test_silu_mul_parity(T, inter):
    import torch
    dah = _dah()
    gu = _rand((T, 2 * inter), T + inter, 3.0)
    gu[0, :8] = torch.tensor([0.0, -30.0, 30.0, -88.0, 1e-6, -1e-6, 10.0, -10.0], device="cuda")
    act = dah.silu_mul(gu)
    torch.cuda.synchronize()
    ref = L.silu_mul(gu.cpu().numpy())
    err = np.abs(act.cpu().numpy() - ref)
    assert np.all(err <= 2e-6 * np.abs(ref) + 1e-30), float(np.max(err / (np.abs(ref) + 1e-30)))


@pytest.mark.parametrize("T,N,K", [(1, 1024, 2048), (48, 1024, 3072), (256, 1024, 3072),
                                   (300, 6144, 1024), (1000, 4096, 1024)])
def test_linear_residual_parity(T, N, K):
    import torch
    dah = _dah()
    x = _rand((T, K), T + K)
    w = (_rand((N, K), N + K) / np.sqrt(K)).to(torch.bfloat16)
    r = _rand((T, N), T + N + K)
    y = torch.empty_like(r)
    lib = dah.lib()
    dah.check(lib.dah_linear_residual(x.data_ptr(), w.data_ptr(), r.data_ptr(), T, N, K,
                                      y.data_ptr(), None), "dah_linear_residual")
    r2 = r.clone()
    dah.check(lib.dah_linear_residual(x.data_ptr(), w.data_ptr(), r2.data_ptr(), T, N, K,
                                      r2.data_ptr(), None), "dah_linear_residual")   # in place
    torch.cuda.synchronize()
    xr, wb, rr = x.cpu().numpy(), _bits(w), r.cpu().numpy()
    ref = P.linear(xr, wb) + rr
    bound = 2.0 ** -16 * P.linear(np.abs(xr), np.abs(O.bf16_bits_to_f64(wb)), "f64") + \
        2.0 ** -23 * np.abs(ref) + 1e-30
    assert np.all(np.abs(y.cpu().numpy() - ref) <= bound)
    assert torch.equal(r2, y)


@pytest.mark.parametrize("N,K", [(6144, 1024), (4096, 2560), (192, 256)])
@pytest.mark.parametrize("T", [1, 7, 17, 33, 256, 300, 1000])
def test_rmsnorm_linear_parity(T, N, K):
    """dah_rmsnorm_linear: the product of the RMS-normed rows (sum of squares
    accumulated in the product, 1/rms on the output rows) against the
    oracle's rmsnorm then linear, on both product kernels.  Gate: the
    product bound of the normed input plus float32 rounding of the norm."""
    import torch
    dah = _dah()
    x = _rand((T, K), 3 * T + K, 2.0)
    g = 1.0 + 0.1 * _rand((K,), K)
    w = (_rand((N, K), N + K) / np.sqrt(K)).to(torch.bfloat16)
    y = torch.full((T + 1, N), float("nan"), device="cuda")
    lib = dah.lib()
    dah.check(lib.dah_rmsnorm_linear(x.data_ptr(), g.data_ptr(), 1e-6, w.data_ptr(), T, N, K,
                                     y.data_ptr(), None), "dah_rmsnorm_linear")
    torch.cuda.synchronize()
    assert torch.isnan(y[T]).all(), "wrote past the output"
    xn = L.rmsnorm(x.cpu().numpy(), g.cpu().numpy())
    wb = _bits(w)
    ref = P.linear(xn, wb)
    absw = np.abs(O.bf16_bits_to_f64(wb))
    bound = (2.0 ** -16 + 2e-6) * P.linear(np.abs(xn), absw, "f64") + 1e-30
    err = np.abs(y[:T].cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    _print(f"[rmsnorm_linear] T={T} N={N} K={K} kernel {dah.linear_kernel(T, N, K)}: "
           f"{float(np.max(err / bound)):.3f} of bound")


@pytest.mark.parametrize("inter,K,norm", [(3072, 1024, True), (1280, 2560, True),
                                          (96, 256, True), (3072, 1024, False)])
@pytest.mark.parametrize("T", [1, 7, 17, 33, 256, 300, 1000])
def test_rmsnorm_swiglu_parity(T, inter, K, norm):
    """dah_rmsnorm_swiglu: the RMS-normed rows' product with the gate and up
    rows, the activation applied in the store, against the oracle's rmsnorm,
    linear and silu_mul, on both product kernels.  Gate: with e the product
    bound of the normed input for each of gate and up (as for
    dah_rmsnorm_linear), act = silu(g) u moves by at most
    1.1 e_g |u| + |silu(g)| e_u + 1.1 e_g e_u (|silu'| <= 1.1), plus the
    float32 rounding of the activation (2e-6 of |act|)."""
    import torch
    dah = _dah()
    x = _rand((T, K), 5 * T + K, 2.0)
    g = (1.0 + 0.1 * _rand((K,), K + 1)) if norm else None
    w = (_rand((2 * inter, K), inter + K) / np.sqrt(K)).to(torch.bfloat16)
    act = torch.full((T + 1, inter), float("nan"), device="cuda")
    dah.rmsnorm_swiglu(x, g, w, act=act[:T])
    torch.cuda.synchronize()
    assert torch.isnan(act[T]).all(), "wrote past the output"
    xn = L.rmsnorm(x.cpu().numpy(), g.cpu().numpy()) if norm else x.cpu().numpy()
    wb = _bits(w)
    gu = P.linear(xn, wb)
    ref = L.silu_mul(gu)
    eb = (2.0 ** -16 + 2e-6) * P.linear(np.abs(xn), np.abs(O.bf16_bits_to_f64(wb)), "f64")
    gate, up = gu[:, :inter], gu[:, inter:]
    e_g, e_u = eb[:, :inter], eb[:, inter:]
    silu = gate / (1.0 + np.exp(-gate))
    bound = 1.1 * e_g * np.abs(up) + np.abs(silu) * e_u + 1.1 * e_g * e_u + \
        2e-6 * np.abs(ref) + 1e-30
    err = np.abs(act[:T].cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err / bound))
    _print(f"[rmsnorm_swiglu] T={T} I={inter} K={K} norm={norm}: "
           f"{float(np.max(err / bound)):.3f} of bound")


def _layer_case(name, H):
    w = dataclasses.replace(W.WORKLOADS[name], num_heads=H)
    t, seq_lens, table, _ = build_layer(w)
    p = W.make_layer_weights(w, 0, "cuda")
    return w, t, seq_lens, table, p


@pytest.mark.parametrize("name,H", [("ragged_f32_b6", 16), ("ragged_f32_b6", 40),
                                    ("b256_s2048", 16), ("b256_s2048_h64", 64)])
def test_decoder_layer_parity(name, H):
    import torch
    dah = _dah()
    w, t, seq_lens, table, p = _layer_case(name, H)
    _print(f"[layer] {name} H={H}")
    every = list(range(w.batch))
    snap = host_snapshot(t, seq_lens, table, every)
    weights = {n: p[n] for n in dah.LAYER_WEIGHTS}
    y = dah.decoder_layer_step(p["x"], weights, t["k_pool"], t["v_pool"], t["block_table"],
                               t["seq_lens"], int(seq_lens.max()), rope_theta=w.rope_theta)
    torch.cuda.synchronize()
    wnp = {n: (_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy())
           for n, v in weights.items()}
    x_host = p["x"].cpu().numpy()
    ref = oracle_map(lambda rows: L.decoder_layer(
        x_host, wnp, snap["k_pool"], snap["v_pool"], snap["block_table"], snap["seq_lens"],
        w.cache_dtype, num_heads=H, theta=w.rope_theta, batch_indices=rows), w.batch, chunk=8)
    tol = 1e-4 if w.cache_dtype == "f32" else 2e-2
    e_abs, e_rel = gates(y.cpu().numpy().astype(np.float64), ref["y"], None, tol,
                         label=f"{name} y")
    _print(f"  y max abs {e_abs:.2e}  rel-to-max {e_rel:.2e}")


def test_layer_rejects_before_launching():
    """Bad attention arguments are caught before the first kernel: the output
    buffer stays untouched."""
    import torch
    dah = _dah()
    w, t, seq_lens, table, p = _layer_case("tiny_f32_b2", 16)
    weights = {n: p[n] for n in dah.LAYER_WEIGHTS}
    y = torch.full_like(p["x"], 7.0)
    with pytest.raises(dah.DahError):
        dah.decoder_layer_step(p["x"], weights, t["k_pool"], t["v_pool"], t["block_table"],
                               t["seq_lens"], 10_000, y=y)    # max_seq_len past the table
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


@pytest.mark.parametrize("name", ["b256_s2048", "ragged_b32"])
def test_layer_under_graph_replay(name):
    """decoder_layer_step captured in one HIP graph (per-sequence plan at
    B=256; fixed splits with the combine launch at B=32 ragged): every
    replay, with eager work and synchronisations between replays, equals the
    eager result bit for bit.  The cache is restored before each run."""
    import torch
    dah = _dah()
    w, t, seq_lens, table, p = _layer_case(name, 16)
    L = int(seq_lens.max())
    weights = {n: p[n] for n in dah.LAYER_WEIGHTS}
    inter = p["w_down"].shape[1]
    ws = torch.empty(dah.layer_workspace_bytes(w.batch, w.hidden, inter, L), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(p["x"])
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def layer():
        dah.decoder_layer_step(p["x"], weights, t["k_pool"], t["v_pool"], t["block_table"],
                               t["seq_lens"], L, y=y, workspace=ws)

    def restore():
        t["k_pool"].copy_(k0)
        t["v_pool"].copy_(v0)

    layer()
    torch.cuda.synchronize()
    want_y, want_k = y.clone(), t["k_pool"].clone()
    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer()
    torch.cuda.synchronize()
    for i in range(3):
        restore()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want_y), f"replay {i}: y differs"
        assert torch.equal(t["k_pool"], want_k), f"replay {i}: cache differs"
        _ = (p["x"] * 2).sum().item()   # eager work between replays
