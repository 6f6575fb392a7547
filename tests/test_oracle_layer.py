"""Pins of the decoder-layer oracle (oracle/layer.py): closed forms of the
hidden-size RMSNorm, silu against SciPy's logistic function, and the
residual structure of the layer (zero output projections leave the stream
unchanged, exactly)."""
import numpy as np
import pytest

from oracle import decode_attention as O
from oracle import layer as L


def test_rmsnorm_closed_forms():
    # a constant row c: mean square c^2, so y = c / sqrt(c^2 + eps) * w
    c, eps = 0.75, 1e-6
    w = np.linspace(0.5, 1.5, 1024)
    y = L.rmsnorm(np.full((2, 1024), c), w, eps)
    assert np.allclose(y, c / np.sqrt(c * c + eps) * w, rtol=1e-15, atol=0)
    # one-hot row of height a over H = 1024: mean square a^2 / 1024
    x = np.zeros((1, 1024))
    x[0, 7] = 3.0
    y = L.rmsnorm(x, np.ones(1024), 0.0)
    assert y[0, 7] == pytest.approx(3.0 / np.sqrt(9.0 / 1024), rel=1e-15)
    assert np.count_nonzero(y) == 1
    # the divisor is the row width (1024 here, 2560 for 4B), not 128
    x = np.ones((1, 2560))
    assert L.rmsnorm(x, np.ones(2560), 0.0)[0, 0] == pytest.approx(1.0, rel=1e-15)


def test_silu_matches_scipy_logistic():
    special = pytest.importorskip("scipy.special")
    z = np.linspace(-30, 30, 2001)
    gu = np.concatenate([z[None], np.ones((1, z.size))], axis=1)
    act = L.silu_mul(gu)[0]
    assert np.allclose(act, z * special.expit(z), rtol=1e-14, atol=1e-300)
    assert L.silu_mul(np.array([[0.0, 5.0]]))[0, 0] == 0.0          # silu(0) = 0
    # the up half multiplies: doubling it doubles the output
    r = np.random.default_rng(0).standard_normal((3, 12))
    r2 = r.copy()
    r2[:, 6:] *= 2
    assert np.allclose(L.silu_mul(r2), 2 * L.silu_mul(r), rtol=1e-15)


def _weights(rng, H=16, hidden=256, inter=512, zero_o=False, zero_down=False):
    def bf(shape, scale):
        v = O.round_to_bf16(rng.standard_normal(shape) * scale)
        return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = {
        "w_in": 1 + 0.1 * rng.standard_normal(hidden),
        "w_qkv": bf(((H + 16) * 128, hidden), hidden ** -0.5),
        "q_gain": 1 + 0.1 * rng.standard_normal(128), "k_gain": 1 + 0.1 * rng.standard_normal(128),
        "w_o": bf((hidden, H * 128), (H * 128) ** -0.5),
        "w_post": 1 + 0.1 * rng.standard_normal(hidden),
        "w_gate_up": bf((2 * inter, hidden), hidden ** -0.5),
        "w_down": bf((hidden, inter), inter ** -0.5),
    }
    if zero_o:
        w["w_o"][:] = 0
    if zero_down:
        w["w_down"][:] = 0
    return w


def _cache(rng, B, L0):
    pages = B * (-(-L0 // 16)) + 4
    kp = rng.standard_normal((pages, 8, 16, 128)).astype(np.float32)
    vp = rng.standard_normal((pages, 8, 16, 128)).astype(np.float32)
    n = -(-L0 // 16)
    table = np.arange(B * n, dtype=np.int32).reshape(B, n)
    return kp, vp, table, np.full(B, L0)


def test_zero_output_projections_leave_the_stream_unchanged():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 256))
    kp, vp, table, lens = _cache(rng, 3, 20)
    w = _weights(rng, zero_o=True, zero_down=True)
    res = L.decoder_layer(x, w, kp, vp, table, lens, "f32")
    assert np.array_equal(res["x1"], x) and np.array_equal(res["y"], x)
    # with only the MLP zeroed, y is the attention residual exactly
    w = _weights(np.random.default_rng(2), zero_down=True)
    res = L.decoder_layer(x, w, kp, vp, table, lens, "f32")
    assert np.array_equal(res["y"], res["x1"]) and not np.array_equal(res["x1"], x)


def test_layer_wires_the_nodes_in_order():
    """The layer's intermediates are the node functions applied in the spec's
    order: the norm feeds the projection, the residual adds o_proj's output,
    and the MLP reads the post-attention norm (checked on a case where each
    stage changes the values)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 256))
    kp, vp, table, lens = _cache(rng, 2, 33)
    w = _weights(rng)
    res = L.decoder_layer(x, w, kp, vp, table, lens, "f32")
    assert np.allclose(np.sqrt(np.mean((res["h"] / w["w_in"]) ** 2, axis=-1)), 1.0, atol=1e-6)
    assert np.allclose(np.sqrt(np.mean((res["h2"] / w["w_post"]) ** 2, axis=-1)), 1.0, atol=1e-6)
    assert res["gu"].shape == (2, 1024) and res["act"].shape == (2, 512)
    assert np.allclose(res["act"], L.silu_mul(res["gu"]))
    assert not np.allclose(res["y"], res["x1"])
