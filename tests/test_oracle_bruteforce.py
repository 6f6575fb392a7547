"""Brute-force pin of the float64 oracle: the whole step evaluated with mpmath
at 50 significant digits on tiny inputs.

The mpmath side is written directly from the node formulas of the
"Qwen3-0.6B" Model Spec page ("Compute-graph nodes": attn.qk_norm,
attn.rope, attn.core) with plain loops, independently of the oracle's
vectorised NumPy.  The oracle must agree to ~1e-13 relative; a wrong index,
sign or normaliser would show up at 1e-6 or worse ("Model conformance" page,
note on typical error sizes).
"""
import numpy as np
import pytest

mpmath = pytest.importorskip("mpmath")
from mpmath import mp, mpf  # noqa: E402

from oracle import decode_attention as O  # noqa: E402


def _mp_norm_rope(x, w, eps, pos, theta):
    """One head: RMSNorm over 128 dims, then rotate pairs (i, i+64)."""
    d = len(x)
    ms = sum(xi * xi for xi in x) / d
    inv = 1 / mp.sqrt(ms + eps)
    y = [x[i] * inv * w[i] for i in range(d)]
    out = list(y)
    for i in range(d // 2):
        ang = pos * mp.power(theta, mpf(-2 * i) / d)
        c, s = mp.cos(ang), mp.sin(ang)
        out[i] = y[i] * c - y[i + d // 2] * s
        out[i + d // 2] = y[i] * s + y[i + d // 2] * c
    return out


def _mp_decode(qh, ks, vs):
    d = len(qh)
    scale = 1 / mp.sqrt(d)
    z = [sum(qh[j] * k[j] for j in range(d)) * scale for k in ks]
    m = max(z)
    e = [mp.exp(zi - m) for zi in z]
    tot = sum(e)
    return [sum(e[s] * vs[s][j] for s in range(len(ks))) / tot for j in range(d)]


@pytest.mark.parametrize("seq_len,seed,H,theta", [(1, 0, 16, 1e6), (5, 1, 16, 1e6), (17, 2, 16, 1e6),
                                                   (33, 3, 16, 1e6), (9, 4, 32, 5e6), (18, 5, 40, 1e6),
                                                   (3, 6, 64, 1e6)])
def test_step_matches_50_digit_brute_force(seq_len, seed, H, theta):
    mp.dps = 50
    G = H // 8
    r = np.random.default_rng([99, seed])
    q = r.standard_normal((1, H, 128))
    kn = r.standard_normal((1, 8, 128)) * 2
    vn = r.standard_normal((1, 8, 128))
    wq = 1 + 0.1 * r.standard_normal(128)
    wk = 1 + 0.1 * r.standard_normal(128)
    npages = -(-seq_len // 16)
    pool_k = r.standard_normal((npages + 2, 8, 16, 128)).astype(np.float32)
    pool_v = r.standard_normal((npages + 2, 8, 16, 128)).astype(np.float32)
    table = r.permutation(npages + 2)[:npages].astype(np.int32)[None]
    eps = 1e-6
    res = O.decode_step(q, kn, vn, wq, wk, pool_k, pool_v, table, np.array([seq_len]), "f32",
                        eps=eps, theta=theta)

    pos = seq_len - 1
    to_mp = lambda a: [mpf(float(t)) for t in a]  # noqa: E731
    wq_m, wk_m = to_mp(wq), to_mp(wk)
    q_rot = [_mp_norm_rope(to_mp(q[0, h]), wq_m, mpf(eps), pos, mpf(theta)) for h in range(H)]
    k_rot = [_mp_norm_rope(to_mp(kn[0, g]), wk_m, mpf(eps), pos, mpf(theta)) for g in range(8)]
    for h in range(H):
        got = res["q_out"][0, h]
        want = np.array([float(t) for t in q_rot[h]])
        assert np.max(np.abs(got - want)) <= 1e-13 * np.max(np.abs(want))
    for h in range(H):
        g = h // G
        ks, vs = [], []
        for s in range(seq_len):
            if s == pos:
                ks.append(k_rot[g]); vs.append(to_mp(vn[0, g]))
            else:
                page, slot = table[0, s // 16], s % 16
                ks.append(to_mp(pool_k[page, g, slot])); vs.append(to_mp(pool_v[page, g, slot]))
        want = np.array([float(t) for t in _mp_decode(q_rot[h], ks, vs)])
        got = res["o"][0, h]
        assert np.max(np.abs(got - want)) <= 1e-13 * max(1.0, np.max(np.abs(want))), h


def _mp_bf16_value(bits):
    """Value of a bfloat16 bit pattern from the format's fields: sign, 8-bit
    biased exponent, 7 stored fraction bits (normal numbers only here)."""
    bits = int(bits)
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    assert 0 < e < 0xFF, "test draws normal bfloat16 values only"
    return sign * (1 + mpf(frac) / 128) * mp.power(2, e - 127)


def _mp_round_bf16(x):
    """Nearest bfloat16 value of x (8 significant bits), ties to the even
    last bit, from the definition: with 2^(ex-1) <= |x| < 2^ex the spacing
    is 2^(ex-8); normal range only."""
    if x == 0:
        return mpf(0)
    _, ex = mp.frexp(x)
    assert -125 <= ex - 1 <= 127, "outside the normal bfloat16 range"
    spacing = mp.power(2, ex - 8)
    q = x / spacing
    f = mp.floor(q)
    r = q - f
    if r > mpf(1) / 2 or (r == mpf(1) / 2 and int(f) % 2 == 1):
        f += 1
    return f * spacing


@pytest.mark.parametrize("seq_len,seed,H", [(1, 10, 16), (6, 11, 16), (17, 12, 16), (21, 13, 64)])
def test_bf16_step_matches_50_digit_brute_force(seq_len, seed, H):
    """The step with a bfloat16 cache: the pool holds bfloat16 bit patterns,
    and the appended key and value are the nearest bfloat16 values of the
    exact roped key and of v_new.  The brute force decodes the stored bit
    patterns from the format's fields and rounds the exact 50-digit key
    itself, so the oracle's own bfloat16 path (its stored k_slot, v_slot,
    and the decode over them) is pinned, not only its float32 path."""
    mp.dps = 50
    G = H // 8
    r = np.random.default_rng([77, seed])
    q = r.standard_normal((1, H, 128))
    kn = r.standard_normal((1, 8, 128)) * 3
    vn = r.standard_normal((1, 8, 128))
    wq = 1 + 0.1 * r.standard_normal(128)
    wk = 1 + 0.1 * r.standard_normal(128)
    npages = -(-seq_len // 16)

    def bf16_bits(shape):     # normal bfloat16 patterns: the top half of float32 draws
        x = r.standard_normal(shape).astype(np.float32)
        x[x == 0] = 1.0
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    pool_k = bf16_bits((npages + 2, 8, 16, 128))
    pool_v = bf16_bits((npages + 2, 8, 16, 128))
    table = r.permutation(npages + 2)[:npages].astype(np.int32)[None]
    eps, theta = 1e-6, 1e6
    res = O.decode_step(q, kn, vn, wq, wk, pool_k, pool_v, table, np.array([seq_len]), "bf16",
                        eps=eps, theta=theta)

    pos = seq_len - 1
    to_mp = lambda a: [mpf(float(t)) for t in a]  # noqa: E731
    q_rot = [_mp_norm_rope(to_mp(q[0, h]), to_mp(wq), mpf(eps), pos, mpf(theta))
             for h in range(H)]
    k_store = [[_mp_round_bf16(t) for t in _mp_norm_rope(to_mp(kn[0, g]), to_mp(wk), mpf(eps),
                                                         pos, mpf(theta))] for g in range(8)]
    v_store = [[_mp_round_bf16(t) for t in to_mp(vn[0, g])] for g in range(8)]
    # the stored slot: exactly the nearest bfloat16 values
    want_k = np.array([[float(t) for t in row] for row in k_store])
    want_v = np.array([[float(t) for t in row] for row in v_store])
    assert np.array_equal(res["k_slot"][0], want_k)
    assert np.array_equal(res["v_slot"][0], want_v)
    for h in range(H):
        g = h // G
        ks, vs = [], []
        for s in range(seq_len):
            if s == pos:
                ks.append(k_store[g]); vs.append(v_store[g])
            else:
                page, slot = table[0, s // 16], s % 16
                ks.append([_mp_bf16_value(b) for b in pool_k[page, g, slot]])
                vs.append([_mp_bf16_value(b) for b in pool_v[page, g, slot]])
        want = np.array([float(t) for t in _mp_decode(q_rot[h], ks, vs)])
        got = res["o"][0, h]
        assert np.max(np.abs(got - want)) <= 1e-13 * max(1.0, np.max(np.abs(want))), h
