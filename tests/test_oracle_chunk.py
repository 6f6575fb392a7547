"""Pins of the oracle's chunk step (several new tokens per sequence, causal
within the chunk): against the single-token decode step (itself pinned
elsewhere), against the same tokens appended one decode step at a time,
against the causality theorem (forward_causal, "Supported models" page,
"Facts proved about the specs") and against a 50-digit brute force.
"""
import numpy as np
import pytest

from oracle import decode_attention as O


def _bits_of(x64):
    """bf16 bit patterns of bf16-exact float64 values."""
    b = np.asarray(x64, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


def _case(seed, lens_old, chunks, dtype="f32", H=16, pages=64):
    r = np.random.default_rng(seed)
    B = len(lens_old)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    N = int(cu[-1])
    seq_lens = np.array(lens_old) + np.array(chunks)
    mpp = max(1, -(-int(seq_lens.max()) // 16))
    perm = r.permutation(pages)
    table = np.zeros((B, mpp), np.int32)
    at = 0
    for b in range(B):
        need = -(-int(seq_lens[b]) // 16)
        table[b, :need] = perm[at:at + need]
        at += need
    shape = (pages, 8, 16, 128)
    if dtype == "f32":
        kp = r.standard_normal(shape).astype(np.float32)
        vp = r.standard_normal(shape).astype(np.float32)
    else:
        kp = _bits_of(O.round_to_bf16(r.standard_normal(shape)))
        vp = _bits_of(O.round_to_bf16(r.standard_normal(shape)))
    return dict(q=r.standard_normal((N, H, 128)), k_new=r.standard_normal((N, 8, 128)) * 2,
                v_new=r.standard_normal((N, 8, 128)), q_gain=1 + 0.1 * r.standard_normal(128),
                k_gain=1 + 0.1 * r.standard_normal(128), k_pool=kp, v_pool=vp, block_table=table,
                seq_lens=seq_lens, cu_tokens=cu)


def _chunk(c, dtype, **kw):
    return O.chunk_step(c["q"], c["k_new"], c["v_new"], c["q_gain"], c["k_gain"], c["k_pool"],
                        c["v_pool"], c["block_table"], c["seq_lens"], c["cu_tokens"], dtype, **kw)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_token_chunks_equal_the_decode_step(dtype):
    c = _case(1, [0, 5, 16, 40], [1, 1, 1, 1], dtype)
    res = _chunk(c, dtype)
    ref = O.decode_step(c["q"], c["k_new"], c["v_new"], c["q_gain"], c["k_gain"], c["k_pool"],
                        c["v_pool"], c["block_table"], c["seq_lens"], dtype)
    for key in ("q_out", "k_slot", "v_slot", "o"):
        assert np.allclose(res[key], ref[key], rtol=0, atol=1e-15), key
    assert list(res["pos"]) == [0, 5, 16, 40]


@pytest.mark.parametrize("dtype,H", [("f32", 16), ("bf16", 16), ("f32", 64)])
def test_chunk_equals_successive_decode_steps(dtype, H):
    """Appending the chunk's tokens one decode step at a time (each step
    writing its key and value into the pools before the next) gives the same
    outputs as the chunk step."""
    c = _case(2, [0, 3, 16, 30], [4, 7, 2, 19], dtype, H=H)
    res = _chunk(c, dtype)
    kp, vp = c["k_pool"].copy(), c["v_pool"].copy()
    outs = []
    for b in range(4):
        n = int(c["cu_tokens"][b + 1] - c["cu_tokens"][b])
        old = int(c["seq_lens"][b]) - n
        for i in range(n):
            t = int(c["cu_tokens"][b]) + i
            L = old + i + 1
            step = O.decode_step(c["q"][t:t + 1], c["k_new"][t:t + 1], c["v_new"][t:t + 1],
                                 c["q_gain"], c["k_gain"], kp, vp, c["block_table"][b:b + 1],
                                 np.array([L]), dtype)
            outs.append(step["o"][0])
            page, slot = O.cache_location(c["block_table"][b], L - 1)
            if dtype == "f32":
                kp[page, :, slot] = step["k_slot"][0]
                vp[page, :, slot] = step["v_slot"][0]
            else:
                kp[page, :, slot] = _bits_of(step["k_slot"][0])
                vp[page, :, slot] = _bits_of(step["v_slot"][0])
    # A float32 pool rounds the stepped keys and values to float32 where the
    # chunk step keeps them in float64 (the oracle's reading for a float32
    # cache); a bf16 pool holds exactly what both compute.
    tol = 1e-6 if dtype == "f32" else 1e-13
    err = float(np.max(np.abs(res["o"] - np.stack(outs))))
    assert err <= tol, err
    if dtype == "f32":
        assert err > 0   # the rounding is really there, so the check is not vacuous


def test_later_tokens_do_not_change_earlier_outputs():
    c = _case(3, [10, 0], [6, 5])
    base = _chunk(c, "f32")
    for t in (3, 5, 10):   # token 3 of sequence 0; its last token; sequence 1's last
        d = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
        d["q"][t] += 5.0
        d["k_new"][t] *= -3.0
        d["v_new"][t] += 7.0
        res = _chunk(d, "f32")
        b = 0 if t < 6 else 1
        first = int(c["cu_tokens"][b])
        assert np.array_equal(res["o"][first:t], base["o"][first:t])       # earlier: identical
        assert not np.array_equal(res["o"][t], base["o"][t])               # the token itself moves
        other = slice(6, 11) if b == 0 else slice(0, 6)
        assert np.array_equal(res["o"][other], base["o"][other])           # other sequence


def test_empty_chunks_and_bad_lengths():
    c = _case(4, [3, 8], [0, 2])
    res = _chunk(c, "f32")
    assert res["o"].shape == (2, 16, 128) and list(res["pos"]) == [8, 9]
    c["seq_lens"] = np.array([3, 1])   # fewer cached positions than chunk tokens
    with pytest.raises(ValueError):
        _chunk(c, "f32")


def test_chunk_brute_force_50_digits():
    mpmath = pytest.importorskip("mpmath")
    mp, mpf = mpmath.mp, mpmath.mpf
    mp.dps = 50
    c = _case(5, [2], [3])
    res = _chunk(c, "f32")
    to_mp = lambda a: [mpf(float(t)) for t in a]  # noqa: E731

    def norm_rope(x, w, pos):
        ms = sum(t * t for t in x) / 128
        inv = 1 / mp.sqrt(ms + mpf(1e-6))
        y = [x[i] * inv * w[i] for i in range(128)]
        out = list(y)
        for i in range(64):
            a = pos * mp.power(mpf(10) ** 6, mpf(-2 * i) / 128)
            out[i] = y[i] * mp.cos(a) - y[i + 64] * mp.sin(a)
            out[i + 64] = y[i] * mp.sin(a) + y[i + 64] * mp.cos(a)
        return out

    wq, wk = to_mp(c["q_gain"]), to_mp(c["k_gain"])
    keys = {g: [] for g in range(8)}
    vals = {g: [] for g in range(8)}
    for s in range(2):
        page, slot = O.cache_location(c["block_table"][0], s)
        for g in range(8):
            keys[g].append(to_mp(c["k_pool"][page, g, slot]))
            vals[g].append(to_mp(c["v_pool"][page, g, slot]))
    for i in range(3):
        pos = 2 + i
        for g in range(8):
            keys[g].append(norm_rope(to_mp(c["k_new"][i, g]), wk, pos))
            vals[g].append(to_mp(c["v_new"][i, g]))   # a float32 cache: the oracle keeps the value
        for h in range(16):
            qh = norm_rope(to_mp(c["q"][i, h]), wq, pos)
            ks, vs = keys[h // 2][:pos + 1], vals[h // 2][:pos + 1]
            z = [sum(qh[d] * k[d] for d in range(128)) / mp.sqrt(128) for k in ks]
            m = max(z)
            e = [mp.exp(t - m) for t in z]
            tot = sum(e)
            want = np.array([float(sum(e[s] * vs[s][d] for s in range(len(ks))) / tot)
                             for d in range(128)])
            assert np.max(np.abs(res["o"][i, h] - want)) <= 1e-13 * max(1.0, np.max(np.abs(want)))


def test_token_subset_matches_the_full_evaluation():
    """`only` evaluates o for chosen tokens: exactly the full step's rows for
    them (same arithmetic), with q_out and the stored slots of every token."""
    c = _case(9, [5, 0, 40], [7, 12, 3], "bf16")
    full = _chunk(c, "bf16")
    only = {0: [0, 6], 1: [11], 2: [1, 2]}
    part = _chunk(c, "bf16", only=only)
    rows = [0, 6, 7 + 11, 19 + 1, 19 + 2]
    assert np.array_equal(part["o"], full["o"][rows])
    assert np.array_equal(part["pos"], full["pos"][rows])
    for key in ("q_out", "k_slot", "v_slot"):
        assert np.array_equal(part[key], full[key])
    assert list(part["pos"]) == [5, 11, 11, 41, 42]
