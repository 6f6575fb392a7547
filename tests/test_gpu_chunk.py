"""GPU parity of the chunk step (several new tokens per sequence, causal
within the chunk: chunked prefill and verification of drafted tokens),
through the C ABI, against the oracle's chunk_step.

With a bfloat16 cache the kernels run on the matrix cores (q as three bf16
terms in the one-tile kernel and two in the shared-page one, weights as
two), so the gates are the bf16 ones: max abs error 2e-2,
relative-to-max <= 1e-4, and q_out within 1e-5.  A float32 cache runs every
token as a VALU decode and gets the strict float32 gates: o and q_out within
1e-5, appended keys within 1e-5 of the exact values.  The appended keys must be
the round-to-nearest-even of the exact value (or its neighbour within float32
error of a midpoint) and the values exact.

Where an exact key element lies within float32 error of a bf16 midpoint,
both roundings are correct, and for a token that attends to only a few
positions the choice moves o by ~1e-4.  The oracle is therefore also
evaluated with every such element rounded the other way (found from the
exact values alone), and a token's gate is 1e-4 x max|o| plus the spread
between the two oracle results.
"""
import numpy as np
import pytest

from dah_testlib import bf16_alternative, check_rounded, cuda_available, gates, pool_to_numpy
from inputs import workloads as W
from oracle import decode_attention as O

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _dah():
    import decode_attention_head_amd as dah
    return dah


def _print(*a):
    print(*a, flush=True)


def _snapshot(t, table, seq_lens, cu, seqs):
    """Host copies of the pages and tokens of the selected sequences, with a
    compact pool and remapped block table (taken before the step runs)."""
    import torch
    pages, rows, toks = [], [], []
    at = 0
    for b in seqs:
        n = W.pages_for(int(seq_lens[b]))
        pages.append(table[b, :n])
        rows.append(np.arange(at, at + n))
        at += n
        toks.append(np.arange(cu[b], cu[b + 1]))
    idx = torch.from_numpy(np.concatenate(pages).astype(np.int64)).to(t["k_pool"].device)
    mini = np.zeros((len(seqs), max(len(r) for r in rows)), np.int32)
    for i, r in enumerate(rows):
        mini[i, :len(r)] = r
    tok = np.concatenate(toks).astype(np.int64)
    sel = torch.from_numpy(tok).to(t["q"].device)
    counts = [int(cu[b + 1] - cu[b]) for b in seqs]
    return {
        "k_pool": pool_to_numpy(t["k_pool"].index_select(0, idx)),
        "v_pool": pool_to_numpy(t["v_pool"].index_select(0, idx)),
        "block_table": mini, "seq_lens": np.asarray(seq_lens)[list(seqs)].astype(np.int64),
        "cu": np.concatenate([[0], np.cumsum(counts)]).astype(np.int64),
        "q": t["q"].index_select(0, sel).cpu().numpy(),
        "k_new": t["k_new"].index_select(0, sel).cpu().numpy(),
        "v_new": t["v_new"].index_select(0, sel).cpu().numpy(),
        "q_gain": t["q_gain"].cpu().numpy(), "k_gain": t["k_gain"].cpu().numpy(),
        "tokens": tok,
        "cache_dtype": "f32" if t["k_pool"].dtype == torch.float32 else "bf16",
    }


def _oracle(s, theta=1e6, k_stored=None):
    return O.chunk_step(s["q"], s["k_new"], s["v_new"], s["q_gain"], s["k_gain"], s["k_pool"],
                        s["v_pool"], s["block_table"], s["seq_lens"], s["cu"], s["cache_dtype"], theta=theta,
                        k_stored=k_stored)


def _check_o(o_gpu, s, ref, theta, label):
    """The gates on o with the admissible-rounding spread (module docstring)."""
    _, k_exact = O.norm_rope(s["q"], s["k_new"], s["q_gain"], s["k_gain"],
                             np.asarray(ref["pos"]) + 1, theta=theta)
    _, k_alt, flagged = bf16_alternative(k_exact)
    spread = np.zeros(len(ref["o"]))
    if flagged.any():
        alt = _oracle(s, theta, k_stored=k_alt)
        spread = np.max(np.abs(alt["o"] - ref["o"]), axis=(1, 2))
    o_gpu = np.asarray(o_gpu, np.float64)
    scale = float(np.max(np.abs(ref["o"])))
    err = np.max(np.abs(o_gpu - ref["o"]), axis=(1, 2))
    assert np.all(np.isfinite(o_gpu)), label
    bad = err > 1e-4 * scale + spread
    assert not bad.any(), (f"{label}: tokens {np.nonzero(bad)[0][:8]} exceed 1e-4 x max|o| + "
                           f"spread; worst {float(np.max(err - spread)) / scale:.3g} rel")
    assert float(np.max(err)) <= 2e-2, label
    return float(np.max(err)), float(np.max(err) / scale), int(flagged.sum())


def _slots(t, table, seq_lens, cu, seqs):
    """(k, v) the cache holds at every chunk position of the selected sequences."""
    import torch
    ks, vs = [], []
    for b in seqs:
        n = int(cu[b + 1] - cu[b])
        for i in range(n):
            pos = int(seq_lens[b]) - n + i
            page, slot = int(table[b, pos // 16]), pos % 16
            ks.append(t["k_pool"][page, :, slot].to(torch.float64).cpu().numpy())
            vs.append(t["v_pool"][page, :, slot].to(torch.float64).cpu().numpy())
    return np.stack(ks), np.stack(vs)


def _run(t, cu, seq_lens, max_chunk, theta=1e6):
    import torch
    dah = _dah()
    q_out, o = dah.chunk_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                   t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                   t["cu_tokens"], max_chunk, int(np.max(seq_lens)),
                                   rope_theta=theta)
    torch.cuda.synchronize()
    return q_out, o


@pytest.mark.parametrize("H", [16, 32, 40, 64])
@pytest.mark.parametrize("theta", [1e6, 5e6])
def test_small_chunks_every_token(H, theta):
    """Chunks of 1, 4, 7, 16, 19 and 33 tokens after 0, 3, 16, 30, 100 and
    9 cached positions (tiles of 16/G tokens with ragged tails, chunks that
    start mid-page, cross pages and start at position 0)."""
    lens_old, chunks = [0, 3, 16, 30, 100, 9], [1, 4, 7, 16, 19, 33]
    t, table, seq_lens, cu = W.make_chunk_inputs(lens_old, chunks, H, "bf16", 11 + H, "cuda",
                                                 pool_pages=64)
    seqs = list(range(len(chunks)))
    snap = _snapshot(t, table, seq_lens, cu, seqs)
    q_out, o = _run(t, cu, seq_lens, max(chunks), theta)
    ref = _oracle(snap, theta)
    e_q = float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"])))
    assert e_q <= 1e-5, f"q_out {e_q:.3g}"
    k_slot, v_slot = _slots(t, table, seq_lens, cu, seqs)
    _, k_exact = O.norm_rope(snap["q"], snap["k_new"], snap["q_gain"], snap["k_gain"],
                             np.array(ref["pos"]) + 1, theta=theta)
    check_rounded(k_slot, k_exact)
    assert np.array_equal(v_slot, ref["v_slot"])
    e_abs, e_rel, nflag = _check_o(o.cpu().numpy(), snap, ref, theta, f"H={H}")
    _print(f"[chunk] H={H} theta={theta:g}: q_out {e_q:.2e}  o {e_abs:.2e} rel {e_rel:.2e} "
           f"({nflag} near-midpoint keys)")


@pytest.mark.parametrize("H", [16, 40, 64])
def test_f32_cache_chunks_every_token(H):
    """A float32 cache (every token a decode over its own prefix): the same
    ragged chunks as above, against the oracle at the float32 gates."""
    lens_old, chunks = [0, 3, 16, 30, 100, 9], [1, 4, 7, 16, 19, 33]
    t, table, seq_lens, cu = W.make_chunk_inputs(lens_old, chunks, H, "f32", 21 + H, "cuda",
                                                 pool_pages=64)
    seqs = list(range(len(chunks)))
    snap = _snapshot(t, table, seq_lens, cu, seqs)
    q_out, o = _run(t, cu, seq_lens, max(chunks))
    ref = _oracle(snap)
    e_q = float(np.max(np.abs(q_out.cpu().numpy() - ref["q_out"])))
    assert e_q <= 1e-5, f"q_out {e_q:.3g}"
    k_slot, v_slot = _slots(t, table, seq_lens, cu, seqs)
    _, k_exact = O.norm_rope(snap["q"], snap["k_new"], snap["q_gain"], snap["k_gain"],
                             np.array(ref["pos"]) + 1)
    assert np.max(np.abs(k_slot - k_exact)) <= 1e-5
    assert np.array_equal(v_slot, ref["v_slot"])
    e_abs, e_rel = gates(o.cpu().numpy().astype(np.float64), ref["o"], None, 1e-5,
                         label=f"f32 H={H}")
    _print(f"[chunk f32] H={H}: q_out {e_q:.2e}  o {e_abs:.2e} rel {e_rel:.2e}")


@pytest.mark.parametrize("name,lens_old,chunk,B,H", [
    ("verify", 2044, 4, 64, 16), ("verify", 2044, 4, 64, 64),
    ("prefill", 0, 1024, 4, 16), ("prefill_after_context", 3000, 512, 4, 40),
    ("prefill_32_heads", 700, 512, 4, 32)])
def test_large_chunks(name, lens_old, chunk, B, H):
    """Verification of 4 drafted tokens over 2,044 cached positions at B=64,
    and chunked prefill of 512-1,024 tokens at 16, 32 and 40 heads (the
    prefill cases on two 16-column blocks per wave): every token of every
    sequence."""
    rng = np.random.default_rng(B + chunk)
    olds = [lens_old + int(x) for x in rng.integers(0, 8, B)] if lens_old else [0] * B
    t, table, seq_lens, cu = W.make_chunk_inputs(olds, [chunk] * B, H, "bf16", 100 + H, "cuda")
    seqs = list(range(B))
    snap = _snapshot(t, table, seq_lens, cu, seqs)
    q_out, o = _run(t, cu, seq_lens, chunk)
    ref = _oracle(snap)
    tok = snap["tokens"]
    e_q = float(np.max(np.abs(q_out.cpu().numpy()[tok] - ref["q_out"])))
    assert e_q <= 1e-5
    e_abs, e_rel, nflag = _check_o(o.cpu().numpy()[tok], snap, ref, 1e6, name)
    _print(f"[chunk {name}] B={B} H={H}: o {e_abs:.2e} rel {e_rel:.2e} ({nflag} near-midpoint keys)")


def test_one_token_chunks_match_the_decode_step():
    """A chunk of one token per sequence is the decode step: the same o up
    to the two kernels' rounding (the decode here runs on the same matrix-
    core form; both are gated against the oracle elsewhere)."""
    import torch
    dah = _dah()
    lens_old = [5, 16, 200, 1000]
    t, table, seq_lens, cu = W.make_chunk_inputs(lens_old, [1] * 4, 16, "bf16", 5, "cuda",
                                                 pool_pages=128)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q_c, o_c = _run(t, cu, seq_lens, 1)
    kc, vc = t["k_pool"].clone(), t["v_pool"].clone()
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    q_d, o_d = dah.decode_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                    t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                    int(seq_lens.max()), num_splits=1)
    torch.cuda.synchronize()
    torch.testing.assert_close(q_c, q_d, rtol=0, atol=1e-6)
    torch.testing.assert_close(o_c, o_d, rtol=0, atol=2.0 ** -16 * float(o_d.abs().max()))
    assert torch.equal(vc, t["v_pool"])


def test_later_tokens_leave_earlier_outputs_bit_identical():
    """forward_causal: changing the last token of a chunk changes no earlier
    token's output, bit for bit (the kernel's masking, not just rounding)."""
    import torch
    lens_old, chunks = [40, 0], [13, 9]
    t, table, seq_lens, cu = W.make_chunk_inputs(lens_old, chunks, 32, "bf16", 9, "cuda",
                                                 pool_pages=32)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    _, o1 = _run(t, cu, seq_lens, 13)
    o1 = o1.clone()
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    for last in (12, 21):
        t["q"][last] += 3.0
        t["k_new"][last] *= -2.0
        t["v_new"][last] += 5.0
    _, o2 = _run(t, cu, seq_lens, 13)
    assert torch.equal(o2[:12], o1[:12]) and torch.equal(o2[13:21], o1[13:21])
    assert not torch.equal(o2[12], o1[12]) and not torch.equal(o2[21], o1[21])


@pytest.mark.parametrize("c,over,dt", [(3, False, "bf16"), (20, True, "bf16"),
                                       (3, False, "f32"), (20, True, "f32")])
def test_out_of_domain_sequences(c, over, dt):
    """seq_len < n_b or > max_seq_len (and n_b > max_chunk): NaN outputs,
    nothing appended; an empty chunk: nothing; other sequences unaffected.
    With a bfloat16 cache, chunks of 3 tokens take the one-tile kernel, of 20
    the shared-page one (three 8-token tiles, one workgroup per KV head); a
    float32 cache takes the per-token kernel."""
    import torch
    lens_old = [20, 20, 20, 20] + ([20] if over else [])
    chunks = [c, c, 0, c] + ([c + 4] if over else [])
    t, table, seq_lens, cu = W.make_chunk_inputs(lens_old, chunks, 16, dt, 13, "cuda",
                                                 pool_pages=32)
    max_seq_len = 20 + c
    t["seq_lens"][1] = 2                    # cannot hold its chunk
    t["seq_lens"][3] = max_seq_len + 37     # past max_seq_len
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    dah = _dah()
    q_out, o = dah.chunk_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                   t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                   t["cu_tokens"], c, max_seq_len)
    torch.cuda.synchronize()
    assert torch.isfinite(o[0:c]).all()
    assert torch.isnan(o[c:2 * c]).all() and torch.isnan(o[2 * c:3 * c]).all()
    if over:   # sequence 4 holds c + 4 > max_chunk tokens: all of them NaN
        assert torch.isnan(o[3 * c:]).all() and o.shape[0] == 4 * c + 4
    changed = (t["k_pool"] != k0).any(dim=3) | (t["v_pool"] != v0).any(dim=3)
    assert int(changed.sum()) == c * 8       # sequence 0's slots, 8 heads each


def test_out_of_domain_on_two_block_waves():
    """The same preconditions where the shared-page kernel takes two 16-column
    blocks per wave (64 sequences of 64-token chunks at 16 heads: eight tiles
    each, 512 workgroups): sequences that cannot hold their chunk, lie past
    max_seq_len or bring more than max_chunk tokens get NaN and no append;
    the others match the oracle."""
    import torch
    B, c = 64, 64
    chunks = [c] * (B - 1) + [c + 4]
    t, table, seq_lens, cu = W.make_chunk_inputs([100] * B, chunks, 16, "bf16", 17, "cuda")
    max_seq_len = 100 + c
    t["seq_lens"][1] = 2                    # cannot hold its chunk
    t["seq_lens"][3] = max_seq_len + 37     # past max_seq_len
    good = [0, 2, 5, 40, 62]
    snap = _snapshot(t, table, t["seq_lens"].cpu().numpy(), cu, good)
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q_out, o = _dah().chunk_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                                      t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                                      t["cu_tokens"], c, max_seq_len)
    torch.cuda.synchronize()
    for b in (1, 3, B - 1):                 # B - 1 holds c + 4 > max_chunk tokens
        assert torch.isnan(o[int(cu[b]):int(cu[b + 1])]).all(), b
    ok = torch.ones(o.shape[0], dtype=torch.bool, device=o.device)
    for b in (1, 3, B - 1):
        ok[int(cu[b]):int(cu[b + 1])] = False
    assert torch.isfinite(o[ok]).all()
    changed = (t["k_pool"] != k0).any(dim=3) | (t["v_pool"] != v0).any(dim=3)
    assert int(changed.sum()) == c * (B - 3) * 8    # every valid token's slot, 8 heads
    ref = _oracle(snap)
    _check_o(o.cpu().numpy()[snap["tokens"]], snap, ref, 1e6, "two-block waves")


@pytest.mark.parametrize("B,c", [(4, 4), (4, 20), (64, 64)])
def test_page_ids_outside_the_pool(B, c):
    """A block-table entry outside the pool (past num_pages, or negative)
    among a sequence's cached pages: every token of that sequence attends to
    it, so its outputs are NaN, nothing is read through it, and its chunk is
    still appended (the tokens' own pages are valid); the other sequences
    match the oracle.  Chunks of 4 tokens take the one-tile kernel, of 20
    the shared-page kernel with one block per wave, 64 at B = 64 two blocks
    per wave."""
    import torch
    t, table, seq_lens, cu = W.make_chunk_inputs([100] * B, [c] * B, 16, "bf16", 23 + c, "cuda")
    num_pages = t["k_pool"].shape[0]
    good = [0, 3] + ([10, B - 1] if B > 4 else [])
    snap = _snapshot(t, table, seq_lens, cu, good)
    t["block_table"][1, 2] = num_pages + 5
    t["block_table"][2, 0] = -1
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()
    q_out, o = _run(t, cu, seq_lens, c)
    for b in (1, 2):
        assert torch.isnan(o[int(cu[b]):int(cu[b + 1])]).all(), b
    changed = (t["k_pool"] != k0).any(dim=3) | (t["v_pool"] != v0).any(dim=3)
    assert int(changed.sum()) == c * B * 8      # every token appended, bad rows included
    ref = _oracle(snap)
    o_good = o.cpu().numpy()[snap["tokens"]]
    assert np.isfinite(o_good).all()
    _check_o(o_good, snap, ref, 1e6, f"page ids outside the pool, c={c}")


@pytest.mark.parametrize("chunk,H,dt", [(4, 16, "bf16"), (16, 16, "bf16"), (64, 64, "bf16"),
                                        (512, 16, "bf16"), (4, 40, "f32")])
def test_chunk_under_graph_replay(chunk, H, dt):
    """chunk_attn_step captured in one HIP graph -- the one-tile kernel, the
    shared-page kernel with 2 heads and with 1 head per workgroup, with one
    and with two 16-column blocks per wave, and the float32 path: every replay, with eager work and synchronisations between
    replays, equals the eager result bit for bit.  The cache is restored
    before each run, since the step appends to it."""
    import torch
    dah = _dah()
    B = 8
    lens_old = [100 + 37 * b for b in range(B)]
    t, table, seq_lens, cu = W.make_chunk_inputs(lens_old, [chunk] * B, H, dt, 31, "cuda")
    L = int(np.max(seq_lens))
    q_out, o = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def step():
        dah.chunk_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"],
                            t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                            t["cu_tokens"], chunk, L, q_out=q_out, o=o)

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
        q_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), f"replay {i}: o differs"
        assert torch.equal(q_out, want_q), f"replay {i}: q_out differs"
        assert torch.equal(t["k_pool"], want_k), f"replay {i}: cache differs"
        _ = (t["q"] * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("lens_old,chunk,B,H", [(0, 40960, 1, 16), (32768, 8192, 2, 64)])
def test_domain_maximum_chunks(lens_old, chunk, B, H):
    """The shape domain's largest chunks (Model Spec page, "At a glance": up
    to 40,960 new tokens and 40,960 positions): a whole 40,960-token prefill,
    and 8,192 tokens after 32,768 cached at 64 heads.  Every q_out against
    the oracle; o at sampled tokens (first, page edges, middle, last), the
    oracle evaluating those tokens alone, with the admissible-rounding
    spread of the module docstring."""
    import torch
    rng = np.random.default_rng(chunk + H)
    t, table, seq_lens, cu = W.make_chunk_inputs([lens_old] * B, [chunk] * B, H, "bf16",
                                                 300 + H, "cuda")
    seqs = list(range(B))
    snap = _snapshot(t, table, seq_lens, cu, seqs)
    q_out, o = _run(t, cu, seq_lens, chunk)
    picks = sorted({0, 1, 15, 16, chunk // 2, chunk - 17, chunk - 2, chunk - 1} |
                   {int(x) for x in rng.integers(0, chunk, 4)})
    only = {b: picks for b in seqs}
    ref = O.chunk_step(snap["q"], snap["k_new"], snap["v_new"], snap["q_gain"], snap["k_gain"],
                       snap["k_pool"], snap["v_pool"], snap["block_table"], snap["seq_lens"],
                       snap["cu"], "bf16", only=only)
    e_q = float(np.max(np.abs(q_out.cpu().numpy()[snap["tokens"]] - ref["q_out"])))
    assert e_q <= 1e-5, f"q_out {e_q:.3g}"
    _, k_exact = O.norm_rope(snap["q"], snap["k_new"], snap["q_gain"], snap["k_gain"],
                             np.repeat(seq_lens[seqs] - chunk, chunk) + np.tile(np.arange(chunk), B)
                             + 1)
    _, k_alt, flagged = bf16_alternative(k_exact)
    spread = np.zeros(len(ref["o"]))
    if flagged.any():
        alt = O.chunk_step(snap["q"], snap["k_new"], snap["v_new"], snap["q_gain"],
                           snap["k_gain"], snap["k_pool"], snap["v_pool"], snap["block_table"],
                           snap["seq_lens"], snap["cu"], "bf16", k_stored=k_alt, only=only)
        spread = np.max(np.abs(alt["o"] - ref["o"]), axis=(1, 2))
    rows = np.concatenate([int(cu[b]) + np.asarray(picks) for b in seqs])
    o_gpu = o.cpu().numpy()[rows].astype(np.float64)
    scale = float(np.max(np.abs(ref["o"])))
    err = np.max(np.abs(o_gpu - ref["o"]), axis=(1, 2))
    assert np.all(np.isfinite(o_gpu))
    assert np.all(err <= 1e-4 * scale + spread), (err / scale)
    assert float(np.max(err)) <= 2e-2
    _print(f"[chunk max] B={B} n={chunk} H={H}: q_out {e_q:.2e}  o rel-to-max "
           f"{float(np.max(err)) / scale:.2e} ({int(flagged.sum())} near-midpoint keys)")
