"""Helpers shared by the GPU tests: build workloads on the device, copy the
pages a set of sequences needs to the host (before the GPU step modifies the
cache), and compare GPU results with the oracle.

Only input marshalling lives here: every expected value is computed by the
oracle from host copies of the generated inputs.  The oracle runs one
sequence at a time; ``oracle_map`` spreads those independent per-sequence
evaluations over host threads (NumPy and its BLAS release the interpreter
lock inside their array work), so that whole batches of the full-size
workloads can be compared element by element within seconds.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from inputs import workloads as W
from oracle import decode_attention as O


def cuda_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def build_layer(w: W.Workload, layer: int = 0, device="cuda", seq_lens=None):
    """Workload tensors on the device plus host-side structure."""
    seq_lens = W.make_seq_lens(w) if seq_lens is None else np.asarray(seq_lens, np.int32)
    table, num_pages = W.make_block_table(w, seq_lens)
    t = W.make_layer(w, layer, device, table=table, num_pages=num_pages, seq_lens=seq_lens)
    return t, seq_lens, table, num_pages


def pool_to_numpy(t):
    import torch
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_snapshot(t: dict, seq_lens, table, batch_indices):
    """Host copies of what the oracle needs for the sampled sequences: their
    pages (as a compact pool with a remapped block table) and the small
    per-sequence tensors."""
    import torch
    pages, rows = [], []
    at = 0
    for b in batch_indices:
        n = W.pages_for(int(seq_lens[b]))
        pages.append(table[b, :n])
        rows.append(np.arange(at, at + n))
        at += n
    idx = torch.from_numpy(np.concatenate(pages).astype(np.int64)).to(t["k_pool"].device)
    mpp = max(len(r) for r in rows)
    mini_table = np.zeros((len(batch_indices), mpp), np.int32)
    for i, r in enumerate(rows):
        mini_table[i, :len(r)] = r
    sel = torch.as_tensor(list(batch_indices), device=t["q"].device, dtype=torch.int64)
    snap = {
        "k_pool": pool_to_numpy(t["k_pool"].index_select(0, idx)),
        "v_pool": pool_to_numpy(t["v_pool"].index_select(0, idx)),
        "block_table": mini_table,
        "seq_lens": np.asarray(seq_lens)[list(batch_indices)].astype(np.int64),
        "q": t["q"].index_select(0, sel).cpu().numpy(),
        "k_new": t["k_new"].index_select(0, sel).cpu().numpy(),
        "v_new": t["v_new"].index_select(0, sel).cpu().numpy(),
        "q_gain": t["q_gain"].cpu().numpy(),
        "k_gain": t["k_gain"].cpu().numpy(),
    }
    return snap


def sample_batch(seq_lens, k: int, seed: int = 0):
    """Up to k sequence indices: the shortest, the longest and a seeded rest."""
    B = len(seq_lens)
    if B <= k:
        return list(range(B))
    rng = np.random.default_rng([seed, B])
    pick = {int(np.argmin(seq_lens)), int(np.argmax(seq_lens))}
    for b in rng.permutation(B):
        if len(pick) >= k:
            break
        pick.add(int(b))
    return sorted(pick)


def host_workers() -> int:
    """Host threads for the oracle: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_map(fn, n_rows: int, chunk: int = 2):
    """fn(rows) for consecutive chunks of the rows 0 .. n_rows-1 of a
    snapshot, on a pool of host threads; the results (arrays, or dicts of
    arrays, with the rows first) concatenated back in row order.  BLAS is
    held to one thread per call meanwhile, so the rows run side by side
    instead of oversubscribing the cores."""
    from threadpoolctl import threadpool_limits
    chunks = [list(range(i, min(n_rows, i + chunk))) for i in range(0, n_rows, chunk)]
    if not chunks:
        raise ValueError("oracle_map: no rows")
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=min(host_workers(), len(chunks))) as ex:
            parts = list(ex.map(fn, chunks))
    if isinstance(parts[0], dict):
        return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    return np.concatenate(parts)


def oracle_decode(snap, cache_dtype):
    """The oracle's decode over every sequence of a host snapshot."""
    return oracle_map(lambda rows: O.paged_decode_gqa(
        snap["q"], snap["k_pool"], snap["v_pool"], snap["block_table"], snap["seq_lens"],
        cache_dtype, batch_indices=rows), len(snap["seq_lens"]))


def oracle_step(snap, cache_dtype, eps=W.RMS_EPS, theta=W.ROPE_THETA):
    """The oracle's decode step over every sequence of a host snapshot
    (theta: the workload's RoPE base)."""
    return oracle_map(lambda rows: O.decode_step(
        snap["q"], snap["k_new"], snap["v_new"], snap["q_gain"], snap["k_gain"], snap["k_pool"],
        snap["v_pool"], snap["block_table"], snap["seq_lens"], cache_dtype, eps=eps, theta=theta,
        batch_indices=rows), len(snap["seq_lens"]))


def read_slots(t, seq_lens, table, batch_indices):
    """The K and V entries the step wrote (position seq_len - 1), as float64 [n,8,128]."""
    import torch
    ks, vs = [], []
    for b in batch_indices:
        pos = int(seq_lens[b]) - 1
        page = int(table[b, pos // W.PAGE_SIZE])
        slot = pos % W.PAGE_SIZE
        ks.append(t["k_pool"][page, :, slot, :].to(torch.float64).cpu().numpy())
        vs.append(t["v_pool"][page, :, slot, :].to(torch.float64).cpu().numpy())
    return np.stack(ks), np.stack(vs)


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    """Distance between adjacent bfloat16 values around |x| (normal range)."""
    _, ex = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(ex - 1, -126) - 7)


def check_rounded(stored: np.ndarray, exact: np.ndarray, fp32_rel: float = 4e-6):
    """A bfloat16 store of a float32 result: either the round-to-nearest of
    the exact value, or its neighbour when the exact value lies within the
    float32 computation error of a rounding midpoint.  That error scales with
    the head row's magnitude, not the element's: the rotation forms
    x_i cos - x_{i+64} sin, which can cancel to a value far smaller than its
    terms (a 1.4e-4 key element from O(0.3) inputs carries ~1e-8 of absolute
    float32 error)."""
    row_scale = np.max(np.abs(exact), axis=-1, keepdims=True)
    bound = 0.5 * bf16_spacing(exact) + fp32_rel * np.maximum(np.abs(exact), row_scale)
    err = np.abs(stored - exact)
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} stored values off by more than half a bf16 step; "
                           f"worst {float(err.max()):.3g}")
    exact_rne = O.round_to_bf16(exact)
    return float(np.mean(stored != exact_rne))


def gates(o_gpu, o_ref, v_mean_dev, tol_abs, tol_rel=1e-4, label=""):
    """The parity gates on o: max abs error <= tol_abs; relative-to-max error
    <= tol_rel; and the error under 1% of the distance to the trivial
    'uniform attention' answer (so a kernel that drops pages cannot pass)."""
    e_abs = O.max_abs_err(o_gpu, o_ref)
    e_rel = O.rel_to_max_err(o_gpu, o_ref)
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    assert e_abs <= tol_abs, f"{label}: max abs err {e_abs:.3g} > {tol_abs}"
    assert e_rel <= tol_rel, f"{label}: max rel-to-max err {e_rel:.3g} > {tol_rel}"
    if v_mean_dev is not None and v_mean_dev > 0:
        assert e_abs <= 0.01 * v_mean_dev, \
            f"{label}: err {e_abs:.3g} not under 1% of distance to uniform ({v_mean_dev:.3g})"
    return e_abs, e_rel


def distance_to_uniform(o_ref, snap, cache_dtype):
    """max |o_ref - mean_s v| over the snapshot's sequences and heads."""
    H = o_ref.shape[1]

    def worst(rows):
        out = []
        for i in rows:
            n = int(snap["seq_lens"][i])
            v = O.gather_sequence(snap["v_pool"], snap["block_table"][i], n, cache_dtype)
            mean = v.mean(axis=0)                             # [8,128]
            out.append(max(float(np.max(np.abs(o_ref[i, h] - mean[h // (H // 8)])))
                           for h in range(H)))
        return np.asarray(out)
    return float(np.max(oracle_map(worst, o_ref.shape[0])))


def bf16_alternative(exact: np.ndarray, fp32_rel: float = 4e-6):
    """(rne, alt, flagged): the round-to-nearest-even bf16 value of every
    exact element, the other admissible rounding where the exact value lies
    within float32 computation error (fp32_rel of its head row's magnitude)
    of a rounding midpoint, and the mask of those elements.  alt equals rne
    elsewhere.  Both come from the exact values only."""
    exact = np.asarray(exact, dtype=np.float64)
    rne = O.round_to_bf16(exact)
    spacing = bf16_spacing(exact)
    other = np.where(exact >= rne, rne + spacing, rne - spacing)  # neighbour across exact
    mid = 0.5 * (rne + other)
    row_scale = np.max(np.abs(exact), axis=-1, keepdims=True)
    flagged = np.abs(exact - mid) <= fp32_rel * np.maximum(np.abs(exact), row_scale)
    alt = np.where(flagged, O.round_to_bf16(other), rne)
    return rne, alt, flagged


def appended_slot_slack(snap, ref, x, w_qkv_bits, num_heads, cache_dtype):
    """Per (sequence, head, dim) bound on how far o may move because the
    appended key and value, which the device derives from its own float32
    projection of x, are stored in a bfloat16 cache as the other neighbour
    of the oracle's rounding.  Both stores are correct roundings of a value
    within the projection's error of a rounding midpoint.  Everything here
    comes from oracle values and the projection's error bound alone.

    The projection's elementwise bound is the projection gate,
    (2^-16 + 2e-6) sum_k |x w| (x enters the matrix cores as two bf16 terms).
    A value element within that bound of a midpoint may move by one bf16
    step s_v; a key element within the bound carried through the norm
    (2 ||e||/rms(k) max|gain|, plus float32 rounding of the norm and the
    rotation, 4e-6 of the row) may move by s_k, shifting the new token's
    score by at most dz = sum |q_d| s_k,d / sqrt(128).  With p the new
    token's softmax weight and o_old the attention over the older positions
    (o = (1 - p) o_old + p v_new), the move of o is at most
        p s_v + p (1 - p) dz e^dz (|v_new - o_old| + s_v).
    A float32 cache stores the device's value unrounded: no slack."""
    from oracle import projections as P
    o_ref = ref["o"]
    if cache_dtype != "bf16":
        return np.zeros_like(o_ref), 0
    n, H = o_ref.shape[0], num_heads
    G = H // 8
    nq, nkv = H * 128, 8 * 128
    absw = np.abs(O.bf16_bits_to_f64(w_qkv_bits))
    eb = (2.0 ** -16 + 2e-6) * P.linear(np.abs(np.asarray(x, np.float64)), absw, "f64")
    eb_k = eb[:, nq:nq + nkv].reshape(n, 8, 128)
    eb_v = eb[:, nq + nkv:].reshape(n, 8, 128)

    def flags(exact, err):
        rne = O.round_to_bf16(exact)
        s = bf16_spacing(exact)
        other = np.where(exact >= rne, rne + s, rne - s)
        return np.abs(exact - 0.5 * (rne + other)) <= err, s

    flag_v, s_v = flags(ref["v"], eb_v)
    _, k_exact = O.norm_rope(ref["q"], ref["k"], snap["q_gain"], snap["k_gain"], snap["seq_lens"])
    rms = np.sqrt(np.mean(ref["k"] ** 2, axis=-1, keepdims=True)) + 1e-30
    gain = float(np.max(np.abs(snap["k_gain"])))
    d_k = (2.0 * np.sqrt(np.sum(eb_k ** 2, axis=-1, keepdims=True)) / rms * gain +
           4e-6 * np.max(np.abs(k_exact), axis=-1, keepdims=True))
    flag_k, s_k = flags(k_exact, d_k)

    def p_new(rows):
        out = []
        for i in rows:
            L = int(snap["seq_lens"][i])
            k_old = O.gather_sequence(snap["k_pool"], snap["block_table"][i], L - 1, cache_dtype) \
                if L > 1 else np.zeros((0, 8, 128))
            k_all = np.concatenate([k_old, ref["k_slot"][i][None]], axis=0)
            out.append(O.attention_weights(ref["q_out"][i], k_all)[:, -1])
        return np.asarray(out)
    p = oracle_map(p_new, n)[:, :, None]                                 # [n,H,1]
    heads = np.arange(H) // G
    sv = (s_v * flag_v)[:, heads]                                         # [n,H,128]
    dz = np.sum(np.abs(ref["q_out"]) * (s_k * flag_k)[:, heads], axis=-1,
                keepdims=True) / np.sqrt(128.0)
    v_new = ref["v_slot"][:, heads]
    with np.errstate(divide="ignore", invalid="ignore"):
        o_old = np.where(p < 1.0, (o_ref - p * v_new) / (1.0 - p), v_new)
    slack = p * sv + p * (1.0 - p) * dz * np.exp(dz) * (np.abs(v_new - o_old) + sv)
    return slack, int(flag_v.sum() + flag_k.sum())
