"""Plain CPU float64 oracle for the Qwen3-0.6B decode-attention block.

TEST INFRASTRUCTURE ONLY.  This module is the independent reference that the
HIP kernels are checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library itself never
does, and it imports nothing from the library.

What it computes, in the order of the model spec's compute graph (the
"Qwen3-0.6B" Model Spec page, section "Compute-graph nodes"):

  1. ``qk_norm``   per-head RMSNorm of q and k over the 128 head dims
  2. ``rope``      rotation of the pairs (i, i+64) by pos * theta^(-2i/128)
  3. ``append``    the new token's roped k and raw v stored in the paged cache
  4. ``decode_gqa`` o[b,h] = sum_{s<seq_lens[b]} softmax_s(<q[b,h],k[b,s,h/2]>/sqrt(128)) v[b,s,h/2]
  5. ``chunk_step`` the same four steps for a chunk of n new tokens per
     sequence, each attending causally to the positions up to its own

Every step is the plain definition evaluated in float64 with NumPy: no
blocking, no online softmax, no fusion.  Inputs are taken exactly as the
device stores them (float32 and bfloat16 widen to float64 without rounding),
which is how the spec's own conformance check promotes an implementation to
binary64 ("Model conformance" page, "How the comparison works", step 3).

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

  * Cache layout: a K pool and a V pool, each ``[num_pages][8][16][128]``
    (page, KV head, slot, dim).  Position s of sequence b lives in page
    ``block_table[b][s // 16]`` at slot ``s % 16``.  The pages fix only the
    page size (16) in the shape domain ("At a glance").
  * ``seq_lens[b]`` counts the new token: the step appends at
    ``pos = seq_lens[b] - 1`` and attends over ``s < seq_lens[b]``.
  * The RMSNorm constant written "H" in the per-head formula is D = 128.
  * RoPE orientation: x'_i = x_i cos - x_{i+64} sin, x'_{i+64} = x_i sin + x_{i+64} cos.
  * A bfloat16 cache stores round-to-nearest-even of the exact value.

Parity pins: every function here is pinned by the CPU tests against closed
forms, invariants the pages state as theorems, and a 50-digit brute force.
"""
from __future__ import annotations

import math

import numpy as np

# Constants of the spec ("Qwen3-0.6B" Model Spec page, "At a glance" and
# "Compute-graph nodes": attn.qk_norm, attn.rope, attn.core).
NUM_HEADS = 16
NUM_KV_HEADS = 8
HEAD_DIM = 128
ROPE_HALF = 64           # pairs (i, i + 64), i < 64
PAGE_SIZE = 16
RMS_EPS = 1e-6
ROPE_THETA = 1e6


# ---------------------------------------------------------------------------
# bfloat16 encoding (the cache's storage type).  bfloat16 is the upper half of
# an IEEE binary32: 1 sign bit, 8 exponent bits, 7 stored mantissa bits.
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    as_f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return as_f32.astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Written from the format's definition: a finite normal bfloat16 with
    exponent e has spacing 2^(e-7); below 2^-126 the spacing stays 2^-133
    (subnormals).  Values that round past the largest finite bfloat16
    (2^127 * (2 - 2^-7)) become infinities.  NaN stays NaN.
    Returns float64 holding exactly representable bfloat16 values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    mag = np.abs(xf)
    # frexp: mag = f * 2^ex with f in [0.5, 1), so 2^(ex-1) <= mag < 2^ex.
    _, ex = np.frexp(mag)
    e = ex.astype(np.float64) - 1.0
    e = np.maximum(e, -126.0)                       # subnormal range shares 2^-133
    spacing_exp = (e - 7).astype(np.int64)
    scaled = np.ldexp(xf, -spacing_exp)             # exact (power-of-two scaling)
    rounded = np.rint(scaled)                       # numpy rint: ties to even
    val = np.ldexp(rounded, spacing_exp)
    max_finite = math.ldexp(2.0 - 2.0 ** -7, 127)
    val = np.where(np.abs(val) > max_finite, np.copysign(np.inf, xf), val)
    val = np.where(mag == 0, xf, val)               # keep signed zeros
    out[finite] = val
    return out


def cache_to_f64(pool_slice: np.ndarray, cache_dtype: str) -> np.ndarray:
    """Widen stored cache entries (float32, or bfloat16 bits as uint16) to float64."""
    if cache_dtype == "bf16":
        return bf16_bits_to_f64(pool_slice)
    if cache_dtype == "f32":
        return np.asarray(pool_slice, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown cache dtype {cache_dtype!r}")


def store_as_cache_dtype(x: np.ndarray, cache_dtype: str) -> np.ndarray:
    """The value a cache of the given dtype holds after storing float64 x.

    float32 cache: the kernel stores its float32 result unchanged; the oracle
    keeps its float64 value (the comparison tolerance covers float32
    rounding).  bfloat16 cache: round-to-nearest-even of x.
    """
    if cache_dtype == "bf16":
        return round_to_bf16(x)
    if cache_dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown cache dtype {cache_dtype!r}")


# ---------------------------------------------------------------------------
# Step 1: attn.qk_norm ("Qwen3-0.6B" page, "Compute-graph nodes", row
# attn.qk_norm; nnterp qwen3 page, "The Notes": one gain for every head).
# ---------------------------------------------------------------------------

def qk_norm(x: np.ndarray, w: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Per-head RMSNorm: y[..., i] = x[..., i] / sqrt(sum_j x[..., j]^2 / 128 + eps) * w[i].

    ``x`` has the head dimension (128) last; ``w`` is one gain vector shared
    by every head.  The mean square is taken over that head only.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    assert x.shape[-1] == HEAD_DIM and w.shape == (HEAD_DIM,)
    mean_sq = np.sum(x * x, axis=-1, keepdims=True) / HEAD_DIM
    return x / np.sqrt(mean_sq + eps) * w


# ---------------------------------------------------------------------------
# Step 2: attn.rope ("Qwen3-0.6B" page, "Compute-graph nodes", row attn.rope:
# pairs (i, i+64) rotated by pos * theta^(-2i/128), i < 64; D=128, rot=128).
# ---------------------------------------------------------------------------

def rope_angles(pos: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """phi[..., i] = pos * theta^(-2i/128) for i < 64, in float64."""
    i = np.arange(ROPE_HALF, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * i / HEAD_DIM)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x: np.ndarray, pos: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate every pair (x_i, x_{i+64}) by phi_i = pos * theta^(-2i/128).

    ``x`` is [..., heads, 128] and ``pos`` broadcasts against x.shape[:-2]
    (one position per token, shared by all its heads).
    """
    x = np.asarray(x, dtype=np.float64)
    phi = rope_angles(pos, theta)[..., None, :]          # [..., 1, 64]
    c, s = np.cos(phi), np.sin(phi)
    lo, hi = x[..., :ROPE_HALF], x[..., ROPE_HALF:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


# ---------------------------------------------------------------------------
# Step 3: the cache append.  The pages name a paged cache with page size 16
# ("At a glance", shape domain) and decode over seq_lens[b] cached positions
# ("Supported models" page, "What every spec covers"); v is not normed (nnterp
# qwen3 page, "The Notes").
# ---------------------------------------------------------------------------

def cache_location(block_table_row: np.ndarray, s: int) -> tuple[int, int]:
    """(physical page, slot) that holds position s of one sequence."""
    return int(block_table_row[s // PAGE_SIZE]), s % PAGE_SIZE


def gather_sequence(pool: np.ndarray, block_table_row: np.ndarray, seq_len: int,
                    cache_dtype: str) -> np.ndarray:
    """Dense float64 [seq_len, 8, 128] view of one sequence's cached K or V.

    ``pool`` is [num_pages, 8, 16, 128]: K[s, g, :] = pool[block_table_row[s // 16], g, s % 16, :].
    """
    s = np.arange(seq_len)
    pages = np.asarray(block_table_row)[s // PAGE_SIZE]
    slots = s % PAGE_SIZE
    # advanced indices on axes 0 and 2, separated by a slice: the result is
    # [seq_len, 8, 128] with the position axis first
    return cache_to_f64(pool[pages, :, slots, :], cache_dtype)


# ---------------------------------------------------------------------------
# Step 4: attn.core = decodeGQA ("Qwen3-0.6B" page, "Compute-graph nodes",
# row attn.core; nnterp qwen3 page: KV head j serves query heads 2j, 2j+1).
# ---------------------------------------------------------------------------

def softmax(z: np.ndarray) -> np.ndarray:
    """softmax over the last axis, with the maximum subtracted (the spec's
    softmax is invariant under that shift: theorem softmax_shift on the
    "Supported models" page, "Facts proved about the specs")."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def group_size(num_heads: int, num_kv_heads: int = NUM_KV_HEADS) -> int:
    """Query heads per KV head.  Qwen3-0.6B has 16 over 8 (G = 2); the family's
    other sizes are 32, 40 and 64 over 8 (nnterp qwen3 page, "Grouped-query
    attention, with 128-wide heads on every size")."""
    if num_heads % num_kv_heads:
        raise ValueError(f"{num_heads} query heads do not split over {num_kv_heads} KV heads")
    return num_heads // num_kv_heads


def decode_gqa_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """One sequence: q [H,128], k/v [S,8,128] (S >= 1) -> o [H,128].

    o[h] = sum_s softmax_s(<q[h], k[s, h // G]> / sqrt(128)) * v[s, h // G],
    G = H / 8 query heads per KV head (G = 2 for Qwen3-0.6B: KV head j serves
    query heads 2j and 2j+1).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] < 1:
        raise ValueError("decodeGQA needs at least one cached position (S >= 1)")
    H = q.shape[0]
    G = group_size(H, k.shape[1])
    o = np.empty((H, HEAD_DIM), dtype=np.float64)
    scale = 1.0 / math.sqrt(HEAD_DIM)
    for h in range(H):
        g = h // G
        scores = (k[:, g, :] @ q[h]) * scale
        p = softmax(scores)
        o[h] = p @ v[:, g, :]
    return o


def attention_weights(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """The softmax weights decodeGQA uses: [H, S] for one sequence."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    G = group_size(q.shape[0], k.shape[1])
    scale = 1.0 / math.sqrt(HEAD_DIM)
    return np.stack([softmax((k[:, h // G, :] @ q[h]) * scale) for h in range(q.shape[0])])


def paged_decode_gqa(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_table: np.ndarray, seq_lens: np.ndarray, cache_dtype: str,
                     batch_indices=None) -> np.ndarray:
    """decodeGQA over a paged cache, for the sequences in ``batch_indices``
    (all by default).  q is [B,H,128] (already normed and roped).
    Returns o [len(batch_indices),H,128] in float64."""
    q = np.asarray(q, dtype=np.float64)
    idx = range(q.shape[0]) if batch_indices is None else list(batch_indices)
    out = []
    for b in idx:
        n = int(seq_lens[b])
        k = gather_sequence(k_pool, block_table[b], n, cache_dtype)
        v = gather_sequence(v_pool, block_table[b], n, cache_dtype)
        out.append(decode_gqa_dense(q[b], k, v))
    return np.stack(out) if out else np.zeros((0, q.shape[1], HEAD_DIM))


# ---------------------------------------------------------------------------
# The whole step: norm -> rope -> append -> decode.
# ---------------------------------------------------------------------------

def norm_rope(q: np.ndarray, k_new: np.ndarray, q_gain: np.ndarray, k_gain: np.ndarray,
              seq_lens: np.ndarray, eps: float = RMS_EPS, theta: float = ROPE_THETA):
    """q [B,H,128], k_new [B,8,128] -> (q_out, k_rot) at pos = seq_lens - 1."""
    pos = np.asarray(seq_lens, dtype=np.float64) - 1.0
    q_out = rope(qk_norm(q, q_gain, eps), pos, theta)
    k_rot = rope(qk_norm(k_new, k_gain, eps), pos, theta)
    return q_out, k_rot


def decode_step(q, k_new, v_new, q_gain, k_gain, k_pool, v_pool, block_table, seq_lens,
                cache_dtype: str, eps: float = RMS_EPS, theta: float = ROPE_THETA,
                batch_indices=None):
    """One decode step for the selected sequences.

    Returns a dict of float64 arrays, one entry per selected sequence:
      q_out  [n,H,128]   normed and roped query (H = 16 for Qwen3-0.6B)
      k_slot [n,8,128]   value the cache holds at pos after the append
      v_slot [n,8,128]
      o      [n,H,128]   attention output
    The pools are read, never modified: the appended position is taken from
    the oracle's own append, every other position from the pools.
    """
    idx = range(np.asarray(q).shape[0]) if batch_indices is None else list(batch_indices)
    res = {"q_out": [], "k_slot": [], "v_slot": [], "o": []}
    for b in idx:
        n = int(seq_lens[b])
        if n < 1:
            raise ValueError("decode step needs seq_lens[b] >= 1 (the new token)")
        q_out, k_rot = norm_rope(np.asarray(q)[b:b + 1], np.asarray(k_new)[b:b + 1],
                                 q_gain, k_gain, np.asarray(seq_lens)[b:b + 1], eps, theta)
        k_slot = store_as_cache_dtype(k_rot[0], cache_dtype)
        v_slot = store_as_cache_dtype(np.asarray(v_new, dtype=np.float64)[b], cache_dtype)
        k = gather_sequence(k_pool, block_table[b], n - 1, cache_dtype) if n > 1 else \
            np.empty((0, NUM_KV_HEADS, HEAD_DIM))
        v = gather_sequence(v_pool, block_table[b], n - 1, cache_dtype) if n > 1 else \
            np.empty((0, NUM_KV_HEADS, HEAD_DIM))
        k = np.concatenate([k, k_slot[None]], axis=0)
        v = np.concatenate([v, v_slot[None]], axis=0)
        res["q_out"].append(q_out[0])
        res["k_slot"].append(k_slot)
        res["v_slot"].append(v_slot)
        res["o"].append(decode_gqa_dense(q_out[0], k, v))
    return {key: np.stack(val) for key, val in res.items()}


# ---------------------------------------------------------------------------
# Error metrics ("Model conformance" page, "How the comparison works", step 4:
# max |impl - spec| / max |spec|), plus the max absolute error.
# ---------------------------------------------------------------------------

def max_abs_err(impl: np.ndarray, ref: np.ndarray) -> float:
    impl = np.asarray(impl, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(impl - ref))) if ref.size else 0.0


def rel_to_max_err(impl: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    denom = float(np.max(np.abs(ref))) if ref.size else 0.0
    return max_abs_err(impl, ref) / denom if denom > 0 else max_abs_err(impl, ref)


# ---------------------------------------------------------------------------
# Chunks of several new tokens per sequence (chunked prefill, verification of
# drafted tokens): the same nodes over positions pos0 .. pos0 + n - 1, each
# token attending causally (the Model Spec page's shape domain allows
# T in [1, 40,960] new tokens; causality is the theorem forward_causal of the
# "Supported models" page).
# ---------------------------------------------------------------------------

def chunk_step(q, k_new, v_new, q_gain, k_gain, k_pool, v_pool, block_table, seq_lens,
               cu_tokens, cache_dtype: str, eps: float = RMS_EPS, theta: float = ROPE_THETA,
               batch_indices=None, k_stored=None, only=None):
    """Sequence b owns tokens cu_tokens[b] .. cu_tokens[b+1]-1 (n_b of them);
    seq_lens[b] counts the cache after the chunk, so token i of the chunk
    sits at position seq_lens[b] - n_b + i and attends to positions 0 .. that
    position: the cached ones from the pools, the chunk's own from its
    appended (normed, roped, stored) keys and values.

    q [N,H,128], k_new/v_new [N,8,128] (N = cu_tokens[B]).  Returns a dict
    of float64 arrays over the tokens of the selected sequences, in order:
    q_out [n,H,128], k_slot / v_slot [n,8,128] (what the cache holds after
    the append), o [n,H,128], and pos [n].

    k_stored, if given ([n,8,128] over the same tokens), replaces the stored
    keys of the chunk: a caller that knows a key value lies within rounding
    error of a bf16 midpoint can evaluate the step with the other admissible
    rounding.

    only, if given ({b: chunk indices i}), evaluates o for those tokens
    alone (for chunks too long to attend every token here): o and pos then
    hold the selected tokens in order, q_out, k_slot and v_slot still every
    token."""
    q = np.asarray(q)
    cu = np.asarray(cu_tokens, dtype=np.int64)
    idx = range(len(cu) - 1) if batch_indices is None else list(batch_indices)
    res = {"q_out": [], "k_slot": [], "v_slot": [], "o": [], "pos": []}
    done = 0
    for b in idx:
        t0, t1 = int(cu[b]), int(cu[b + 1])
        n = t1 - t0
        L = int(seq_lens[b])
        if n < 1:
            continue
        if L < n:
            raise ValueError("seq_lens[b] must count the chunk's tokens")
        pos = np.arange(L - n, L, dtype=np.float64)
        q_out = rope(qk_norm(q[t0:t1], q_gain, eps), pos, theta)
        k_rot = rope(qk_norm(np.asarray(k_new)[t0:t1], k_gain, eps), pos, theta)
        k_slot = store_as_cache_dtype(k_rot, cache_dtype)
        if k_stored is not None:
            k_slot = np.asarray(k_stored, dtype=np.float64)[done:done + n]
        done += n
        v_slot = store_as_cache_dtype(np.asarray(v_new, dtype=np.float64)[t0:t1], cache_dtype)
        old = L - n
        k_old = gather_sequence(k_pool, block_table[b], old, cache_dtype) if old else \
            np.empty((0, NUM_KV_HEADS, HEAD_DIM))
        v_old = gather_sequence(v_pool, block_table[b], old, cache_dtype) if old else \
            np.empty((0, NUM_KV_HEADS, HEAD_DIM))
        k_all = np.concatenate([k_old, k_slot], axis=0)
        v_all = np.concatenate([v_old, v_slot], axis=0)
        chosen = range(n) if only is None else [int(i) for i in only.get(b, [])]
        for i in chosen:
            p = old + i
            res["o"].append(decode_gqa_dense(q_out[i], k_all[:p + 1], v_all[:p + 1]))
            res["pos"].append(p)
        res["q_out"].extend(q_out)
        res["k_slot"].extend(k_slot)
        res["v_slot"].extend(v_slot)
    return {key: (np.array(val, dtype=np.int64) if key == "pos" else np.stack(val))
            if val else np.zeros((0,)) for key, val in res.items()}
