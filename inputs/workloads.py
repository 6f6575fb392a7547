"""Seeded synthetic workloads for the decode-attention path.

This module only draws inputs: shapes, sequence lengths, page tables and
random values.  It holds none of the method's arithmetic, so both the HIP
path (through the binding) and the CPU oracle can consume what it produces.

Shapes follow the "Qwen3-0.6B" Model Spec page ("At a glance": shape domain
B <= 256 sequences, S <= 40,960 cached positions, page size 16;
"Tensors of the main nodes": q [B,16,128], k/v [B,S,8,128]).  The family
workloads keep those shapes but give q the head count of a larger member
(nnterp qwen3 page, "Grouped-query attention, with 128-wide heads on every
size": 32, 40 or 64 query heads over the same 8 KV heads) and, for the 4B-2507
pair, RoPE base 5e6 ("What loads as this family").  Values follow
the conformance methodology of the "Model conformance" page ("How the
comparison works", step 1): O(1) activations and norm gains perturbed away
from 1 (here 1 + N(0, 0.1)).

Cache layout (shared contract with the library): a K pool and a V pool, each
``[num_pages, 8, 16, 128]`` = (physical page, KV head, slot, dim), in float32
or bfloat16.  ``block_table[b, j]`` is the physical page of sequence b's
logical page j; entries past a sequence's last page are 0 and never read.

Host-side structure (lengths, tables, outlier positions) comes from NumPy's
PCG64 seeded per workload.  Large value tensors come from torch's generator
on the target device, seeded per (workload, layer, tensor), so generation on
a GPU never round-trips through host memory.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

NUM_HEADS = 16
NUM_KV_HEADS = 8
HEAD_DIM = 128
PAGE_SIZE = 16
RMS_EPS = 1e-6
ROPE_THETA = 1e6
HIDDEN = 1024   # Qwen3-0.6B ("At a glance"); 2560 for 4B, 5120 for 14B/32B (nnterp qwen3 page)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    cache_dtype: str                 # "f32" or "bf16"
    seed: int
    num_layers: int = 1
    lens_kind: str = "fixed"          # fixed | uniform | loguniform | list
    lens_args: tuple = ()
    pool_pages: int | None = None     # None: exactly the pages the batch needs
    key_outlier: float | None = None  # multiply one cached key position by this
    num_heads: int = NUM_HEADS        # query heads (16, 32, 40 or 64) over 8 KV heads
    rope_theta: float = ROPE_THETA
    hidden: int = HIDDEN              # model width the projections map from and to
    description: str = ""

    def seq_lens(self) -> np.ndarray:
        return make_seq_lens(self)

    def max_seq_len(self) -> int:
        return int(self.seq_lens().max())

    def max_pages_per_seq(self) -> int:
        return pages_for(self.max_seq_len())


def pages_for(seq_len: int) -> int:
    return (int(seq_len) + PAGE_SIZE - 1) // PAGE_SIZE


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32_b2", batch=2, cache_dtype="f32", seed=0,
                 lens_kind="list", lens_args=(7, 12), pool_pages=16,
                 description="fp32 cache; B=2, seq_lens {7,12}; 16-page pool, "
                             "block table from a seeded permutation"),
        Workload("ragged_b32", batch=32, cache_dtype="bf16", seed=1,
                 lens_kind="uniform", lens_args=(512, 4096), pool_pages=65536,
                 description="bf16 cache; B=32, seq_lens uniform in [512,4096]; "
                             "pages scattered through a 65,536-page pool"),
        Workload("b256_s2048", batch=256, cache_dtype="bf16", seed=2,
                 lens_kind="fixed", lens_args=(2048,), pool_pages=65536,
                 description="bf16 cache; B=256, every seq_len 2048 (128 pages); "
                             "random block table in a 65,536-page pool"),
        Workload("long_b4_s40960", batch=4, cache_dtype="bf16", seed=3,
                 lens_kind="list", lens_args=(40960, 40960, 32768, 16384),
                 pool_pages=65536, key_outlier=8.0,
                 description="bf16 cache; B=4, seq_lens {40960,40960,32768,16384}; "
                             "one cached key position per sequence scaled by 8"),
        Workload("stack28_b128", batch=128, cache_dtype="bf16", seed=4, num_layers=28,
                 lens_kind="loguniform", lens_args=(16, 16384), pool_pages=None,
                 description="28 layers, each with its own bf16 pool and gains; "
                             "B=128, seq_lens log-uniform in [16,16384]; one block "
                             "table shared by all layers"),
        # The same cache as b256_s2048 (identical seeds, so identical KV bytes)
        # read by the larger family members' query heads.
        Workload("b256_s2048_h32", batch=256, cache_dtype="bf16", seed=2,
                 lens_kind="fixed", lens_args=(2048,), pool_pages=65536, num_heads=32,
                 rope_theta=5e6,
                 description="b256_s2048 with 32 query heads (group size 4) and "
                             "RoPE base 5e6, the 4B-2507 attention shape"),
        Workload("b256_s2048_h40", batch=256, cache_dtype="bf16", seed=2,
                 lens_kind="fixed", lens_args=(2048,), pool_pages=65536, num_heads=40,
                 description="b256_s2048 with 40 query heads (group size 5), the 14B shape"),
        Workload("b256_s2048_h64", batch=256, cache_dtype="bf16", seed=2,
                 lens_kind="fixed", lens_args=(2048,), pool_pages=65536, num_heads=64,
                 description="b256_s2048 with 64 query heads (group size 8), the 32B shape"),
        Workload("ragged_f32_b6", batch=6, cache_dtype="f32", seed=5,
                 lens_kind="list", lens_args=(1, 16, 17, 100, 333, 1024), pool_pages=256,
                 description="fp32 cache; B=6, seq_lens {1,16,17,100,333,1024} (one "
                             "position, a full page, a page plus one, ragged tails); "
                             "the small case for every head count"),
    ]
}


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([w.seed, stream]))


def make_seq_lens(w: Workload) -> np.ndarray:
    rng = _rng(w, 1)
    if w.lens_kind == "fixed":
        lens = np.full(w.batch, w.lens_args[0])
    elif w.lens_kind == "list":
        lens = np.array(w.lens_args)
        assert lens.size == w.batch
    elif w.lens_kind == "uniform":
        lo, hi = w.lens_args
        lens = rng.integers(lo, hi + 1, size=w.batch)
    elif w.lens_kind == "loguniform":
        lo, hi = w.lens_args
        lens = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=w.batch)))
        lens = np.clip(lens, lo, hi)
    else:
        raise ValueError(w.lens_kind)
    return lens.astype(np.int32)


def make_block_table(w: Workload, seq_lens: np.ndarray | None = None):
    """(block_table int32 [B, max_pages_per_seq], num_pages).

    Every sequence gets distinct physical pages drawn from a seeded
    permutation of the pool."""
    if seq_lens is None:
        seq_lens = make_seq_lens(w)
    need = np.array([pages_for(n) for n in seq_lens], dtype=np.int64)
    total = int(need.sum())
    num_pages = total if w.pool_pages is None else int(w.pool_pages)
    if num_pages < total:
        raise ValueError(f"{w.name}: pool of {num_pages} pages < {total} needed")
    rng = _rng(w, 2)
    perm = rng.permutation(num_pages)[:total].astype(np.int32)
    mpps = max(1, int(need.max()))
    table = np.zeros((w.batch, mpps), dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    return table, num_pages


def outlier_positions(w: Workload, seq_lens: np.ndarray) -> np.ndarray:
    """One cached position per sequence, uniform over [0, seq_len - 1)."""
    rng = _rng(w, 3)
    return np.array([rng.integers(0, max(1, int(n) - 1)) for n in seq_lens], dtype=np.int64)


def _torch_generator(torch, device, w: Workload, layer: int, tensor_id: int):
    g = torch.Generator(device=device)
    g.manual_seed(((w.seed * 1009 + layer) * 64 + tensor_id) & 0x7FFFFFFFFFFF)
    return g


def make_layer(w: Workload, layer: int, device, table=None, num_pages=None, seq_lens=None):
    """Random tensors of one layer on ``device`` (torch tensors).

    Returns dict with q [B,H,128] (H = w.num_heads), k_new/v_new [B,8,128]
    (float32, pre-norm),
    q_gain/k_gain [128] (float32), k_pool/v_pool [num_pages,8,16,128] in the
    cache dtype, and the int32 block_table and seq_lens."""
    import torch

    if seq_lens is None:
        seq_lens = make_seq_lens(w)
    if table is None:
        table, num_pages = make_block_table(w, seq_lens)
    elif num_pages is None:
        raise ValueError("make_layer: pass num_pages together with table")
    B = w.batch
    cdt = torch.float32 if w.cache_dtype == "f32" else torch.bfloat16

    def randn(shape, tensor_id, dtype=torch.float32):
        return torch.randn(shape, generator=_torch_generator(torch, device, w, layer, tensor_id),
                           device=device, dtype=dtype)

    out = {
        "q": randn((B, w.num_heads, HEAD_DIM), 0),
        "k_new": randn((B, NUM_KV_HEADS, HEAD_DIM), 1),
        "v_new": randn((B, NUM_KV_HEADS, HEAD_DIM), 2),
        "q_gain": 1.0 + 0.1 * randn((HEAD_DIM,), 3),
        "k_gain": 1.0 + 0.1 * randn((HEAD_DIM,), 4),
        "k_pool": randn((num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM), 5, cdt),
        "v_pool": randn((num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM), 6, cdt),
        "block_table": torch.from_numpy(table).to(device),
        "seq_lens": torch.from_numpy(np.asarray(seq_lens, dtype=np.int32)).to(device),
    }
    if w.key_outlier is not None:
        pos = outlier_positions(w, seq_lens)
        pages = torch.from_numpy(table[np.arange(B), pos // PAGE_SIZE].astype(np.int64)).to(device)
        slots = torch.from_numpy((pos % PAGE_SIZE).astype(np.int64)).to(device)
        kp = out["k_pool"]
        kp[pages, :, slots, :] = kp[pages, :, slots, :] * w.key_outlier
    return out


def poison_unused(layer_tensors: dict, seq_lens: np.ndarray, table: np.ndarray,
                  include_new_slot: bool = False, value: float = float("nan")):
    """Fill every cache entry that no sequence may read with ``value``:
    unused pages, and slots at or past seq_len in each last page.  With
    ``include_new_slot`` the slot at seq_len - 1 (where a step appends) is
    poisoned as well."""
    import torch

    kp, vp = layer_tensors["k_pool"], layer_tensors["v_pool"]
    num_pages = kp.shape[0]
    used = np.zeros(num_pages, dtype=bool)
    for b, n in enumerate(seq_lens):
        used[table[b, :pages_for(n)]] = True
    unused_idx = torch.from_numpy(np.nonzero(~used)[0]).to(kp.device)
    if unused_idx.numel():
        kp[unused_idx] = value
        vp[unused_idx] = value
    for b, n in enumerate(seq_lens):
        n = int(n)
        first = n - 1 if include_new_slot else n      # first position to poison
        last_page = (n - 1) // PAGE_SIZE              # logical page holding position n-1
        if first // PAGE_SIZE == last_page:           # poisoned slots share that page
            phys = int(table[b, last_page])
            kp[phys, :, first % PAGE_SIZE:, :] = value
            vp[phys, :, first % PAGE_SIZE:, :] = value
    return layer_tensors


def algorithmic_kv_bytes(seq_lens: np.ndarray, cache_dtype: str) -> int:
    """Bytes of K and V the decode must read: every cached position of every
    sequence, 8 KV heads x 128 dims x (K and V) x element size."""
    elt = 4 if cache_dtype == "f32" else 2
    return int(np.sum(np.asarray(seq_lens, dtype=np.int64))) * NUM_KV_HEADS * HEAD_DIM * 2 * elt


def make_projections(w: Workload, layer: int, device):
    """Inputs of the projections around the block (torch tensors on device):
    x [B, hidden] float32 ~ N(0,1) (the block's input, one token per
    sequence); w_qkv [(H + 16) * 128, hidden] and w_o [hidden, H * 128] in
    bfloat16, entries N(0,1) / sqrt(fan-in) so that outputs stay O(1), as
    the conformance check draws linear weights ("Model conformance" page,
    "How the comparison works", step 1)."""
    import torch

    H = w.num_heads
    n_qkv = (H + 2 * NUM_KV_HEADS) * HEAD_DIM

    def randn(shape, tensor_id):
        return torch.randn(shape, generator=_torch_generator(torch, device, w, layer, tensor_id),
                           device=device, dtype=torch.float32)

    return {
        "x": randn((w.batch, w.hidden), 10),
        "w_qkv": (randn((n_qkv, w.hidden), 11) / math.sqrt(w.hidden)).to(torch.bfloat16),
        "w_o": (randn((w.hidden, H * HEAD_DIM), 12) / math.sqrt(H * HEAD_DIM)).to(torch.bfloat16),
    }


def make_chunk_inputs(lens_old, chunks, num_heads: int, cache_dtype: str, seed: int, device,
                      pool_pages: int | None = None):
    """Inputs of a chunk step: sequence b holds lens_old[b] cached positions
    and receives chunks[b] new tokens (seq_lens = lens_old + chunks).
    Values N(0,1), gains 1 + N(0, 0.1); pages of every sequence drawn from a
    seeded permutation of the pool; unused pool pages hold N(0,1) too.
    Returns torch tensors on `device` and the host block table."""
    import torch

    lens_old = np.asarray(lens_old, np.int64)
    chunks = np.asarray(chunks, np.int64)
    B = len(lens_old)
    seq_lens = (lens_old + chunks).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    N = int(cu[-1])
    need = np.array([pages_for(n) for n in seq_lens], np.int64)
    total = int(need.sum())
    num_pages = max(total, 1) if pool_pages is None else int(pool_pages)
    rng = np.random.Generator(np.random.PCG64([seed, 2]))
    perm = rng.permutation(num_pages)[:total].astype(np.int32)
    table = np.zeros((B, max(1, int(need.max()))), np.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n]
        at += n
    g = torch.Generator(device=device)
    g.manual_seed(seed * 7919 + 17)
    cdt = torch.float32 if cache_dtype == "f32" else torch.bfloat16

    def randn(shape, dtype=torch.float32):
        return torch.randn(shape, generator=g, device=device, dtype=dtype)

    t = {
        "q": randn((N, num_heads, HEAD_DIM)),
        "k_new": randn((N, NUM_KV_HEADS, HEAD_DIM)),
        "v_new": randn((N, NUM_KV_HEADS, HEAD_DIM)),
        "q_gain": 1.0 + 0.1 * randn((HEAD_DIM,)),
        "k_gain": 1.0 + 0.1 * randn((HEAD_DIM,)),
        "k_pool": randn((num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM), cdt),
        "v_pool": randn((num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM), cdt),
        "block_table": torch.from_numpy(table).to(device),
        "seq_lens": torch.from_numpy(seq_lens).to(device),
        "cu_tokens": torch.from_numpy(cu).to(device),
    }
    return t, table, seq_lens, cu


INTERMEDIATE = 3072   # Qwen3-0.6B MLP width (Model Spec page: mlp.act I = 3072)


def make_layer_weights(w: Workload, layer: int, device, inter: int = INTERMEDIATE):
    """A decoder layer's weights on `device` (random, as the conformance check
    draws them: "Model conformance" page, "How the comparison works", step 1):
    the projections of make_projections, q/k gains of make_layer's draw,
    norm gains 1 + N(0, 0.1), gate_up [2I, hidden] and down [hidden, I] with
    entries N(0,1)/sqrt(fan-in) in bfloat16; plus the input x [B, hidden]."""
    import torch

    p = make_projections(w, layer, device)

    def randn(shape, tensor_id):
        return torch.randn(shape, generator=_torch_generator(torch, device, w, layer, tensor_id),
                           device=device, dtype=torch.float32)

    return {
        "x": p["x"], "w_qkv": p["w_qkv"], "w_o": p["w_o"],
        "w_in": 1.0 + 0.1 * randn((w.hidden,), 20),
        "q_gain": 1.0 + 0.1 * randn((HEAD_DIM,), 3),
        "k_gain": 1.0 + 0.1 * randn((HEAD_DIM,), 4),
        "w_post": 1.0 + 0.1 * randn((w.hidden,), 21),
        "w_gate_up": (randn((2 * inter, w.hidden), 22) / math.sqrt(w.hidden)).to(torch.bfloat16),
        "w_down": (randn((w.hidden, inter), 23) / math.sqrt(inter)).to(torch.bfloat16),
    }
