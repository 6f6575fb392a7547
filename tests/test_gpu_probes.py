"""GPU checks of the benchmark's paged-read probe (include/dah_probe.h): it
reads exactly the K and V tiles the decode reads -- for each sequence and KV
head, the head's tile of every page of the sequence's prefix -- which the
XOR of everything it loaded, recomputed on the host, pins down."""
import numpy as np
import pytest

from dah_testlib import build_layer, cuda_available
from inputs import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _host_xor(pool_words, table, lens, max_seq_len):
    """sink[b, g] = XOR over the pages p < ceil(len/16) of sequence b of every
    32-bit word of KV head g's tile (pool_words: [num_pages, 8, words])."""
    B = len(lens)
    out = np.zeros((B, 8), np.uint32)
    for b, n in enumerate(lens):
        if not 1 <= n <= max_seq_len:
            continue
        ids = table[b, :(n + 15) // 16]
        out[b] = np.bitwise_xor.reduce(pool_words[ids], axis=(0, 2))
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_read_probe_reads_the_decode_tiles(dtype):
    import torch
    from decode_attention_head_amd.probes import probe_paged_read
    lens = [1, 16, 17, 100, 333, 1024, 5, 0]
    w = W.Workload("probe_case", batch=len(lens), cache_dtype=dtype, seed=44, lens_kind="list",
                   lens_args=tuple(max(n, 1) for n in lens), pool_pages=200)
    t, seq_lens, table, num_pages = build_layer(w)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")   # one empty sequence
    sl_cpu = np.array(lens)
    L = 1024
    sink = torch.full((8 * len(lens),), -1, dtype=torch.int32, device="cuda")
    probe_paged_read(t["k_pool"], t["v_pool"], t["block_table"], sl, L, sink)
    torch.cuda.synchronize()

    def words(pool):
        return pool.cpu().contiguous().view(torch.int32).numpy().view(np.uint32).reshape(
            pool.shape[0], 8, -1)
    kx = _host_xor(words(t["k_pool"]), table, sl_cpu, L)
    vx = _host_xor(words(t["v_pool"]), table, sl_cpu, L)
    got = sink.cpu().numpy().view(np.uint32).reshape(len(lens), 8)
    want = kx ^ vx
    want[sl_cpu < 1] = 0          # nothing read: the folded accumulator stays zero
    assert np.array_equal(got, want)


def test_probe_copy_refuses_mismatched_sizes_before_launching():
    """The copy probe takes its byte count from the tensors: a destination
    smaller (or larger) than the source, as a clamped slice of a smaller
    tensor gives, is refused before any launch, and the destination keeps
    its contents.  A matching pair copies exactly."""
    import torch
    from decode_attention_head_amd.probes import probe_copy, probe_read
    src = torch.arange(1 << 14, dtype=torch.int32, device="cuda")          # 64 KiB
    small = torch.full((1 << 13,), -7, dtype=torch.int32, device="cuda")   # 32 KiB
    big = torch.full((1 << 15,), -7, dtype=torch.int32, device="cuda")     # 128 KiB
    for dst in (small, big, big[: (1 << 14) + 4]):
        with pytest.raises(ValueError):
            probe_copy(src, dst)
    with pytest.raises(ValueError):
        probe_copy(src[: 1 << 30], small)       # the slice clamps to 64 KiB: still refused
    with pytest.raises(ValueError):
        probe_copy(src[::2], small)             # not contiguous
    torch.cuda.synchronize()
    assert bool((small == -7).all()) and bool((big == -7).all())
    with pytest.raises(ValueError):
        probe_read(src, torch.zeros(4, dtype=torch.int32, device="cuda"), 8)   # sink too small
    dst = torch.empty_like(src)
    assert probe_copy(src, dst) == src.numel() * 4
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
