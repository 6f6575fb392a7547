"""Benchmark of the decode-attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b256_s2048]

A step is one pass of the whole hot path over the batch: one call of
decode_attn_step (q/k RMSNorm, RoPE, cache append and split-S decodeGQA, in
one kernel launch when one split suffices, plus the log-sum-exp combine
otherwise) per layer of the workload -- one for every workload but
stack28_b128, whose step runs its 28 layers, each with its own cache and
gains.  `value` is the workload's K/V bytes over the host-timed mean of K
steps (W untimed warm-up steps first).  HIP events recorded on the launch
stream bracket the calls of every --event-every'th step (by default enough
for at least 10 launches) for the roofline figures.  Inputs are synthetic,
seeded and resident in HBM before timing starts.

The JSON line reports
  value           KV-read throughput, GB/s = (sum of seq_lens * 4096 B) / step time
  roofline        the step's decode kernel (dominant kernel): algorithmic KV
                  bytes per launch / its average duration measured with HIP
                  events on the launch stream, against MI355X's 8 TB/s HBM peak
  configs         the five workloads (tiny float32 B=2; ragged B=32; the B=256,
                  S=2048 headline; 4 long contexts; the 28-layer ragged stack),
                  each timed alone: 5 warm-up steps, then the median of 50 steps
                  bracketed by HIP events, with a 1 GiB scratch read before each
                  (outside the events) so that no step finds K/V in the
                  last-level cache; plan, kernel, GB/s, % of 8 TB/s, seqs/s,
                  and the error of the first step's o and q_out against the
                  float64 oracle over every sequence (both layers 0 and 27 of
                  the stack)
  cpu_baseline    the float64 CPU oracle over every sequence of the headline
                  workload on a pool of worker processes (one core each, all
                  host cores), repeated to about 10 s of work, and its
                  single-core rate (about 3 s); the oracle's first pass over
                  each workload gives the per-config errors
  prefill         chunk_attn_step with 1,024 new tokens per sequence at the
                  end of the four long_b4_s40960 contexts (--prefill-tokens):
                  graph-replayed time, attention TFLOP/s and % of the bf16
                  dense matrix-core peak

--chunk N also times chunk_attn_step with N new tokens per sequence (the
workload's lengths counting them), under "chunk": HIP-graph-replayed time,
K/V bytes (each cached position once per sequence) and attention flops.

--layer also times decoder_layer_step (input_norm, the block with its
projections, residuals, SwiGLU MLP) on the same batch, graph-replayed.

--block also times the projections on either side of the block (attn.qkv_proj
before the step, attn.o_proj after it) on the same batch and reports them under
"block": per-launch durations (HIP events), their bytes and flops, and the
whole x -> qkv_proj -> decode_attn_step -> o_proj pass.

--kernel valu|mfma forces the decode kernel's form (measurement aid).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from inputs import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
KERNEL_SOURCE = os.path.join(ROOT, "decode_attention_head_amd", "csrc", "dah_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"decode_split_kernel_{workload}_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="b256_s2048", choices=sorted(W.WORKLOADS))
    ap.add_argument("--num-splits", type=int, default=0, help="0 = planner's choice")
    ap.add_argument("--event-every", type=int, default=0, metavar="N",
                    help="bracket the calls of every N-th timed step with HIP events "
                         "(default: steps/10, at most 10, so that >= 10 launches are timed)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (its rate and each workload's error)")
    ap.add_argument("--cpu-seconds", type=float, default=None, help=argparse.SUPPRESS)
    ap.add_argument("--config-iters", type=int, default=50, metavar="N",
                    help="timed steps per workload in the five-workload report (0 skips it)")
    ap.add_argument("--kernel", choices=["valu", "mfma"], default=None,
                    help="force the decode kernel form (sets DAH_DECODE_KERNEL; a measurement "
                         "aid: the VALU form exists for float32 caches and up to 2 query heads "
                         "per KV head with bfloat16)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time paged_decode_gqa alone (profiling aid)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming-read probe (practical bandwidth ceiling) and the "
                         "paged-read probe (the decode's access pattern alone)")
    ap.add_argument("--chunk", type=int, default=0, metavar="N",
                    help="also time chunk_attn_step with N new tokens per sequence")
    ap.add_argument("--prefill-tokens", type=int, default=1024, metavar="N",
                    help="the prefill record: chunk_attn_step with N new tokens per sequence "
                         "over the long_b4_s40960 lengths (0 skips it)")
    ap.add_argument("--layer", action="store_true",
                    help="also time decoder_layer_step on the same batch")
    ap.add_argument("--block", action="store_true",
                    help="also time qkv_proj and o_proj around the step")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run 3 plain device copies of this many MiB (a kernel of "
                         "known traffic, to calibrate rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary of this workload's fused step, if it was taken on the current
    kernel source; else None."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != source_digest():
        return None
    return float(m_val.group(1))


# ---------------------------------------------------------------------------
# CPU baseline leg: the float64 oracle on the host's cores.  A pool of worker
# processes (spawned before this process touches the GPU, so no worker holds a
# GPU context) maps the oracle's decode step over sequences; each config's
# host copy of its inputs reaches the workers as memory-mapped .npy files.
# The oracle's outputs on those sequences are also what each config's error
# against the GPU is computed from.
# ---------------------------------------------------------------------------

_SNAP_KEYS = ("q", "k_new", "v_new", "q_gain", "k_gain", "k_pool", "v_pool", "block_table",
              "seq_lens")
_worker_snaps = {}


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)            # one core per worker process


def _worker_rows(task):
    """Oracle decode step over rows of a snapshot directory (worker side)."""
    path, rows, cache_dtype, theta = task
    snap = _worker_snaps.get(path)
    if snap is None:
        _worker_snaps.clear()
        snap = {k: np.load(os.path.join(path, k + ".npy"), mmap_mode="r") for k in _SNAP_KEYS}
        _worker_snaps[path] = snap
    from oracle import decode_attention as O
    r = O.decode_step(snap["q"], snap["k_new"], snap["v_new"], snap["q_gain"], snap["k_gain"],
                      snap["k_pool"], snap["v_pool"], snap["block_table"], snap["seq_lens"],
                      cache_dtype, theta=theta, batch_indices=rows)
    return rows, r["q_out"], r["o"]


def host_workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


class OraclePool:
    """Worker processes running the unchanged oracle, one core each."""

    def __init__(self, workers: int):
        import multiprocessing as mp
        self.workers = workers
        self.pool = mp.get_context("spawn").Pool(workers, initializer=_worker_init)
        self.pool.map(_worker_init_done, range(workers))       # all started and warm
        self.dirs = []

    def _dump(self, snap: dict, tag: str) -> str:
        import shutil
        import tempfile
        need = sum(np.asarray(snap[k]).nbytes for k in _SNAP_KEYS)
        base = None                     # memory-backed /dev/shm when it has room, else /tmp
        if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > 2 * need:
            base = "/dev/shm"
        path = tempfile.mkdtemp(prefix=f"dah_oracle_{tag}_", dir=base)
        self.dirs.append(path)
        for k in _SNAP_KEYS:
            np.save(os.path.join(path, k + ".npy"), np.ascontiguousarray(snap[k]))
        return path

    def run(self, snap: dict, tag: str, cache_dtype: str, theta: float, rows=None,
            serial: bool = False, repeat: int = 1):
        """(q_out, o, seconds): the oracle over `rows` of the snapshot (all by
        default), `repeat` times over, timed from submission to the last
        result.  serial: one worker, one sequence at a time (the single-core
        rate)."""
        path = self._dump(snap, tag)
        n = len(snap["seq_lens"])
        rows = list(range(n)) if rows is None else list(rows)
        # longest sequences first, so that the pool's tail is short
        order = sorted(rows, key=lambda b: -int(snap["seq_lens"][b]))
        tasks = [(path, [b], cache_dtype, theta) for b in order] * repeat
        self.pool.apply(_worker_rows, ((path, order[:1], cache_dtype, theta),))   # map the files
        t0 = time.perf_counter()
        if serial:
            results = [self.pool.apply(_worker_rows, (tk,)) for tk in tasks]
        else:
            results = self.pool.map(_worker_rows, tasks, chunksize=1)
        secs = time.perf_counter() - t0
        H = snap["q"].shape[1]
        q_out = np.zeros((n, H, W.HEAD_DIM))
        o = np.zeros((n, H, W.HEAD_DIM))
        for rws, qo, oo in results:
            q_out[rws], o[rws] = qo, oo
        import shutil
        shutil.rmtree(path, ignore_errors=True)
        return q_out[rows], o[rows], secs

    def close(self):
        import shutil
        self.pool.terminate()
        self.pool.join()
        for path in self.dirs:
            shutil.rmtree(path, ignore_errors=True)


def _worker_init_done(_):
    return os.getpid()


def oracle_errors(q_gpu, o_gpu, q_ref, o_ref):
    """max abs error and the pages' relative-to-max error ("Model conformance"
    page, "How the comparison works", step 4) of o, and q_out's max abs."""
    o_gpu = np.asarray(o_gpu, np.float64)
    e = float(np.max(np.abs(o_gpu - o_ref)))
    return {"o_max_abs": e, "o_rel_to_max": e / float(np.max(np.abs(o_ref))),
            "q_out_max_abs": float(np.max(np.abs(np.asarray(q_gpu, np.float64) - q_ref))),
            "finite": bool(np.all(np.isfinite(o_gpu)))}


def _graph_us(torch, fn, n):
    """Mean time of fn over n calls captured in one HIP graph and replayed
    (no host launch cost between the kernels, as a serving loop would run)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / n


def time_block(dah, torch, w, t, L, ws, stream, args):
    """qkv_proj and o_proj around the step, each alone, and the three in
    sequence (the step reads the projection's q, k, v), each captured in a
    HIP graph and replayed."""
    p = W.make_projections(w, 0, t["q"].device)
    B, H, hid = w.batch, w.num_heads, w.hidden
    q, k, v = dah.qkv_proj(p["x"], p["w_qkv"], H)
    q_out, o = torch.empty_like(q), torch.empty_like(q)
    y = torch.empty((B, hid), dtype=torch.float32, device=o.device)
    o_ws = torch.empty(max(dah.linear_workspace_bytes(B, hid, H * W.HEAD_DIM), 256),
                       dtype=torch.uint8, device=o.device)

    def qkv():
        dah.qkv_proj(p["x"], p["w_qkv"], H, q=q, k=k, v=v)

    def oproj():
        dah.o_proj_ws(o, p["w_o"], y=y, workspace=o_ws)

    def oproj_unsplit():
        dah.o_proj(o, p["w_o"], y=y)

    def step():
        dah.decode_attn_step(q, k, v, t["q_gain"], t["k_gain"], t["k_pool"], t["v_pool"],
                             t["block_table"], t["seq_lens"], L, rope_theta=w.rope_theta,
                             num_splits=args.num_splits, q_out=q_out, o=o, workspace=ws)

    def whole():
        qkv()
        step()
        oproj()

    n = 20
    qkv_us, o_us = _graph_us(torch, qkv, n), _graph_us(torch, oproj, n)
    o_unsplit_us = _graph_us(torch, oproj_unsplit, n)
    step_us, whole_us = _graph_us(torch, step, n), _graph_us(torch, whole, n)

    def stats(us, n_out, k_in):
        byts = n_out * k_in * 2 + B * k_in * 4 + B * n_out * 4   # bf16 weights, f32 x and y
        flop = 2.0 * B * n_out * k_in
        return {"us": round(us, 2), "bytes": byts, "gbs": round(byts / us / 1e3, 1),
                "tflops": round(flop / us / 1e6, 2)}
    n_qkv = (H + 2 * W.NUM_KV_HEADS) * W.HEAD_DIM
    o_kernel, o_slices = dah.linear_ws_kernel(B, hid, H * W.HEAD_DIM)
    return {"qkv_proj": stats(qkv_us, n_qkv, hid), "o_proj": stats(o_us, hid, H * W.HEAD_DIM),
            "o_proj_unsplit_us": round(o_unsplit_us, 2), "o_proj_k_slices": o_slices,
            "o_proj_kernel": o_kernel,
            "step_us": round(step_us, 2), "block_us": round(whole_us, 2), "hidden": hid,
            "timing": "HIP graph replay of 20 calls, mean per call",
            "note": "x [B,hidden] f32, bf16 weights; block = qkv_proj + decode_attn_step + "
                    "o_proj_ws (k split into a workspace, the reduce included)"}


def time_layer(dah, torch, w, t, L, args):
    """decoder_layer_step on the workload's batch, graph-replayed; the cache
    is restored afterwards (each call appends)."""
    p = W.make_layer_weights(w, 0, t["q"].device)
    weights = {n: p[n] for n in dah.LAYER_WEIGHTS}
    inter = p["w_down"].shape[1]
    ws = torch.empty(dah.layer_workspace_bytes(w.batch, w.hidden, inter, L, args.num_splits,
                                               w.num_heads, w.cache_dtype),
                     dtype=torch.uint8, device=t["q"].device)
    y = torch.empty_like(p["x"])
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def run():
        dah.decoder_layer_step(p["x"], weights, t["k_pool"], t["v_pool"], t["block_table"],
                               t["seq_lens"], L, rope_theta=w.rope_theta,
                               num_splits=args.num_splits, y=y, workspace=ws)
    us = _graph_us(torch, run, 10)
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    H, hid = w.num_heads, w.hidden
    weight_bytes = 2 * hid * ((H + 16) * 128 + H * 128 + 3 * inter)
    return {"us": round(us, 2), "tokens_per_s": round(w.batch / (us * 1e-6), 1),
            "hidden": hid, "inter": inter, "weight_bytes": weight_bytes,
            "timing": "HIP graph replay of 10 calls, mean per call"}


def time_chunk(dah, torch, w, seq_lens, num_pages, n):
    """chunk_attn_step with n new tokens per sequence of the workload (its
    seq_lens count them), bf16 cache, graph-replayed."""
    lens = np.asarray(seq_lens, np.int64)
    if np.any(lens < n):
        return {"skipped": f"sequences shorter than {n} tokens"}
    B, H = w.batch, w.num_heads
    t, table, sl, cu = W.make_chunk_inputs(lens - n, [n] * B, H, "bf16", 777, "cuda",
                                           pool_pages=max(num_pages, int(sum(
                                               W.pages_for(int(x)) for x in lens))))
    L = int(sl.max())
    q_out, o = torch.empty_like(t["q"]), torch.empty_like(t["q"])
    k0, v0 = t["k_pool"].clone(), t["v_pool"].clone()

    def run():
        dah.chunk_attn_step(t["q"], t["k_new"], t["v_new"], t["q_gain"], t["k_gain"], t["k_pool"],
                            t["v_pool"], t["block_table"], t["seq_lens"], t["cu_tokens"], n, L,
                            q_out=q_out, o=o)
    us = _graph_us(torch, run, 10)
    t["k_pool"].copy_(k0)
    t["v_pool"].copy_(v0)
    kv_bytes = int(lens.sum()) * W.NUM_KV_HEADS * W.HEAD_DIM * 2 * 2
    attended = sum(int(L0) * n - n * (n - 1) // 2 for L0 in lens)   # sum over tokens of (pos + 1)
    flop = 4.0 * W.HEAD_DIM * H * attended
    return {"tokens_per_seq": n, "us": round(us, 2), "kv_bytes": kv_bytes,
            "kv_gbs": round(kv_bytes / us / 1e3, 1), "tflops": round(flop / us / 1e6, 2),
            "tokens_per_s": round(B * n / (us * 1e-6), 1),
            "timing": "HIP graph replay of 10 calls (append + attention launches), mean per call"}


# The five workloads every run reports (tiny float32 reference, ragged B=32,
# the B=256 S=2048 headline, long contexts, the 28-layer ragged stack).
CONFIGS = ["tiny_f32_b2", "ragged_b32", "b256_s2048", "long_b4_s40960", "stack28_b128"]
FLUSH_BYTES = 1 << 30   # scratch read between timed iterations (past the last-level cache)
CPU_BASELINE_SECONDS = 10.0   # oracle work the CPU baseline is timed over (all host cores)
CPU_SINGLE_SECONDS = 3.0      # and its single-core rate


def time_config(dah, torch, name, flush, iters, warmup, num_splits, want_check):
    """One workload: decode_attn_step over its layers, `warmup` untimed steps,
    then `iters` steps each bracketed by HIP events on the launch stream with
    a 1 GiB scratch read before it (outside the events), so that no step finds
    the previous step's K/V in the last-level cache.  Returns the timing
    record, and (when want_check) host snapshots of the checked layers taken
    before any step and the GPU outputs of the first step, for the oracle."""
    from dah_testlib import host_snapshot
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    w = W.WORKLOADS[name]
    nl = w.num_layers
    seq_lens = W.make_seq_lens(w)
    table, num_pages = W.make_block_table(w, seq_lens)
    layers = [W.make_layer(w, layer, dev, table=table, num_pages=num_pages, seq_lens=seq_lens)
              for layer in range(nl)]
    B, H, L = w.batch, w.num_heads, int(seq_lens.max())
    plan = dah.plan_decode(B, L, num_splits, num_heads=H, cache_dtype=w.cache_dtype)
    ws = torch.empty(max(dah.workspace_bytes(B, L, num_splits, num_heads=H,
                                             cache_dtype=w.cache_dtype), 256),
                     dtype=torch.uint8, device=dev)
    checked = sorted({0, nl - 1})
    snaps = {c: host_snapshot(layers[c], seq_lens, table, range(B)) for c in checked} \
        if want_check else {}
    q_out = torch.empty_like(layers[0]["q"])
    o = torch.empty_like(layers[0]["q"])

    def step():
        for tl in layers:
            dah.decode_attn_step(tl["q"], tl["k_new"], tl["v_new"], tl["q_gain"], tl["k_gain"],
                                 tl["k_pool"], tl["v_pool"], tl["block_table"], tl["seq_lens"],
                                 L, rope_theta=w.rope_theta, num_splits=num_splits, q_out=q_out,
                                 o=o, workspace=ws)

    outs = {}
    if want_check:
        for c, tl in enumerate(layers):
            qo_c, o_c = dah.decode_attn_step(tl["q"], tl["k_new"], tl["v_new"], tl["q_gain"],
                                             tl["k_gain"], tl["k_pool"], tl["v_pool"],
                                             tl["block_table"], tl["seq_lens"], L,
                                             rope_theta=w.rope_theta, num_splits=num_splits,
                                             workspace=ws)
            if c in snaps:
                outs[c] = (qo_c.cpu().numpy(), o_c.cpu().numpy())
    from decode_attention_head_amd.probes import probe_read
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    for _ in range(warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        probe_read(flush, sink, 4096)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    med = float(np.median(us))
    kv = nl * W.algorithmic_kv_bytes(seq_lens, w.cache_dtype)
    rec = {
        "batch": B, "layers": nl, "heads": H, "cache": w.cache_dtype,
        "seq_lens": (f"all {L}" if int(seq_lens.min()) == L else
                     f"{int(seq_lens.min())}..{L}, sum {int(seq_lens.sum())}"),
        "plan": plan["mode"], "kernel": plan["kernel"], "workgroups": plan["workgroups"],
        "splits": plan["splits"],
        "kv_bytes_per_step": kv,
        "step_us_median": round(med, 2),
        "step_us_mean": round(float(np.mean(us)), 2),
        "step_us_min_max": [round(float(us.min()), 2), round(float(us.max()), 2)],
        "kv_gbs": round(kv / med / 1e3, 1),
        "pct_hbm_peak": round(100.0 * kv / med / 1e3 / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(B / (med * 1e-6), 1),
        "timing": f"HIP events around each of {iters} steps after {warmup} warm-up steps, "
                  f"median; a {FLUSH_BYTES >> 30} GiB scratch read before each timed step",
    }
    del layers, ws
    return rec, snaps, outs, w


def main():
    args = parse()
    if args.cpu_seconds is not None and args.cpu_seconds <= 0:   # older spelling
        args.no_cpu_baseline = True
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if args.kernel:
        os.environ["DAH_DECODE_KERNEL"] = args.kernel
    # The oracle's worker processes start before anything touches the GPU.
    pool = None if args.no_cpu_baseline else OraclePool(host_workers())
    try:
        run(args, pool)
    finally:
        if pool is not None:
            pool.close()


def run(args, pool):
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import decode_attention_head_amd as dah

    w = W.WORKLOADS[args.workload]
    nl = w.num_layers
    if nl > 1 and (args.block or args.layer or args.chunk):
        sys.exit("--block, --layer and --chunk time one-layer workloads")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    seq_lens = W.make_seq_lens(w)
    table, num_pages = W.make_block_table(w, seq_lens)
    layers = [W.make_layer(w, layer, dev, table=table, num_pages=num_pages, seq_lens=seq_lens)
              for layer in range(nl)]
    t = layers[0]
    B = w.batch
    L = int(seq_lens.max())
    H = w.num_heads
    plan = dah.plan_decode(B, L, args.num_splits, num_heads=H, cache_dtype=w.cache_dtype)
    ws_bytes = dah.workspace_bytes(B, L, args.num_splits, num_heads=H, cache_dtype=w.cache_dtype)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    q_outs = [torch.empty_like(t["q"]) for _ in range(nl)]
    o = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream(dev)

    def step(layer):
        tl = layers[layer]
        dah.decode_attn_step(tl["q"], tl["k_new"], tl["v_new"], tl["q_gain"], tl["k_gain"],
                             tl["k_pool"], tl["v_pool"], tl["block_table"], tl["seq_lens"], L,
                             rope_theta=w.rope_theta, num_splits=args.num_splits,
                             q_out=q_outs[layer], o=o, workspace=ws)

    def decode(layer):
        tl = layers[layer]
        dah.paged_decode_gqa(q_outs[layer], tl["k_pool"], tl["v_pool"], tl["block_table"],
                             tl["seq_lens"], L, num_splits=args.num_splits, o=o, workspace=ws)

    run_layer = decode if args.decode_only else step
    if args.decode_only:
        for layer in range(nl):
            step(layer)
    for _ in range(args.warmup):
        for layer in range(nl):
            run_layer(layer)
    torch.cuda.synchronize()

    # Every `every`-th timed step's calls are bracketed by HIP events; by
    # default at least 10 of them (every 2nd step of 20, every 10th of 200).
    every = args.event_every or max(1, min(10, args.steps // 10))
    timed = [i for i in range(args.steps) if i % every == every - 1] or [args.steps - 1]
    starts = {(i, layer): torch.cuda.Event(enable_timing=True) for i in timed for layer in range(nl)}
    ends = {(i, layer): torch.cuda.Event(enable_timing=True) for i in timed for layer in range(nl)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for layer in range(nl):
            ev = starts.get((i, layer))
            if ev is not None:
                ev.record(stream)
                run_layer(layer)
                ends[(i, layer)].record(stream)
            else:
                run_layer(layer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    launch_ms_all = [starts[key].elapsed_time(ends[key]) for key in starts]
    launch_ms = float(np.mean(launch_ms_all))

    if args.copy_probe > 0:
        from decode_attention_head_amd.probes import probe_copy
        src = torch.ones(args.copy_probe * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            probe_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    probe_gbs = None
    if not args.no_read_probe:
        # Practical ceiling: the K pool streamed by a plain non-temporal read
        # kernel; the best of a few grid sizes.
        from decode_attention_head_amd.probes import probe_read
        src = t["k_pool"].view(torch.uint8).reshape(-1)
        sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
        best = 0.0
        for blocks in (512, 2048, 16384):
            for _ in range(2):
                probe_read(src, sink, blocks)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(10):
                probe_read(src, sink, blocks)
            ev[1].record(stream)
            torch.cuda.synchronize()
            best = max(best, 10 * src.numel() / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9)
        probe_gbs = round(best, 1)

    kv_bytes = W.algorithmic_kv_bytes(seq_lens, w.cache_dtype)   # per layer
    paged_gbs = None
    if not args.no_read_probe and plan["mode"] == "per_sequence":
        # The decode's own access pattern without its arithmetic (one
        # workgroup per sequence, wave g reading head g's tiles of every page):
        # the ceiling of that pattern, for the one-workgroup-per-sequence plan.
        from decode_attention_head_amd.probes import probe_paged_read
        sink = torch.empty(8 * B, dtype=torch.int32, device=dev)

        def paged():
            probe_paged_read(t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], L, sink)
        for _ in range(2):
            paged()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(10):
            paged()
        ev[1].record(stream)
        torch.cuda.synchronize()
        # the same algorithmic K/V bytes as `achieved`
        paged_gbs = round(10 * kv_bytes / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9, 1)
    gbs = nl * kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (launch_ms * 1e-3) / 1e9
    default_run = args.num_splits == 0 and not args.decode_only and not args.kernel
    traffic = read_traffic(w.name) if default_run else None

    block = time_block(dah, torch, w, t, L, ws, stream, args) if args.block else None
    chunk = time_chunk(dah, torch, w, seq_lens, num_pages, args.chunk) if args.chunk > 0 else None
    layer = time_layer(dah, torch, w, t, L, args) if args.layer else None
    del layers, t, ws, q_outs, o
    torch.cuda.empty_cache()

    # The chunked-prefill record: N-token chunks at the end of the four long
    # contexts, graph-replayed, against the bf16 dense matrix-core peak.
    prefill = None
    if args.prefill_tokens > 0:
        pw = W.WORKLOADS["long_b4_s40960"]
        p_lens = W.make_seq_lens(pw)
        _, p_pages = W.make_block_table(pw, p_lens)
        prefill = time_chunk(dah, torch, pw, p_lens, p_pages, args.prefill_tokens)
        if "tflops" in prefill:
            prefill = {"workload": pw.name, **prefill,
                       "pct_bf16_dense_peak": round(100.0 * prefill["tflops"] / BF16_PEAK_TFLOPS, 2)}
        torch.cuda.empty_cache()

    # The five workloads, each timed on its own, median of args.config_iters
    # steps with the last-level cache flushed between them; then the
    # oracle leg over their sequences (CPU rate, and each config's error).
    configs = {}
    cpu = None
    if args.config_iters > 0:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        flush.fill_(1)
        for name in CONFIGS:
            rec, snaps, outs, cw = time_config(dah, torch, name, flush, args.config_iters, 5,
                                               args.num_splits, pool is not None)
            torch.cuda.empty_cache()
            if pool is not None:
                errs, osecs, oseqs, okv = [], 0.0, 0, 0
                for c, snap in snaps.items():
                    q_ref, o_ref, secs = pool.run(snap, f"{name}_{c}", cw.cache_dtype,
                                                  cw.rope_theta)
                    errs.append(oracle_errors(outs[c][0], outs[c][1], q_ref, o_ref))
                    osecs += secs
                    oseqs += len(snap["seq_lens"])
                    okv += W.algorithmic_kv_bytes(snap["seq_lens"], cw.cache_dtype)
                tol = 1e-5 if cw.cache_dtype == "f32" else 2e-2
                worst = {k: max(e[k] for e in errs) for k in ("o_max_abs", "o_rel_to_max",
                                                             "q_out_max_abs")}
                rec["parity"] = {
                    **{k: float(f"{v:.3g}") for k, v in worst.items()},
                    "tol_max_abs": tol,
                    "within": bool(all(e["finite"] for e in errs) and worst["o_max_abs"] <= tol
                                   and worst["q_out_max_abs"] <= tol and
                                   worst["o_rel_to_max"] <= 1e-4),
                    "compared": f"every sequence of layer(s) {sorted(snaps)}: o and q_out of "
                                f"the first step against the float64 oracle",
                }
                rec["oracle"] = {"seqs_per_s": round(oseqs / osecs, 2),
                                 "kv_gbs": round(okv / osecs / 1e9, 3),
                                 "seconds": round(osecs, 2), "cores": pool.workers}
                if name == "b256_s2048":
                    # The baseline proper: the same oracle over every sequence,
                    # repeated until about CPU_BASELINE_SECONDS of work.
                    snap = snaps[0]
                    reps = int(min(64, max(1, np.ceil(CPU_BASELINE_SECONDS / max(osecs, 1e-3)))))
                    _, _, ps = pool.run(snap, f"{name}_baseline", cw.cache_dtype, cw.rope_theta,
                                        repeat=reps)
                    n1 = min(len(snap["seq_lens"]), 32)
                    _, _, s1 = pool.run(snap, f"{name}_serial", cw.cache_dtype, cw.rope_theta,
                                        rows=range(n1), serial=True)
                    kv1 = W.algorithmic_kv_bytes(snap["seq_lens"][:n1], cw.cache_dtype)
                    reps1 = int(min(16, max(1, np.ceil(CPU_SINGLE_SECONDS / max(s1, 1e-3)))))
                    if reps1 > 1:
                        _, _, s1 = pool.run(snap, f"{name}_serial", cw.cache_dtype,
                                            cw.rope_theta, rows=range(n1), serial=True,
                                            repeat=reps1)
                    cpu = {
                        "value": round(reps * okv / ps / 1e9, 4),
                        "unit": "GB/s",
                        "seqs_per_s": round(reps * oseqs / ps, 2),
                        "cores": pool.workers,
                        "host_cpus": len(os.sched_getaffinity(0)),
                        "kind": "oracle",
                        "sample": f"all {oseqs} sequences of b256_s2048, {reps} passes, one "
                                  f"float64 NumPy decode step per sequence and pass, on "
                                  f"{pool.workers} worker processes ({ps:.1f} s)",
                        "single_core": {"value": round(reps1 * kv1 / s1 / 1e9, 4),
                                        "unit": "GB/s",
                                        "seqs_per_s": round(reps1 * n1 / s1, 2),
                                        "sample": f"{n1} sequences x {reps1} passes, one at a "
                                                  f"time, one core ({s1:.1f} s)"},
                    }
            configs[name] = rec
            del snaps, outs
        del flush
        torch.cuda.empty_cache()

    line = {
        "metric": "paged GQA decode KV-read GB/s (% of HBM peak) and seqs/s at B=256",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 KV, f32 compute" if w.cache_dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) q/k/v, gains 1+N(0,0.1), random block table)",
        "config": {
            "workload": w.name,
            "batch": B,
            "seq_len": "fixed 2048" if w.name.startswith("b256_s2048") else f"max {L}",
            "heads": f"{H} q / 8 kv, D=128, page 16",
            "rope_theta": w.rope_theta,
            "layers": nl,
            "kv_bytes_per_step": nl * kv_bytes,
            "plan": plan["mode"],
            "kernel": plan["kernel"],
            "workgroups": plan["workgroups"],
            "step": ("paged_decode_gqa" if args.decode_only else "decode_attn_step") +
                    (f" x {nl} layers" if nl > 1 else ""),
        },
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(B / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": (("decode_balanced_kernel" if plan["mode"] == "balanced"
                        else "decode_split_kernel") + f" [{plan['kernel']}]" +
                       ("" if args.decode_only else " (fused step)") +
                       ("" if plan["mode"] == "per_sequence" else " + combine")),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": (os.path.relpath(traffic_file(w.name), ROOT) +
                               " (rocprofv3 FETCH_SIZE and WRITE_SIZE of this kernel source, "
                               "scaled by a plain copy's counters)") if traffic else None,
            "avg_launch_us": round(launch_ms * 1e3, 2),
            "median_launch_us": round(float(np.median(launch_ms_all)) * 1e3, 2),
            "launches_timed": len(starts),
            "probe_read_gbs": probe_gbs,
            "frac_of_probe_read": None if not probe_gbs else round(achieved / probe_gbs, 4),
            "paged_read_gbs": paged_gbs,
            "frac_of_paged_read": None if not paged_gbs else round(achieved / paged_gbs, 4),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": cpu,
    }
    if configs:
        line["configs"] = configs
    if block is not None:
        line["block"] = block
    if chunk is not None:
        line["chunk"] = chunk
    if prefill is not None:
        line["prefill"] = prefill
    if layer is not None:
        line["layer"] = layer
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
