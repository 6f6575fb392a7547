"""Benchmark of the decode-attention block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b256_s2048]

A step is one pass of the whole hot path over the batch: one call of
decode_attn_step (q/k RMSNorm, RoPE, cache append and split-S decodeGQA, in
one kernel launch when one split suffices, plus the log-sum-exp combine
otherwise) per layer of the workload -- one for every workload but
stack28_b128, whose step runs its 28 layers, each with its own cache and
gains.  HIP events recorded on the launch stream bracket the layer calls of
every --event-every'th step (default 10): an event pair costs ~7 us of GPU
time per step, which would otherwise be counted into the step time.  Inputs
are synthetic, seeded and resident in HBM before timing starts.

The JSON line reports
  value           KV-read throughput, GB/s = (sum of seq_lens * 4096 B) / step time
  roofline        the step's decode kernel (dominant kernel): algorithmic KV
                  bytes per launch / its average duration measured with HIP
                  events on the launch stream, against MI355X's 8 TB/s HBM peak
  cpu_baseline    the float64 CPU oracle on a bounded sample of the same workload

--chunk N also times chunk_attn_step with N new tokens per sequence (the
workload's lengths counting them), under "chunk": HIP-graph-replayed time,
K/V bytes (each cached position once per sequence) and attention flops.

--layer also times decoder_layer_step (input_norm, the block with its
projections, residuals, SwiGLU MLP) on the same batch, graph-replayed.

--block also times the projections on either side of the block (attn.qkv_proj
before the step, attn.o_proj after it) on the same batch and reports them under
"block": per-launch durations (HIP events), their bytes and flops, and the
whole x -> qkv_proj -> decode_attn_step -> o_proj pass.
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
    ap.add_argument("--event-every", type=int, default=10, metavar="N",
                    help="bracket the calls of every N-th timed step with HIP events")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time paged_decode_gqa alone (profiling aid)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming-read probe (practical bandwidth ceiling) and the "
                         "paged-read probe (the decode's access pattern alone)")
    ap.add_argument("--chunk", type=int, default=0, metavar="N",
                    help="also time chunk_attn_step with N new tokens per sequence")
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


def cpu_baseline(w, t, seq_lens, table, budget_s):
    """Time the oracle's decode step, one sequence at a time, until the
    budget is spent.  Host copies of each sequence's pages are made before
    its timer starts."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import decode_attention as O
    from dah_testlib import host_snapshot
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    order = np.random.default_rng(7).permutation(len(seq_lens))
    done, elapsed, kv_bytes = 0, 0.0, 0
    for b in order:
        snap = host_snapshot(t, seq_lens, table, [int(b)])
        t0 = time.perf_counter()
        O.decode_step(snap["q"], snap["k_new"], snap["v_new"], snap["q_gain"], snap["k_gain"],
                      snap["k_pool"], snap["v_pool"], snap["block_table"], snap["seq_lens"],
                      w.cache_dtype, theta=w.rope_theta)
        elapsed += time.perf_counter() - t0
        done += 1
        kv_bytes += W.algorithmic_kv_bytes(seq_lens[[int(b)]], w.cache_dtype)
        if elapsed >= budget_s:
            break
    return {
        "value": kv_bytes / elapsed / 1e9,
        "unit": "GB/s",
        "seqs_per_s": done / elapsed,
        "cores": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{done} of {len(seq_lens)} sequences of {w.name}, full decode step each "
                  f"(float64 NumPy, {elapsed:.1f} s)",
    }


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
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
    q_out = q_outs[0]
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

    run = decode if args.decode_only else step
    if args.decode_only:
        for layer in range(nl):
            step(layer)
    for _ in range(args.warmup):
        for layer in range(nl):
            run(layer)
    torch.cuda.synchronize()

    every = max(1, args.event_every)
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
                run(layer)
                ends[(i, layer)].record(stream)
            else:
                run(layer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    launch_ms = float(np.mean([starts[key].elapsed_time(ends[key]) for key in starts]))

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
    traffic = read_traffic(w.name) if (args.num_splits == 0 and not args.decode_only) else None

    block = time_block(dah, torch, w, t, L, ws, stream, args) if args.block else None
    chunk = time_chunk(dah, torch, w, seq_lens, num_pages, args.chunk) if args.chunk > 0 else None
    layer = time_layer(dah, torch, w, t, L, args) if args.layer else None

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, t, seq_lens, table, args.cpu_seconds)

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
            "avg_launch_us": round(launch_ms * 1e3, 2),
            "launches_timed": len(starts),
            "probe_read_gbs": probe_gbs,
            "frac_of_probe_read": None if not probe_gbs else round(achieved / probe_gbs, 4),
            "paged_read_gbs": paged_gbs,
            "frac_of_paged_read": None if not paged_gbs else round(achieved / paged_gbs, 4),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": cpu,
    }
    if block is not None:
        line["block"] = block
    if chunk is not None:
        line["chunk"] = chunk
    if layer is not None:
        line["layer"] = layer
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
