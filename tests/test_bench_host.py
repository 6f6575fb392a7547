"""CPU checks of bench.py's host-side pieces: the oracle leg's process pool
returns exactly what the oracle computes in-process (same sequences, same
order, every row), in both its parallel and its single-core mode and over
repeated passes, and the
benchmark refuses more than one GPU before touching any device."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import decode_attention as O  # noqa: E402


def _snapshot(seed=3):
    r = np.random.default_rng(seed)
    lens = np.array([1, 16, 17, 90, 300, 41], np.int64)
    pages = [(-(-int(n) // 16)) for n in lens]
    total = sum(pages)
    table = np.zeros((len(lens), max(pages)), np.int32)
    perm = r.permutation(total + 3)
    at = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[at:at + n]
        at += n

    def bits(shape):
        x = r.standard_normal(shape).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return {"q": r.standard_normal((len(lens), 16, 128)).astype(np.float32),
            "k_new": r.standard_normal((len(lens), 8, 128)).astype(np.float32),
            "v_new": r.standard_normal((len(lens), 8, 128)).astype(np.float32),
            "q_gain": (1 + 0.1 * r.standard_normal(128)).astype(np.float32),
            "k_gain": (1 + 0.1 * r.standard_normal(128)).astype(np.float32),
            "k_pool": bits((total + 3, 8, 16, 128)), "v_pool": bits((total + 3, 8, 16, 128)),
            "block_table": table, "seq_lens": lens}


def test_oracle_pool_matches_in_process_oracle():
    snap = _snapshot()
    want = O.decode_step(snap["q"], snap["k_new"], snap["v_new"], snap["q_gain"],
                         snap["k_gain"], snap["k_pool"], snap["v_pool"], snap["block_table"],
                         snap["seq_lens"], "bf16", theta=5e6)
    pool = bench.OraclePool(2)
    try:
        q_out, o, secs = pool.run(snap, "t", "bf16", 5e6)
        assert secs > 0
        assert np.array_equal(q_out, want["q_out"]) and np.array_equal(o, want["o"])
        q1, o1, _ = pool.run(snap, "s", "bf16", 5e6, rows=[4, 0, 2], serial=True)
        assert np.array_equal(o1, want["o"][[4, 0, 2]])
        assert np.array_equal(q1, want["q_out"][[4, 0, 2]])
        # repeated passes (the baseline's timing) return the same rows
        q3, o3, _ = pool.run(snap, "r", "bf16", 5e6, repeat=3)
        assert np.array_equal(q3, want["q_out"]) and np.array_equal(o3, want["o"])
    finally:
        pool.close()
    for path in pool.dirs:
        assert not os.path.exists(path)


def test_oracle_errors_report():
    ref = np.ones((2, 16, 128))
    got = ref.copy()
    got[1, 3, 5] += 0.5
    e = bench.oracle_errors(ref * 2, got, ref * 2, ref)
    assert e["o_max_abs"] == 0.5 and e["o_rel_to_max"] == 0.5 and e["q_out_max_abs"] == 0.0
    assert e["finite"]


def test_bench_refuses_several_gpus():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr
