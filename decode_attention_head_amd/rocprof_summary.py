"""Condense rocprofv3 CSV output of the benchmark into the short text
summaries kept under profiles/.

    python -m decode_attention_head_amd.rocprof_summary trace DIR --out FILE --cmd "..."
    python -m decode_attention_head_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR \
        --copy-mib 1024 --out FILE --cmd "..."

`trace` lists per-kernel call counts and durations from a --kernel-trace
--stats run.  `counters` lists the mean per dispatch of every counter in
one or more --pmc runs for the kernels named by --kernel (substrings), with
a few ratios (waves, instructions per wave, LDS bank-conflict cycles per LDS
instruction).  `traffic` turns FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
two separate --pmc runs) into HBM bytes per decode launch, each counter
scaled by what it reads for the probe copy kernel, whose traffic is known
exactly (copy-mib MiB read and the same written).  The summary records a
digest of the kernel source, so a reader can tell whether the counters
still describe the current kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(PKG, "csrc", "dah_kernels.hip")
DECODE_KERNEL = "decode_split_kernel"
COPY_KERNEL = "probe_copy_kernel"


def source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= 70 else name[:67] + "..."


def trace_summary(d: str) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    out = [f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        out.append(f"{_short(r['Name']):70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                   f"{float(r['Percentage']):6.2f}")
    return "\n".join(out)


def pair_summary(d: str, first: str, second: str) -> str:
    """Per step of a split or balanced plan: the decode launch (kernel names
    containing `first`), the idle time until the merge launch (`second`) that
    follows it on the same queue starts, the merge launch, and the span from
    the decode's start to the merge's end -- from the start and end
    timestamps of a --kernel-trace run."""
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv")))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dec, gap, mrg, span = [], [], [], []
    for a, b in zip(rows, rows[1:]):
        if first in a["Kernel_Name"] and second in b["Kernel_Name"]:
            s0, e0 = int(a["Start_Timestamp"]), int(a["End_Timestamp"])
            s1, e1 = int(b["Start_Timestamp"]), int(b["End_Timestamp"])
            dec.append(e0 - s0)
            gap.append(s1 - e0)
            mrg.append(e1 - s1)
            span.append(e1 - s0)
    if not dec:
        return f"no {first} launch followed by {second}"

    def stat(v):
        v = sorted(v)
        return f"{sum(v) / len(v) / 1e3:10.2f} {v[len(v) // 2] / 1e3:10.2f}"
    return "\n".join([
        f"pairs: {len(dec)}  ({first} -> {second})",
        f"{'':24s} {'avg_us':>10s} {'median_us':>10s}",
        f"{'decode launch':24s} {stat(dec)}",
        f"{'gap before the merge':24s} {stat(gap)}",
        f"{'merge launch':24s} {stat(mrg)}",
        f"{'decode start to merge end':24s} {stat(span)}",
    ])


def _counter_means(d: str, counter: str):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    agg = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def _pick(means: dict, key: str) -> float:
    hits = [v for k, v in means.items() if key in k]
    if len(hits) != 1:
        raise ValueError(f"expected one kernel matching {key!r}, found {len(hits)}")
    return hits[0]


def traffic_summary(fetch_dir: str, write_dir: str, copy_mib: int) -> str:
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_scale = copy_kib / _pick(fetch, COPY_KERNEL)
    w_scale = copy_kib / _pick(write, COPY_KERNEL)
    d_fetch = _pick(fetch, DECODE_KERNEL)
    d_write = _pick(write, DECODE_KERNEL)
    hbm = (d_fetch * f_scale + d_write * w_scale) * 1024.0
    lines = [
        f"kernel_source_sha256_16: {source_digest()}",
        f"copy_probe_bytes_each_way: {copy_mib * 1024 * 1024}",
        f"copy_probe_FETCH_SIZE_KiB: {_pick(fetch, COPY_KERNEL):.3f}",
        f"copy_probe_WRITE_SIZE_KiB: {_pick(write, COPY_KERNEL):.3f}",
        f"fetch_scale: {f_scale:.6f}",
        f"write_scale: {w_scale:.6f}",
        f"decode_FETCH_SIZE_KiB_per_launch: {d_fetch:.3f}",
        f"decode_WRITE_SIZE_KiB_per_launch: {d_write:.3f}",
        f"decode_fetch_bytes_per_launch: {d_fetch * f_scale * 1024.0:.0f}",
        f"decode_write_bytes_per_launch: {d_write * w_scale * 1024.0:.0f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
    ]
    return "\n".join(lines)


def _all_counter_means(d: str):
    """{kernel name: {counter: mean value per dispatch}} of one --pmc run."""
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}


def counters_summary(dirs, kernels) -> str:
    out = [f"kernel_source_sha256_16: {source_digest()}"]
    for key in kernels:
        merged = {}
        name = None
        for d in dirs:
            hits = {k: v for k, v in _all_counter_means(d).items() if key in k}
            if len(hits) != 1:
                raise ValueError(f"{d}: expected one kernel matching {key!r}, found {len(hits)}")
            (name, vals), = hits.items()
            merged.update(vals)
        out.append(f"[{_short(name)}]")
        for c in sorted(merged):
            out.append(f"  {c:32s} {merged[c]:20.3f}")
        waves = merged.get("SQ_WAVES")
        if waves:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
                      "SQ_INSTS_SALU"):
                if c in merged:
                    out.append(f"  {c + ' per wave':32s} {merged[c] / waves:20.1f}")
        if merged.get("SQ_INSTS_LDS"):
            if "SQ_LDS_BANK_CONFLICT" in merged:
                out.append(f"  {'bank-conflict cycles per LDS instr':32s} "
                           f"{merged['SQ_LDS_BANK_CONFLICT'] / merged['SQ_INSTS_LDS']:20.4f}")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--pair", nargs=2, metavar=("DECODE", "MERGE"),
                   help="also time each DECODE launch, the gap and the MERGE launch after it")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("--copy-mib", type=int, required=True)
    n = sub.add_parser("counters")
    n.add_argument("dirs", nargs="+")
    n.add_argument("--kernel", action="append", required=True,
                   help="substring naming one kernel in every run (repeatable)")
    for p in (t, c, n):
        p.add_argument("--out", required=True)
        p.add_argument("--cmd", action="append", default=[],
                       help="command that produced the data (repeatable)")
        p.add_argument("--note", default="")
    a = ap.parse_args()
    if a.mode == "trace":
        body = trace_summary(a.dir)
        if a.pair:
            body += "\n" + pair_summary(a.dir, *a.pair)
    elif a.mode == "traffic":
        body = traffic_summary(a.fetch_dir, a.write_dir, a.copy_mib)
    else:
        body = counters_summary(a.dirs, a.kernel)
    head = [f"# rocprofv3 {a.mode} summary"]
    head += [f"# command: {c}" for c in a.cmd]
    if a.note:
        head.append(f"# {a.note}")
    with open(a.out, "w") as f:
        f.write("\n".join(head) + "\n" + body + "\n")
    print(open(a.out).read())


if __name__ == "__main__":
    main()
