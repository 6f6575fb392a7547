"""CPU tests of the rocprofv3 summary tool (decode_attention_head_amd.rocprof_summary)
on small CSV files written here in rocprofv3's column layout."""
import csv
import os

import pytest

from decode_attention_head_amd import rocprof_summary as rs


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counters(d, rows):
    _write(os.path.join(d, "host", "run_counter_collection.csv"),
           ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
           [(i, k, c, v) for i, (k, c, v) in enumerate(rows)])


def test_trace_summary(tmp_path):
    _write(os.path.join(tmp_path, "host", "run_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [("void decode_split_kernel<1, true, 2, true>(DecodeArgs)", 55, 1, 324430.0, 56.0,
             317840.0, 438740.0)])
    out = rs.trace_summary(str(tmp_path)).splitlines()
    assert out[1].split()[-5:] == ["55", "324.43", "317.84", "438.74", "56.00"]


def test_traffic_summary_scales_by_the_copy_probe(tmp_path):
    fetch, write = os.path.join(tmp_path, "f"), os.path.join(tmp_path, "w")
    # The copy moves 1 MiB each way; FETCH_SIZE reads half of it (factor 2).
    _counters(fetch, [("probe_copy_kernel(...)", "FETCH_SIZE", 512.0),
                      ("decode_split_kernel<...>", "FETCH_SIZE", 1000.0),
                      ("decode_split_kernel<...>", "FETCH_SIZE", 1002.0)])
    _counters(write, [("probe_copy_kernel(...)", "WRITE_SIZE", 1024.0),
                      ("decode_split_kernel<...>", "WRITE_SIZE", 10.0)])
    got = dict(ln.split(": ") for ln in rs.traffic_summary(fetch, write, 1).splitlines())
    assert float(got["fetch_scale"]) == 2.0 and float(got["write_scale"]) == 1.0
    assert float(got["decode_fetch_bytes_per_launch"]) == 2 * 1001.0 * 1024
    assert float(got["hbm_bytes_per_launch"]) == (2 * 1001.0 + 10.0) * 1024


def test_counters_summary_merges_runs_and_forms_ratios(tmp_path):
    a, b = os.path.join(tmp_path, "a"), os.path.join(tmp_path, "b")
    k = "void chunk_prefill_kernel<2, 8>(ChunkArgs)"
    _counters(a, [(k, "SQ_WAVES", 4096.0), (k, "SQ_INSTS_LDS", 100.0), (k, "SQ_INSTS_LDS", 300.0),
                  (k, "SQ_LDS_BANK_CONFLICT", 50.0), ("other_kernel", "SQ_WAVES", 1.0)])
    _counters(b, [(k, "SQ_INSTS_VALU", 8192.0)])
    out = rs.counters_summary([a, b], ["chunk_prefill"])
    vals = {ln.split()[0]: ln.split()[1] for ln in out.splitlines()[2:] if len(ln.split()) == 2}
    assert float(vals["SQ_INSTS_LDS"]) == 200.0          # mean per dispatch
    assert float(vals["SQ_INSTS_VALU"]) == 8192.0       # from the second run
    assert "bank-conflict cycles per LDS instr 0.2500" in " ".join(out.split())
    assert "SQ_INSTS_VALU per wave 2.0" in " ".join(out.split())


def test_counters_summary_wants_one_kernel_per_name(tmp_path):
    _counters(str(tmp_path), [("decode_split_kernel<1>", "SQ_WAVES", 1.0),
                              ("decode_split_kernel<2>", "SQ_WAVES", 1.0)])
    with pytest.raises(ValueError):
        rs.counters_summary([str(tmp_path)], ["decode_split_kernel"])


def test_pair_summary_times_decode_gap_and_merge(tmp_path):
    # two steps: decode 50 us, 3 us idle, merge 4 us; an unrelated kernel between steps
    rows = []
    t = 1_000_000
    for i in range(2):
        rows.append(("KERNEL_DISPATCH", "void decode_split_kernel<1, true, 2, false>(DecodeArgs)",
                     t, t + 50_000))
        rows.append(("KERNEL_DISPATCH", "combine_splits_kernel(float const*, ...)",
                     t + 53_000, t + 57_000))
        rows.append(("KERNEL_DISPATCH", "probe_read_kernel(...)", t + 60_000, t + 61_000))
        t += 100_000
    _write(os.path.join(tmp_path, "host", "run_kernel_trace.csv"),
           ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = rs.pair_summary(str(tmp_path), "decode_split_kernel", "combine").splitlines()
    assert out[0].startswith("pairs: 2")
    assert out[2].split()[-2:] == ["50.00", "50.00"]
    assert out[3].split()[-2:] == ["3.00", "3.00"]
    assert out[4].split()[-2:] == ["4.00", "4.00"]
    assert out[5].split()[-2:] == ["57.00", "57.00"]
