"""Host logic of bench.py's trace summary: the dominant kernel's in-stack mean
and the timing loop's are split by dispatch order, and the bench line takes
the in-stack figure only while the kernel's sources match the recorded hash."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _write_trace(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, start, dur_ns in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start,
                        "End_Timestamp": start + dur_ns})


def test_summarize_trace_splits_stack_and_loop(tmp_path, monkeypatch):
    dom = "void q4::(anonymous namespace)::%s(q4::Args)" % bench.DOMINANT_KERNEL
    other = "void q4::(anonymous namespace)::k_gemv<64, 4, 1, 2, 0, false>(q4::Args)"
    loop_n = bench.DOMINANT_REPS * bench.PHI3["layers"]
    rows, t = [], 1_000
    for i in range(200):  # the stack's tokens: 8000 ns each, with other kernels between
        rows.append((dom, t, 8000)); t += 10_000
        rows.append((other, t, 5000)); t += 10_000
    for i in range(loop_n):  # the timing loop: 7000 ns each
        rows.append((dom, t, 7000)); t += 10_000
    rows.reverse()  # the summary sorts by start time
    trace = tmp_path / "trace.csv"
    _write_trace(trace, rows)
    out = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "STACK_TRACE_PROFILE", str(out))
    bench.summarize_trace(str(trace), "0")
    rec = [json.loads(l) for l in open(out) if l.startswith("{")][-1]
    assert rec["in_stack_dispatches"] == 200 and rec["loop_dispatches"] == loop_n
    assert rec["in_stack_us"] == pytest.approx(8.0) and rec["loop_us"] == pytest.approx(7.0)
    assert rec["bytes_per_launch"] == 28311552
    assert rec["source_hash"] == bench.kernel_source_hash()

    line = bench.in_stack_line(28311552.0)
    assert line["us_per_launch"] == pytest.approx(8.0)
    assert line["frac"] == pytest.approx(28311552 / 8e-6 / 1e9 / bench.HBM_PEAK_GBS, abs=1e-4)

    # other kernel sources, or another kernel size: not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.in_stack_line(28311552.0) is None


def test_summarize_trace_needs_the_loop(tmp_path, monkeypatch):
    dom = "void q4::(anonymous namespace)::%s(q4::Args)" % bench.DOMINANT_KERNEL
    trace = tmp_path / "trace.csv"
    _write_trace(trace, [(dom, 1000 + 10_000 * i, 7000) for i in range(10)])
    monkeypatch.setattr(bench, "STACK_TRACE_PROFILE", str(tmp_path / "summary.md"))
    with pytest.raises(SystemExit):
        bench.summarize_trace(str(trace), "0")
