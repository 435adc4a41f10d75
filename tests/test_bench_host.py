"""bench.py's host logic, on the CPU: the split of a profiler's dispatches by
the line's launch sequence, the kernel-trace and counter summaries written
for profiles/ (from synthetic rocprofv3 CSV files of known values), the
counter record that the line's roofline takes only at a matching kernel
source hash, and the multi-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_split_by_launch_sequence():
    rows = list(range(10))
    seq = [["a", [2, 3]], ["b", [4]], ["c", [5]]]
    out = bench._split(rows, seq)
    assert out == {"a": [[0, 1], [2, 3, 4]], "b": [[5, 6, 7, 8]]}   # c is not fully covered


def _trace_rows(sequence, durations):
    """kernel_trace.csv rows, one per dispatch in launch order: workload w's
    phase p launches take durations[w][p] ns each; a foreign kernel sits
    between every two of ours (it must be ignored)."""
    rows, t, did = [], 1000, 0
    for name, counts in sequence:
        for p, cnt in enumerate(counts):
            for _ in range(cnt):
                d = durations[name][p]
                did += 1
                rows.append({"Kernel_Name": "void ecmd::k_linear<%s>" % name, "Dispatch_Id": did,
                             "Start_Timestamp": t, "End_Timestamp": t + d})
                t += d + 100
                did += 1
                rows.append({"Kernel_Name": "at::native::reduce_kernel", "Dispatch_Id": did,
                             "Start_Timestamp": t, "End_Timestamp": t + 50})
                t += 150
    return rows


def test_summarize_trace(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    seq = [["headline:axpby_f32", [3, 4, 4]], ["headline:axpby_f32@staggered", [2, 4]],
           ["copy_f32", [2, 5, 3, 3, 1]]]
    # ns per launch, per phase
    dur = {"headline:axpby_f32": [9000, 500000, 510000], "headline:axpby_f32@staggered": [9000, 490000],
           "copy_f32": [9000, 320000, 321000, 325000, 330000]}
    d = tmp_path / "kt"
    _write_csv(str(d / "kt_kernel_trace.csv"), _trace_rows(seq, dur))
    _write_csv(str(d / "kt_kernel_stats.csv"), [{"Name": "void ecmd::k_linear<copy_f32>", "Calls": 14}])
    line = {"kernel_source_hash": "feedbeef", "launch_sequence": seq, "step_us": {"median_us": 502.0},
            "placement": {"step_us": {"median_us": 491.0}},
            "commands": {"copy_f32": {"cold": {"median_us": 326.0}, "warm": {"avg_us": 321.0}}}}
    bj = tmp_path / "line.json"
    bj.write_text("noise\n" + json.dumps(line) + "\n")
    bench.summarize_trace(str(d), str(bj), "the command")
    table = open(os.path.join(bench.PROFILES, "kernel_trace_summary.md")).read()
    assert "the command" in table and "feedbeef" in table
    rows = {r.split("|")[1].strip(): [c.strip() for c in r.split("|")[2:]] for r in table.splitlines()
            if r.startswith("| ") and not r.startswith("| workload")}
    # the headline's cold steps are its second phase; a command's cold launches its fourth, its
    # back-to-back launches its second
    assert rows["headline:axpby_f32"][1] == "500.000" and rows["headline:axpby_f32"][2] == "502.000"
    assert rows["headline:axpby_f32@staggered"][1] == "490.000" and rows["headline:axpby_f32@staggered"][2] == "491.000"
    assert rows["copy_f32"][1] == "325.000" and rows["copy_f32"][2] == "326.000"
    assert rows["copy_f32"][6] == "320.000" and rows["copy_f32"][7] == "321.000"
    per = open(os.path.join(bench.PROFILES, "kernel_trace_copy_f32.txt")).read()
    assert "Calls: 14" in per and "kernel source hash: feedbeef" in per
    assert os.path.exists(os.path.join(bench.PROFILES, "kernel_trace_headline_axpby_f32_staggered.txt"))


def _counter_rows(sequence, kib):
    rows, did = [], 0
    for name, counts in sequence:
        for cnt in counts:
            for _ in range(cnt):
                did += 1
                rows.append({"Kernel_Name": "void ecmd::k_linear<%s>" % name, "Dispatch_Id": did,
                             "Start_Timestamp": did * 10, "Counter_Name": "X", "Counter_Value": kib[name]})
    # the cache flush: a foreign kernel reading 1 GiB
    did += 1
    rows.append({"Kernel_Name": "at::native::reduce_kernel", "Dispatch_Id": did, "Start_Timestamp": did * 10,
                 "Counter_Name": "X", "Counter_Value": 524288.0})
    return rows


def test_summarize_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    seq = [["headline:axpby_f32", [1, 2, 2]], ["copy_f32", [1, 2, 2, 2, 1]], ["axpby_f32", [1, 2, 2, 2, 1]]]
    line = {"launch_sequence": seq}
    for counter, kib in (("FETCH_SIZE", {"headline:axpby_f32": 1.0, "copy_f32": 524288.0, "axpby_f32": 1048600.0}),
                         ("WRITE_SIZE", {"headline:axpby_f32": 1.0, "copy_f32": 1048576.0, "axpby_f32": 1048576.0})):
        _write_csv(str(tmp_path / counter / "p_counter_collection.csv"), _counter_rows(seq, kib))
        (tmp_path / (counter + ".json")).write_text(json.dumps(line) + "\n")
    bench.summarize_counters(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "FETCH_SIZE.json"),
                             str(tmp_path / "WRITE_SIZE"), str(tmp_path / "WRITE_SIZE.json"), "cmd")
    rec = json.load(open(os.path.join(bench.PROFILES, "counters_axpby_f32.json")))
    rd, wr = W.algorithmic_read_write("axpby_f32")
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_scale_from_flush"] == pytest.approx(2.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(1048600.0 * 1024 * 2.0)
    assert rec["read_ratio"] == pytest.approx(1048600.0 * 1024 * 2.0 / rd)
    assert rec["write_ratio"] == pytest.approx(1048576.0 * 1024 / wr)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    assert not os.path.exists(os.path.join(bench.PROFILES, "counters_headline_axpby_f32.json"))
    summary = open(os.path.join(bench.PROFILES, "counters_summary.md")).read()
    assert "scaled by 2.0000" in summary and "| axpby_f32 |" in summary


def test_counters_record_needs_the_current_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "counters_axpby_f32.json").write_text(json.dumps({"kernel_source_hash": "old", "x": 1}))
    assert bench.counters_record("axpby_f32", "new") is None
    assert bench.counters_record("axpby_f32", "old")["x"] == 1
    assert bench.counters_record("copy_f32", "old") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_summarize_lds(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    seq = [["headline:transposed_2d", [1, 2, 2]], ["transposed_2d", [1, 2, 2, 2, 1]]]
    rows, did = [], 0
    for name, counts in seq:
        for cnt in counts:
            for _ in range(cnt):
                did += 1
                for c, v in (("SQ_INSTS_LDS", 64.0), ("SQ_LDS_IDX_ACTIVE", 200.0),
                             ("SQ_LDS_BANK_CONFLICT", 10.0 if name == "transposed_2d" else 0.0)):
                    rows.append({"Kernel_Name": "void ecmd::k_tiled<%s>" % name, "Dispatch_Id": did,
                                 "Start_Timestamp": did * 10, "Counter_Name": c, "Counter_Value": v})
    _write_csv(str(tmp_path / "lds" / "p_counter_collection.csv"), rows)
    bj = tmp_path / "lds.json"
    bj.write_text(json.dumps({"kernel_source_hash": "abc", "launch_sequence": seq}) + "\n")
    bench.summarize_lds(str(tmp_path / "lds"), str(bj), "the command")
    text = open(os.path.join(bench.PROFILES, "lds_bank_conflicts.md")).read()
    row = [r for r in text.splitlines() if r.startswith("| transposed_2d |")]
    assert len(row) == 1 and "| 8 | 64 | 200 | 10 | 5.00 % |" in row[0], row
    assert "headline:" not in text and "the command" in text
