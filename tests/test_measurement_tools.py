"""The measurement bookkeeping on the CPU: counter averaging and scaling,
the fused-launch byte model, the source-hash and key rules that decide when
bench.py may report a counted figure, the kernel-trace summary's launch
selection, and the per-row distinct-key counts behind the state bytes.

The figures are synthetic (hand-made counter CSVs and a hand-made trace
database); each expected value follows from the rule under test.
"""
import argparse
import csv
import json
import sqlite3

import numpy as np
import pytest

import bench
from sparse_attention_kv_request_amd import counters, profile_summary, workloads

KIB = 1024


def _counter_csv(path, kernel, counter, values, other=None):
    """One row per dispatch of `kernel` (and of `other` in between)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Grid_Size"])
        w.writeheader()
        d = 0
        for v in values:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": v, "Grid_Size": 1024})
            d += 1
            if other:
                w.writerow({"Dispatch_Id": d, "Kernel_Name": other, "Counter_Name": counter,
                            "Counter_Value": 999999, "Grid_Size": 1024})
                d += 1


@pytest.fixture
def counter_files(tmp_path, monkeypatch):
    """Calibration that reads exactly the copied bytes (factor 1) on WRITE_SIZE
    and half of them on FETCH_SIZE (factor 2, as the MI355X runs read), and a
    kernel with 3 warm-up and 4 timed dispatches."""
    calib_kib = counters.CALIB_BYTES / KIB
    _counter_csv(tmp_path / "cf.csv", "__amd_rocclr_copyBuffer", "FETCH_SIZE", [calib_kib / 2] * 3)
    _counter_csv(tmp_path / "cw.csv", "__amd_rocclr_copyBuffer", "WRITE_SIZE", [calib_kib] * 3)
    fetch = [10_000.0] * 3 + [100.0, 200.0, 300.0, 400.0]      # KiB per dispatch
    write = [10_000.0] * 3 + [50.0, 50.0, 50.0, 50.0]
    _counter_csv(tmp_path / "f.csv", "hisparse::lru_token_plan<1024, 2, 4>", "FETCH_SIZE", fetch,
                 other="hisparse::miss_copy<256, 4>")
    _counter_csv(tmp_path / "w.csv", "hisparse::lru_token_plan<1024, 2, 4>", "WRITE_SIZE", write,
                 other="hisparse::miss_copy<256, 4>")
    monkeypatch.setattr(counters, "COUNTERS", tmp_path / "traffic.json")
    return tmp_path


def _record(tmp, kernel, workload, line, fused=False):
    (tmp / "line.json").write_text("noise\n" + json.dumps(line) + "\n")
    args = argparse.Namespace(
        fetch=str(tmp / "f.csv"), write=str(tmp / "w.csv"), calib_fetch=str(tmp / "cf.csv"),
        calib_write=str(tmp / "cw.csv"), kernel=kernel, match="", calib_kernel="copyBuffer",
        skip=3, limit=0, workload=workload, warmup=5, steps=20,
        bench_line=str(tmp / "line.json"), fused=fused, cmd="test")
    counters.record(args)
    key = counters.traffic_key(kernel, workload, 5, 20)
    return json.loads(counters.COUNTERS.read_text())["entries"][key]


def test_record_scales_by_the_calibration_and_skips_warmup(counter_files):
    line = {"state_roofline": {"bytes_per_launch": 300_000,
                               "kernel_model_bytes_per_launch": 250_000},
            "roofline": {"bytes_per_launch": 1_000_000}}
    e = _record(counter_files, "lru_token_plan", "2 split", line)
    # mean of the 4 timed dispatches (250 KiB fetch, 50 KiB write), the other
    # kernel's rows ignored; FETCH_SIZE doubled by the calibration
    assert e["fetch_bytes_per_launch"] == 2 * 250 * KIB
    assert e["write_bytes_per_launch"] == 50 * KIB
    assert e["traffic_bytes_per_launch"] == 550 * KIB
    assert e["algorithmic_bytes_per_launch"] == 300_000
    assert e["traffic_over_algorithmic"] == round(550 * KIB / 300_000, 3)
    assert e["traffic_over_kernel_model"] == round(550 * KIB / 250_000, 3)


def test_fused_launches_add_the_copied_bytes(counter_files):
    """A launch that copies its misses moves the state bytes plus every miss
    read from the host tier and written to HBM."""
    line = {"state_roofline": {"bytes_per_launch": 300_000,
                               "kernel_model_bytes_per_launch": 250_000},
            "roofline": {"bytes_per_launch": 1_000_000}}
    e = _record(counter_files, "lru_token_plan", "2", line, fused=True)
    assert e["algorithmic_bytes_per_launch"] == 300_000 + 2 * 1_000_000
    assert e["kernel_model_bytes_per_launch"] == 250_000 + 2 * 1_000_000


def test_copy_kernel_bytes_are_read_plus_write(counter_files):
    line = {"roofline": {"bytes_per_launch": 123_456}}
    e = _record(counter_files, "miss_copy", "1", line)
    assert e["algorithmic_bytes_per_launch"] == 2 * 123_456


def test_traffic_is_reported_only_for_the_same_sources_and_launches(counter_files,
                                                                     monkeypatch):
    line = {"state_roofline": {"bytes_per_launch": 1}, "roofline": {"bytes_per_launch": 1}}
    e = _record(counter_files, "lru_token_plan", "2", line, fused=True)
    want = e["traffic_bytes_per_launch"]
    assert bench.traffic_from_profiles("lru_token_plan", 2, 5, 20) == want
    # another warm-up, step count or workload: not the launches counted
    assert bench.traffic_from_profiles("lru_token_plan", 2, 2, 20) is None
    assert bench.traffic_from_profiles("lru_token_plan", 2, 5, 10) is None
    assert bench.traffic_from_profiles("lru_token_plan", "2 split", 5, 20) is None
    # changed sources: the figure no longer applies
    monkeypatch.setattr(counters, "kernel_hash", lambda k: "0" * 16)
    assert bench.traffic_from_profiles("lru_token_plan", 2, 5, 20) is None


def test_kernel_hash_covers_the_fusion_rule():
    """The rule that lets a call copy inside the plan kernel lives in copy.h,
    so the plan kernels' counted figures depend on it."""
    for k in ("lru_token_plan", "lru_page_plan", "clock_plan", "miss_copy"):
        assert "copy.h" in counters.KERNEL_SOURCES[k]


def test_profile_summary_selects_the_timed_launches(tmp_path):
    db = tmp_path / "run.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, duration integer)")
    t = 0
    # plan: 2 warm-up (1000 ns), 3 timed (2000 ns), 2 later (9000 ns); copy: 1 probe, 3 timed
    rows = ([("void hisparse::(anonymous namespace)::plan_k<1024, 2>(PlanArgs)", 1000)] * 2 +
            [("void hisparse::(anonymous namespace)::plan_k<1024, 2>(PlanArgs)", 2000)] * 3 +
            [("void hisparse::(anonymous namespace)::plan_k<1024, 2>(PlanArgs)", 9000)] * 2 +
            [("void hisparse::(anonymous namespace)::copy_k(CopyArgs)", 50000)] +
            [("void hisparse::(anonymous namespace)::copy_k(CopyArgs)", 4000)] * 3)
    for name, dur in rows:
        con.execute("insert into kernels values (?, ?, ?)", (name, t, dur))
        t += 10
    con.commit()
    con.close()
    out = {r[0]: r for r in profile_summary.summarize(str(db), 2, 3, {"copy_k": 1})}
    plan, copy = out["plan_k<1024, 2>"], out["copy_k"]
    assert plan[1] == 7 and plan[3] == 3 and plan[4] == pytest.approx(2.0)
    assert copy[1] == 4 and copy[3] == 3 and copy[4] == pytest.approx(4.0)


def test_distinct_keys_count_tokens_over_steps_and_pages():
    trace = np.array([[[[[5, 5, 7, -1], [7, 9, -1, 5]]]]], np.int32)   # [L, T, B, S, K]
    w = workloads.config(3, batch=1, layers=1, steps=1, num_steps=2, top_k=4)
    assert bench.distinct_keys(w, trace)[0, 0, 0] == 3                   # {5, 7, 9}
    wp = workloads.config(5, batch=1, layers=1, steps=1, top_k=4)
    pages = np.array([[[[[0, wp.page_size - 1, wp.page_size, 3 * wp.page_size]]]]], np.int32)
    assert bench.distinct_keys(wp, pages)[0, 0, 0] == 3                  # pages {0, 1, 3}


def test_state_bytes_follow_the_scope_table_definition():
    w = workloads.config(2)
    base = bench.state_bytes_defined(w, 0, 0)
    assert base == 16 * w.top_k + 4 * w.hot
    assert bench.state_bytes_defined(w, 10, 0) - base == 36 * 10        # per miss
    assert bench.state_bytes_defined(w, 0, 7) - base == 4 * 7           # per distinct key
