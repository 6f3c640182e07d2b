"""CPU checks of bench.py's measurement helpers: the kernel-name shortening,
the rocprofv3 summaries (a kernel-trace database and per-dispatch counter
CSVs, both synthetic here) and the traffic record lookup."""
import csv
import json
import os
import sqlite3
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_short_kernel_names():
    assert bench._short_kernel(
        "void vx::(anonymous namespace)::decode_step_kernel<unsigned short, 128, 4, 1, 2, 4, "
        "false>(vx::StepArgs)") == "decode_step_kernel<unsigned short, 128, 4, 1, 2, 4, false>"
    assert bench._short_kernel("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    # a parenthesis inside the template arguments does not end the name
    assert bench._short_kernel("void f<g(int)>(int)") == "f<g(int)>"
    long = "void " + "k" * 200 + "(int)"
    assert len(bench._short_kernel(long)) == 90


def _write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                           "Workgroup_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_counters(tmp_path):
    d = tmp_path / "pass" / "host"
    d.mkdir(parents=True)
    k1 = "void vx::(anonymous namespace)::score_kernel<unsigned short, 128>(vx::ScoreArgs)"
    k2 = "__amd_rocclr_copyBuffer"
    rows = []
    # dispatch 1 and 3 of k1 (two counter instances each, summed), 2 of k2
    for did, kern, vals in ((1, k1, (10.0, 5.0)), (2, k2, (7.0,)), (3, k1, (20.0, 1.0))):
        for v in vals:
            rows.append({"Dispatch_Id": did, "Kernel_Name": kern, "Grid_Size": 1024,
                         "Workgroup_Size": 512, "Counter_Name": "FETCH_SIZE", "Counter_Value": v})
    _write_counters(d / "p_counter_collection.csv", rows)
    out = bench.summarize_counters(str(tmp_path), "score")
    assert list(out) == ["score_kernel<unsigned short, 128> grid=1024 block=512"]
    s = out["score_kernel<unsigned short, 128> grid=1024 block=512"]
    assert s["dispatches"] == 2 and s["values"] == [15.0, 21.0]
    assert s["min"] == 15.0 and s["max"] == 21.0 and s["median"] == 21.0
    both = bench.summarize_counters(str(tmp_path), ".")
    assert list(both)[0].startswith("score_kernel") and len(both) == 2   # first-dispatch order


def test_summarize_trace(tmp_path):
    db = tmp_path / "k_results.db"
    con = sqlite3.connect(db)
    con.execute("create table rocpd_info_kernel_symbol (id integer, display_name text)")
    con.execute("create table rocpd_kernel_dispatch (kernel_id integer, grid_size_x integer, "
                "grid_size_y integer, grid_size_z integer, workgroup_size_x integer, "
                "group_segment_size integer, start integer, end integer)")
    con.execute("insert into rocpd_info_kernel_symbol values (1, 'void vx::combine_kernel<float, 64>(vx::CombineArgs)')")
    con.execute("insert into rocpd_info_kernel_symbol values (2, 'void vx::(anonymous namespace)::topk_kernel(vx::TopkArgs)')")
    # two combine launches (2 us and 4 us), then one top-k launch (3 us)
    for kid, st, en in ((1, 0, 2000), (1, 10000, 14000), (2, 20000, 23000)):
        con.execute("insert into rocpd_kernel_dispatch values (?, 512, 1, 1, 256, 4112, ?, ?)",
                    (kid, st, en))
    con.commit()
    con.close()
    lines = bench.summarize_trace(str(db)).splitlines()
    assert lines[0].startswith("| kernel |") and len(lines) == 4
    assert lines[2] == "| `combine_kernel<float, 64>` | 2x1x1 | 256 | 4112 | 2 | 3.00 | 4.00 | 2.00 |"
    assert lines[3] == "| `topk_kernel` | 2x1x1 | 256 | 4112 | 1 | 3.00 | 3.00 | 3.00 |"


def test_traffic_record_keyed_to_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "_ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "block_sparse_paged_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "include").mkdir()
    (tmp_path / "block_sparse_paged_amd" / "csrc" / "a.hip").write_text("kernel v1")
    (tmp_path / "include" / "vx.h").write_text("header")
    assert bench.measured_traffic("w") is None                     # no record
    rec = {"source_sha256": bench._source_sha256(),
           "workloads": {"w": {"hbm_bytes_per_step": 1234}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w") == 1234
    assert bench.measured_traffic("other") is None
    (tmp_path / "block_sparse_paged_amd" / "csrc" / "a.hip").write_text("kernel v2")
    assert bench.measured_traffic("w") is None                     # sources changed
