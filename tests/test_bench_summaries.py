"""bench.py's host logic on the CPU: the profile summaries it writes from rocprofv3 databases
(SQLite files of the tables it reads, with known values) and the traffic figure the bench line
reports; --gpus above 1 is refused."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM = "void tbg::gemm_ring_kernel<256, 256, 2, 0, 0, 1, 0, 0>(tbg::GemmParams)"
GEMM5 = "void tbg::gemm_ring_kernel<256, 256, 2, 0, 1, 1, 0, 0>(tbg::GemmParams)"
COPY = "__amd_rocclr_copyBuffer"


def _counters_db(path, counter, values):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text, "
              "value real, duration int)")
    d = 0
    for name, vals in values.items():
        for v, dur in vals:
            d += 1
            c.execute("insert into counters_collection values (?, ?, ?, ?, ?)", (name, d, counter, v, dur))
    c.commit()
    c.close()


def _trace_db(path, avg_us):
    c = sqlite3.connect(path)
    c.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
              "percentage real)")
    c.execute("insert into top_kernels values (?, ?, ?, ?, ?)", (GEMM, 10, 10 * avg_us, avg_us, 100.0))
    c.commit()
    c.close()


def test_traffic_from_counter_databases(tmp_path):
    # the calibration copy moves 512 MiB each way; FETCH_SIZE reads half of it (scale 2), WRITE_SIZE all
    copy_kib = (512 << 20) / 1024
    fetch = {COPY: [(copy_kib / 2, 1)] * 5, GEMM: [(1000000.0, 700000)] * 4 + [(9e9, 700000)],
             GEMM5: [(2000000.0, 1200000)] * 5}
    write = {COPY: [(copy_kib, 1)] * 5, GEMM: [(131072.0, 700000)] * 5, GEMM5: [(458752.0, 1200000)] * 5}
    for sub in ("trace", "fetch", "write"):
        os.makedirs(tmp_path / sub)
    _trace_db(str(tmp_path / "trace" / "run_results.db"), 700.0)
    _counters_db(str(tmp_path / "fetch" / "run_results.db"), "FETCH_SIZE", fetch)
    _counters_db(str(tmp_path / "write" / "run_results.db"), "WRITE_SIZE", write)
    out = tmp_path / "profiles"
    os.makedirs(out)
    cmds = {k: k for k in ("trace", "fetch", "write", "sq", "copytrace")}
    t = bench.summarize_profiles(str(tmp_path / "trace" / "run_results.db"), str(tmp_path / "fetch" / "run_results.db"),
                                 str(tmp_path / "write" / "run_results.db"), str(out), cmds)
    assert abs(t["fetch_scale"] - 2.0) < 1e-12 and abs(t["write_scale"] - 1.0) < 1e-12
    # medians per dispatch (the outlier dispatch does not move them), in bytes
    assert t["fetch_bytes"] == round(1000000.0 * 1024 * 2)
    assert t["write_bytes"] == round(131072.0 * 1024)
    assert t["hbm_bytes_per_launch"] == t["fetch_bytes"] + t["write_bytes"]
    assert t["algorithmic_bytes"] == 3 * 8192 * 8192 * 2
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    text = (out / "gemm_8192_hbm_counters.md").read_text()
    gbs = t["hbm_bytes_per_launch"] / 700e-6 / 1e9
    assert f"{gbs:.0f} GB/s" in text
    assert "700.000" in (out / "gemm_8192_kernel_trace.md").read_text()
    saved = json.loads((out / "gemm_8192_traffic.json").read_text())
    assert saved["hbm_bytes_per_launch"] == t["hbm_bytes_per_launch"]
    # the 16384x14336x4096 kernel gets its own figures
    assert saved["c5"]["fetch_bytes"] == round(2000000.0 * 1024 * 2)
    assert saved["c5"]["write_bytes"] == round(458752.0 * 1024)
    assert saved["c5"]["algorithmic_bytes"] == (16384 * 4096 + 4096 * 14336 + 16384 * 14336) * 2
    assert "16384×14336×4096 | FETCH_SIZE" in text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("cold", [0, 20])
def test_trace_summary_sets_timed_dispatches_beside_the_bench_line(tmp_path, cold):
    """The traced bench run's timed steps are the `steps` dispatches of the 8192^3 kernel before
    its `cold_calls` cold-cache calls (the last ones when there are none): the summary gives their
    average next to the bench line's own HIP-event figure."""
    for sub in ("trace", "fetch", "write"):
        os.makedirs(tmp_path / sub)
    db = str(tmp_path / "trace" / "run_results.db")
    _trace_db(db, 700.0)
    c = sqlite3.connect(db)
    c.execute("create table kernels (name text, start int, duration int)")
    # ns: settle / warm-up dispatches, then 20 timed ones, then (with cold calls) the spread
    # region's 5 + 20 and the cold-cache calls
    spread = 25 if cold else 0
    durs = [800000] * 30 + [700000] * 20 + [750000] * spread + [900000] * cold
    for i, d in enumerate(durs):
        c.execute("insert into kernels values (?, ?, ?)", (GEMM, i, d))
    c.execute("insert into kernels values (?, ?, ?)", ("other", 99, 5))
    c.commit()
    c.close()
    copy_kib = (512 << 20) / 1024
    _counters_db(str(tmp_path / "fetch" / "run_results.db"), "FETCH_SIZE",
                 {COPY: [(copy_kib / 2, 1)] * 5, GEMM: [(1000000.0, 700000)] * 5})
    _counters_db(str(tmp_path / "write" / "run_results.db"), "WRITE_SIZE",
                 {COPY: [(copy_kib, 1)] * 5, GEMM: [(131072.0, 700000)] * 5})
    out = tmp_path / "profiles"
    os.makedirs(out)
    line = {"steps": 20, "value": 1500.0, "roofline": {"kernel_ms": 0.7, "achieved": 1570.7, "frac": 0.6241,
                                                        "flops_per_launch": 2 * 8192 ** 3}}
    if cold:
        line["per_config"] = {"c4": {"cold_ms": 0.9, "cold_calls": cold}}
        line["roofline"]["spread_calls"] = spread
    cmds = {k: k for k in ("trace", "fetch", "write", "sq", "copytrace")}
    cmds["bench_line"] = line
    t = bench.summarize_profiles(db, str(tmp_path / "fetch" / "run_results.db"),
                                 str(tmp_path / "write" / "run_results.db"), str(out), cmds)
    text = (out / "gemm_8192_kernel_trace.md").read_text()
    assert "| timed 20 | 700.00 | 700.00 |" in text
    assert f"| all {50 + spread + cold} |" in text and "kernel_ms 0.7" in text
    assert abs(t["gemm_trace_avg_us"] - 700.0) < 1e-9


def _hw_id(se, sh, cu):
    return (se << 13) | (sh << 12) | (cu << 8)


def test_timeline_stats_and_profile(tmp_path):
    """timeline_stats on hand-made timelines: three workgroups, two on one CU (XCD 1, SE 2, SA 1,
    CU 5) and one on another; times in 100 MHz ticks, 2 GHz shader clock."""
    # start, first tile, loop done, stores done, shader ticks, HW_ID, XCC_ID, 0
    tl = [[1000, 1100, 1500, 1520, 2 * 520 * 10, _hw_id(2, 1, 5), 1, 0],
          [1010, 1130, 1530, 1560, 2 * 550 * 10, _hw_id(2, 1, 5), 1, 0],
          [1005, 1105, 1405, 1425, 2 * 420 * 10, _hw_id(0, 0, 3), 4, 0]]
    s = bench.timeline_stats(tl, ktiles=4, tile_bytes=1000)
    assert s["workgroups"] == 3 and s["cus"] == 2 and s["max_wg_per_cu"] == 2
    assert s["start_us"] == {"median": 0.05, "max": 0.1}
    assert s["first_tile_us"] == 1.0  # median of 1.0, 1.2, 1.0 µs
    assert s["k_loop_us"] == 4.0 and s["per_k_tile_us"] == 1.0
    assert s["epilogue_us"] == 0.2
    assert s["end_us"] == {"min": 4.25, "median": 5.2, "max": 5.6}
    assert s["clock_ghz"] == 2.0
    # the two workgroups on CU 5 copied 2 * 4 * 1000 bytes between 11.0 and 15.3 µs at 2 GHz
    assert s["copy_bytes_per_clk_per_cu"] == round(8000 / (4.3 * 1e3 * 2.0), 1)
    line = {"timeline": "c2", "M": 1024, "N": 1024, "K": 1024, "out": "bf16", "config": "ring 64x64/3",
            "launch_us": 6.1}
    line.update(s)
    path = tmp_path / "timeline.jsonl"
    path.write_text(json.dumps(line) + "\n")
    bench.write_timeline_profile(str(path), str(tmp_path))
    md = (tmp_path / "gemm_ring_timeline.md").read_text()
    assert "## c2: 1024×1024×1024 (B K×N, bf16 out)" in md
    assert "| ring 64x64/3 | 3 | 2 | 2 | 6.1 | 5.6 | 1.0 | 4.0 | 1.0 | 0.2 | 2.0 | 0.9 |" in md
    # per XCD: XCD 1 holds the two workgroups on CU 5, XCD 4 the third
    assert s["xcds"] == [{"xcd": 1, "workgroups": 2, "clock_ghz": 2.0, "k_loop_us": 4.0},
                         {"xcd": 4, "workgroups": 1, "clock_ghz": 2.0, "k_loop_us": 3.0}]
    assert "| 1 | 2 | 2.0 | 4.0 |" in md and "| 4 | 1 | 2.0 | 3.0 |" in md


def test_correlation():
    assert bench._correlation([1, 2, 3], [2, 4, 6]) == 1.0
    assert bench._correlation([1, 2, 3], [3, 2, 1]) == -1.0
    assert bench._correlation([1, 2], [1, 2]) is None
