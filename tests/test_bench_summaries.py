"""bench.py's host logic on the CPU: the profile summaries it writes from rocprofv3 databases
(SQLite files of the tables it reads, with known values) and the traffic figure the bench line
reports; --gpus above 1 is refused."""
import json
import os
import sqlite3
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM = "void tbg::gemm_ring_kernel<256, 256, 2, 0, 0, 1, 0>(tbg::GemmParams)"
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
    fetch = {COPY: [(copy_kib / 2, 1)] * 5, GEMM: [(1000000.0, 700000)] * 4 + [(9e9, 700000)]}
    write = {COPY: [(copy_kib, 1)] * 5, GEMM: [(131072.0, 700000)] * 5}
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


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
