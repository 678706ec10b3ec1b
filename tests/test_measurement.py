"""Host side of the measurement: the rocprofv3 summary tool and bench.py's contract checks
that need no GPU."""

import json
import os
import sqlite3
import subprocess
import sys

import pytest

from rejection_sampling_verify_specdec_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id int, "
                "counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_traffic_scales_by_the_largest_copy(tmp_path):
    nb = 512 << 20
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    # the device reports FETCH_SIZE as half the bytes, WRITE_SIZE exactly (KiB); a small
    # unrelated copy must not enter the calibration
    _counter_db(fetch, [("__amd_rocclr_copyBuffer", 1, "FETCH_SIZE", 4.0),
                        ("__amd_rocclr_copyBuffer", 2, "FETCH_SIZE", nb / 2 / 1024),
                        ("k_cycle_stats<true>", 3, "FETCH_SIZE", 1000.0),
                        ("k_cycle_stats<true>", 4, "FETCH_SIZE", 1002.0)])
    _counter_db(write, [("__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", 8.0),
                        ("__amd_rocclr_copyBuffer", 2, "WRITE_SIZE", nb / 1024),
                        ("k_cycle_stats<true>", 3, "WRITE_SIZE", 10.0),
                        ("k_cycle_stats<true>", 4, "WRITE_SIZE", 10.0)])
    text, info = profsum.traffic(fetch, write, "k_cycle_stats", "copyBuffer", nb, 2_000_000)
    assert info["fetch_scale"] == pytest.approx(2.0)
    assert info["write_scale"] == pytest.approx(1.0)
    assert info["fetch_bytes_per_launch"] == pytest.approx(1001.0 * 1024 * 2)
    assert info["write_bytes_per_launch"] == pytest.approx(10.0 * 1024)
    assert "ratio" in text


def test_traffic_json_is_stamped_with_the_kernel_sources(tmp_path):
    nb = 1 << 20
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    _counter_db(fetch, [("copyBuffer", 1, "FETCH_SIZE", nb / 2 / 1024), ("kx", 2, "FETCH_SIZE", 1.0)])
    _counter_db(write, [("copyBuffer", 1, "WRITE_SIZE", nb / 1024), ("kx", 2, "WRITE_SIZE", 1.0)])
    out = tmp_path / "kx_wl_traffic.json"
    profsum.main(["traffic", fetch, write, "--kernel", "kx", "--calib-kernel", "copyBuffer",
                  "--calib-bytes", str(nb), "--json", str(out), "--workload", "wl",
                  "--cmd", "rocprofv3 ..."])
    d = json.loads(out.read_text())
    assert d["source_sha256_16"] == profsum.source_hash()
    assert d["bytes_per_launch"] == pytest.approx(2048 + 1024)
    assert d["workload"] == "wl" and d["command"] == "rocprofv3 ..."


def test_source_hash_tracks_every_kernel_source():
    h = profsum.source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_sequence_lists_the_last_matching_dispatches_in_order(tmp_path):
    db = str(tmp_path / "k.db")
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start int, end int)")
    con.executemany("insert into kernels values (?, ?, ?)", [
        ("void sd::k_cycle_pass<true, true>(sd::KvArgs)", 1000, 26000),
        ("at::native::fill", 26000, 30000),
        ("void sd::k_cycle_pass<true, true>(sd::KvArgs)", 30500, 40000),
        ("void sd::k_cycle_decide<true>(sd::SampleArgs)", 40000, 120000),
    ])
    con.commit()
    con.close()
    lines = profsum.sequence(db, "k_cycle_", 2).splitlines()
    assert lines[1].split()[-2:] == ["9.50", "0.00"]          # the second pass, no gap shown
    assert "k_cycle_decide" in lines[2] and lines[2].split()[-2:] == ["80.00", "0.00"]
    assert lines[-1].split()[-1] == "89.50"                   # span of the two
    lines = profsum.sequence(db, "k_cycle_", 3).splitlines()
    assert lines[2].split()[-1] == "4.50"                     # gap past the fill


def test_counters_average_per_dispatch(tmp_path):
    db = str(tmp_path / "c.db")
    _counter_db(db, [("k_cycle_topk_merge<true>", 1, "SQ_WAVES", 10.0),
                     ("k_cycle_topk_merge<true>", 1, "SQ_WAVES", 6.0),      # summed per dispatch
                     ("k_cycle_topk_merge<true>", 2, "SQ_WAVES", 20.0),
                     ("k_cycle_topk_merge<true>", 1, "SQ_BUSY_CYCLES", 100.0),
                     ("k_cycle_topk_merge<true>", 2, "SQ_BUSY_CYCLES", 300.0),
                     ("other", 3, "SQ_WAVES", 999.0)])
    lines = profsum.counters(db, ["k_cycle_topk_merge"]).splitlines()
    assert lines[0].startswith("k_cycle_topk_merge: 2 dispatches")
    vals = {ln.split()[0]: float(ln.split()[1]) for ln in lines[1:]}
    assert vals == {"SQ_BUSY_CYCLES": 200.0, "SQ_WAVES": 18.0}
