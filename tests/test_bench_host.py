"""Host logic of bench.py on the CPU: the one-GPU guard, the FLOP count of a tree, the traffic
reader's staleness check, and the profile summarisers on small databases shaped like rocprofv3's
(``kernels`` and ``pmc_events`` views)."""
import os
import sqlite3
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stdout


def test_visible_pairs_counts_prefix_plus_ancestors():
    parents = np.array([[-1, 0, 1, 1], [-1, 0, 0, 0]])
    # depths [0,1,2,2] and [0,1,1,1]: each node sees P + depth + 1 keys
    assert bench.visible_pairs(parents, 10) == (11 + 12 + 13 + 13) + (11 + 12 + 12 + 12)
    assert bench.visible_pairs(np.array([[-1]]), 0) == 1


def test_traffic_is_ignored_for_another_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "pmc.txt"
    f.write_text("kernel_source_sha256: 0123456789abcdef\nhbm_bytes_per_launch: 1000\n")
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(f))
    assert bench.read_traffic() is None
    f.write_text(f"kernel_source_sha256: {bench.kernel_sha()}\nhbm_bytes_per_launch: 1234.5\n")
    assert bench.read_traffic() == 1234.5


def make_db(path, dispatches, counters):
    """dispatches: [(dispatch_id, kernel name, start, duration)]; counters: [(dispatch_id,
    counter, [per-instance values])]."""
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, dispatch_id int, start int, duration int)")
    con.execute("create table pmc_events (name text, dispatch_id int, counter_name text, counter_value real)")
    names = {}
    for d, name, start, dur in dispatches:
        names[d] = name
        con.execute("insert into kernels values (?,?,?,?)", (name, d, start, dur))
    for d, cn, vals in counters:
        for v in vals:
            con.execute("insert into pmc_events values (?,?,?,?)", (names[d], d, cn, v))
    con.commit()
    con.close()


def test_counter_summary_sums_instances_per_dispatch(tmp_path):
    db = str(tmp_path / "c.db")
    make_db(db, [(1, "verify_attn_kernel(x)", 0, 10), (2, "verify_attn_kernel(x)", 20, 10), (3, "other", 40, 5)],
            [(1, "MfmaFlopsBF16", [1.0, 2.0, 3.0]), (2, "MfmaFlopsBF16", [2.0, 2.0, 2.0]),
             (1, "MfmaUtil", [50.0]), (2, "MfmaUtil", [70.0]), (3, "MfmaUtil", [1.0]),
             (1, "SQ_LDS_BANK_CONFLICT", [1.0, 1.0]), (2, "SQ_LDS_BANK_CONFLICT", [1.0, 1.0]),
             (1, "SQ_LDS_IDX_ACTIVE", [100.0]), (2, "SQ_LDS_IDX_ACTIVE", [100.0])])
    text = bench.summarize_counters(db, "cmd")
    assert "mfma_bf16_flop_per_launch: 6" in text      # (1+2+3 + 2+2+2) / 2 dispatches
    assert "mfma_busy_pct: 60.00" in text                # the other kernel is left out
    assert "lds_bank_conflict_cycles_per_active_cycle: 0.0200" in text


def test_trace_summary_leaves_out_warmup(tmp_path):
    db = str(tmp_path / "t.db")
    make_db(db, [(1, "k", 0, 5000), (2, "k", 10, 1000), (3, "k", 20, 3000)], [])
    text = bench.summarize_trace(db, "cmd", skip=1)
    line = [l for l in text.splitlines() if l.startswith("k ")][0].split()
    calls, avg, avg_timed = int(line[1]), float(line[2]), float(line[3])
    assert calls == 3 and avg == pytest.approx(3.0) and avg_timed == pytest.approx(2.0)


def test_clock_summary_scales_the_peak_with_the_clock():
    # 1.2e12 FLOP in 1000 us = 1200 TFLOP/s; at a median of 1920 MHz the peak is 2500 * 0.8 = 2000
    samples = [(0.1, 95.0, 244.0), (1.5, 1900.0, 1390.0), (1.7, 1920.0, 1395.0), (1.9, 1940.0, 1400.0),
               (2.1, 0.0, 0.0)]
    r = bench.clock_summary(samples, 1000.0, 1.2e12)
    assert r["samples"] == 3 and r["gfx_clock_mhz_median"] == 1920.0 and r["gfx_clock_mhz_range"] == [1900.0, 1940.0]
    assert r["socket_power_w_median"] == 1395.0
    assert r["tflops"] == 1200.0 and r["peak_at_clock_tflops"] == 2000.0 and r["frac_at_clock"] == 0.6
    assert bench.clock_summary([], 1000.0, 1.2e12) == {"error": "no clock samples"}
    # a load shorter than the reading period still reports what it saw
    assert bench.clock_summary([(0.1, 2100.0, 800.0)], 1000.0, 1.2e12)["samples"] == 1
