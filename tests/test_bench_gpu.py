"""The benchmark's JSON line on the GPU: a short default run prints one line with the fields the
measurement contract asks for, at the headline workload, with consistent figures."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    print("[bench] --steps 3 --warmup 1 --no-cpu-baseline --no-detail-tables", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--no-detail-tables"], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, p.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["vs_baseline"] is None
    assert d["config"]["workload"] == "s64-p4096-q33"
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 2500.0 and 0 < r["frac"] < 1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # the whole step (verify + accept + compaction) is longer than the verify call alone
    assert 0 < d["value"] <= r["achieved"]
    assert d["detail"]["verify_us_per_call"] <= d["ms_per_step"] * 1e3
    if r["traffic"] is not None:  # HBM bytes counted per launch are at least the algorithmic bytes
        assert r["traffic"] >= d["detail"]["algorithmic_bytes"]
    assert "cpu_baseline" not in d
