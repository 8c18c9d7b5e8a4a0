"""GPU check of bench.py's output contract on a short run of the one-layer
workload: one JSON line with the required fields, a roofline entry whose
achieved rate follows from its own bytes and time, and the CPU baseline."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "gqa1",
                        "--steps", "5", "--warmup", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert abs(rf["achieved"] - rf["bytes_per_call"] / (rf["us_per_call"] * 1e3)) <= 0.01 * rf["achieved"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert d["launch_floor"]["kernels"] == 2


def test_default_line_is_the_long_context_workload():
    """The default line: dense decode attention with the append at B=8,
    L=131072 as value and roofline, the Quest step beside it, and the oracle
    baseline with its parity check on sampled units."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-legs"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["config"]["workload"].startswith("long_context") and d["config"]["seq_len"] == 131072
    rf = d["roofline"]
    assert abs(rf["achieved"] - rf["bytes_per_call"] / (rf["us_per_call"] * 1e3)) <= 0.01 * rf["achieved"]
    assert rf["bytes_per_call"] >= 4294967296
    q = d["quest"]
    assert q["us_per_step"] > 0 and q["byte_model_ratio"] == 0.09375
    assert set(q["stages"]) == {"append_score", "select_sparse_attention"}
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["host_cores"] >= cb["cores"]
    p = cb["parity"]
    assert p["dense_max_abs_err"] <= 2e-3 and p["quest_max_abs_err"] <= 2e-3
    assert p["idx_rule_violations"] == 0 and p["idx_units"] == 16
