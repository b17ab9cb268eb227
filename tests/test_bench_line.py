"""bench.py's output contract on the GPU: a short run prints exactly one JSON line on stdout with
the fields a reader of the benchmark takes (metric, value, unit, steps, ms_per_step, ...), a
roofline object whose figures agree with one another, the CPU oracle's baseline, and the sampled
rows of the timed call checked against the oracle."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_short_bench_run_prints_one_contract_line():
    print("[gpu case] bench.py --steps 5 --warmup 2 (no decode, extra or metric rows)", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "2", "--no-decode", "--no-extra", "--no-metric-rows",
                        "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [line for line in r.stdout.splitlines() if line.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 5, 2)
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["scaling"] == "weak" and d["data"] == "synthetic" and d["value"] > 0
    assert "workload" in d["config"] and (d["config"]["m"], d["config"]["hidden"]) == (4096, 7168)

    rf = d["roofline"]
    assert (rf["bound"], rf["unit"], rf["peak"]) == ("hbm", "GB/s", 8000.0)
    assert rf["achieved"] == d["value"] and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # achieved = algorithmic bytes per launch / average launch time, the time of one step
    rate = rf["algorithmic_bytes_per_launch"] / (rf["avg_launch_us"] * 1e-6) / 1e9
    assert abs(rate / rf["achieved"] - 1) < 1e-3
    assert abs(d["ms_per_step"] * 1e3 / rf["avg_launch_us"] - 1) < 1e-3
    assert rf["algorithmic_bytes_per_launch"] == 2 * 11 * 4096 * 7168 + 2 * 7168
    assert rf["traffic"] is None or abs(rf["traffic"] / rf["algorithmic_bytes_per_launch"] - 1) < 0.01

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["sample"]
    assert d["parity_sampled_rows_ok"] is True
