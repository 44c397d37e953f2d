"""bench.py on the GPU: one short run of a small workload prints one JSON line
with the contract's keys, the live engine clock and the roofline at it."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_json_line_with_measured_clock():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "gpt2-medium-causal",
                        "--steps", "3", "--warmup", "2", "--no-cpu-baseline", "--back-to-back", "20"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["value"] > 0
    clk = out["clock"]["measured"]
    assert clk is not None
    assert 100 < clk["mhz_min"] <= clk["mhz_mean"] <= clk["mhz_max"] < 3000
    assert len(clk["mhz_per_xcd"]) == 8
    roof = out["roofline"]
    assert roof["bound"] == "mfma" and 0 < roof["frac"] < 1
    # the peak scaled to the measured clock is the 2.4 GHz peak times its ratio
    assert abs(roof["peak_at_measured_clock"] - roof["peak"] * clk["mhz_mean"] / 2400) < 1e-6 * roof["peak"]
