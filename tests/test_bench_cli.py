"""bench.py's command-line contract, checked without a GPU."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_contract_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--no-cpu-baseline",
                 "--back-to-back"):
        assert flag in r.stdout


def test_stored_traffic_records_are_well_formed():
    """profiles/hbm_traffic.json: one record per bench part, each naming the
    kernel sources whose hash it was measured with."""
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    for part in ("prefill", "decode"):
        r = rec[part]
        assert r["bytes"] > 0
        assert len(r["source_sha256_16"]) == 16
        for src in r["sources"]:
            assert os.path.exists(os.path.join(ROOT, "exact_io_aware_attn_amd", "csrc", src))
