"""bench.py's output contract, checked end to end on the GPU: one JSON line
with the throughput, its roofline object, the oracle baseline and the
workload descriptor, for the tiny workload (a few seconds).  The bench runs
as a child process, as a user would start it."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tiny_workload_bench_line():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "1", "--steps", "5",
                        "--warmup", "2"], capture_output=True, text=True, cwd=ROOT, timeout=180)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, p.stdout
    d = json.loads(lines[0])
    assert d["metric"].startswith("split-KV attention fwd TFLOP/s")
    assert d["unit"] == "TFLOP/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["warmup_steps_run"] >= 2
    assert d["ms_per_step"] > 0 and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["config"]["workload"] == "tiny" and d["config"]["valid_flops"] == 311808

    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert 0 < r["achieved"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["algorithmic_bytes"] == 26560
    assert r["us_per_call"] > 0 and r["us_per_call_graph"] > 0 and r["us_per_call_prepared"] > 0
    assert len(r["kernel_source_sha256_16"]) == 16

    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    par = d["parity"]
    assert par["max_abs"] <= 1e-2 and par["mean_abs"] <= 1e-3 and par["lse_max_abs"] <= 1e-3

    desc = d["descriptor"]
    assert desc["input_seed_base"] == 1000 and desc["compute_units"] > 0
    assert desc["arch"].startswith("gfx950")
    assert desc["kernel_source_sha256_16"] == r["kernel_source_sha256_16"]
