"""Host-side checks of bench.py's contract (no GPU needed).

* more than one GPU is refused with a message and a non-zero exit;
* the HBM traffic figure comes from a committed counter summary only while
  the kernel source it was taken on is unchanged."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr + p.stdout
    assert '"metric"' not in p.stdout


def test_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": "0123456789abcdef", "hbm_bytes_per_launch": 12345}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / f"{bench.KERNEL_NAME}_demo_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "0123456789abcdef")
    assert bench.load_traffic("demo") == 12345
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "fedcba9876543210")
    assert bench.load_traffic("demo") is None
    assert bench.load_traffic("no_such_workload") is None


def test_committed_profiles_name_the_sources_they_cover():
    """Every committed traffic record carries a 16-hex-digit source hash and a
    positive byte count."""
    prof = os.path.join(ROOT, "profiles")
    recs = [f for f in os.listdir(prof) if f.endswith("_traffic.json")]
    assert recs
    for f in recs:
        r = json.load(open(os.path.join(prof, f)))
        h = r["kernel_source_sha256_16"]
        assert len(h) == 16 and int(h, 16) >= 0, f
        assert r["hbm_bytes_per_launch"] > 0, f


def test_git_head_follows_a_symbolic_ref(tmp_path, monkeypatch):
    """The descriptor's revision: HEAD's ref resolved to its commit id, or
    None where no repository metadata travels with the tree."""
    git = tmp_path / ".git"
    (git / "refs" / "heads").mkdir(parents=True)
    (git / "HEAD").write_text("ref: refs/heads/main\n")
    (git / "refs" / "heads" / "main").write_text("0123abcd" * 5 + "\n")
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(tmp_path / "bench.py"))
    assert bench._git_head() == "0123abcd" * 5
    (git / "HEAD").write_text("fedc" * 10 + "\n")          # detached
    assert bench._git_head() == "fedc" * 10
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(tmp_path / "sub" / "bench.py"))
    assert bench._git_head() is None


def test_reported_figures_keep_small_values():
    """Throughputs are reported to two decimals, but a launch-bound workload's
    TFLOP/s (well below 0.01) keeps four significant digits instead of
    rounding to zero."""
    assert bench.figure(1298.6612) == 1298.66
    assert bench.figure(0.52) == 0.52
    assert bench.figure(0.0078123) == 0.007812
    assert bench.figure(0.0) == 0.0
    assert bench.figure(1298.6612 / 2500, 4) == 0.5195
    assert bench.figure(0.0078123 / 2500, 4) == 3.125e-06
