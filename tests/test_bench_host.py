"""Host-side logic of bench.py (no GPU): the single-GPU refusal and the
HBM-traffic record that is only reported for the kernel sources it was
measured on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "only --gpus 1" in res.stderr
    assert json.loads(res.stdout.strip().splitlines()[-1])["error"]


def test_traffic_needs_matching_kernel_sources(tmp_path, monkeypatch):
    rec = {"source_hash": bench.kernel_source_hash(),
           "kernels": {"bwd_dkdv": {"hbm_bytes_per_launch": 123.0}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic("bwd_dkdv") == 123.0
    assert bench.load_traffic("no_such_kernel") is None
    rec["source_hash"] = "0" * 16  # counters taken on other sources
    f.write_text(json.dumps(rec))
    assert bench.load_traffic("bwd_dkdv") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic("bwd_dkdv") is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "k.hip").write_text("int f() { return 1; }  // one\n")
    monkeypatch.setattr(bench, "CSRC", str(src))
    h1 = bench.kernel_source_hash()
    (src / "k.hip").write_text("/* block */\nint f() { return 1; }  // another comment\n\n")
    assert bench.kernel_source_hash() == h1
    (src / "k.hip").write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h1

