"""Host-side logic of bench.py (no GPU): the single-GPU refusal, the
HBM-traffic record that is only reported for the kernel sources it was
measured on, and its derivation from rocprofv3 counter runs."""
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


def _counter_csv(path, rows):
    path.mkdir()
    lines = ["Kernel_Name,Counter_Name,Counter_Value"]
    lines += [f"{k},C,{v}" for k, v in rows]
    (path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_traffic_from_counter_runs(tmp_path):
    """The traffic file derived from a synthetic counter run: each counter is
    scaled so the largest copy reads 512 MiB, averaged over a kernel's
    dispatches, and durations are the last traced dispatches' mean."""
    fwd = "_ZN4attn15fwd_mfma_kernelIDF16bLi64ELb1ELi0EEEvPKT_"
    dq = "_ZN4attn13bwd_dq_kernelIDF16bLi64ELb1ELb0ELb1EEEvPKT_"
    kv = "_ZN4attn15bwd_dkdv_kernelIDF16bLi64ELb1ELb0ELb0EEEvPKT_"
    cp = bench.COPY_KERNEL
    # FETCH reads half of the copy's bytes (scale 2), WRITE all of them (scale 1);
    # a smaller copy in the same run must not be taken for the calibration.
    _counter_csv(tmp_path / "step_FETCH_SIZE",
                 [(cp, 1024.0), (cp, 262144.0), (fwd, 100.0), (fwd, 300.0), (dq, 50.0), (kv, 10.0)])
    _counter_csv(tmp_path / "step_WRITE_SIZE",
                 [(cp, 524288.0), (fwd, 40.0), (dq, 20.0), (kv, 30.0)])
    tr = tmp_path / "step_trace"
    tr.mkdir()
    spans = [(fwd, 0, 1000), (fwd, 5000, 7000), (dq, 1000, 4000), (kv, 4000, 4500)]
    (tr / "run_kernel_trace.csv").write_text(
        "Kernel_Name,Start_Timestamp,End_Timestamp\n"
        + "".join(f"{k},{b},{e}\n" for k, b, e in spans))
    out = tmp_path / "traffic.json"
    bench.traffic_from(str(tmp_path), str(out))
    rec = json.loads(out.read_text())
    assert rec["source_hash"] == bench.kernel_source_hash()
    k = rec["kernels"]
    assert k["fwd"]["kernel"] == "fwd_mfma_kernel<__bf16, 64, true, 0>"
    assert k["bwd_dq"]["kernel"] == "bwd_dq_kernel<__bf16, 64, true, false, true>"
    assert k["fwd"]["hbm_bytes_per_launch"] == (200.0 * 2 + 40.0) * 1024
    assert k["bwd_dq"]["hbm_bytes_per_launch"] == (50.0 * 2 + 20.0) * 1024
    assert k["bwd_dkdv"]["hbm_bytes_per_launch"] == (10.0 * 2 + 30.0) * 1024
    assert k["fwd"]["avg_us"] == 1.5 and k["bwd_dq"]["avg_us"] == 3.0
    assert set(k) == {"fwd", "bwd_dq", "bwd_dkdv"}  # only the runs that are there


def test_traffic_from_needs_the_calibration_copy(tmp_path):
    import pytest

    kernel = "_ZN4attn15fwd_mfma_kernelIDF16bLi64ELb1ELi0EEEvPKT_"
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        _counter_csv(tmp_path / f"step_{ctr}", [(kernel, 1.0)])
    tr = tmp_path / "step_trace"
    tr.mkdir()
    (tr / "run_kernel_trace.csv").write_text(
        "Kernel_Name,Start_Timestamp,End_Timestamp\n" + kernel + ",0,1000\n")
    with pytest.raises(SystemExit, match="calibration copy"):
        bench.traffic_from(str(tmp_path), str(tmp_path / "traffic.json"))


def test_kernel_label_of_plain_and_template_kernels():
    assert bench.kernel_label("_ZN4attn16split_combine_kernelIDF16_Li256EEEvPKf") == \
        "split_combine_kernel<_Float16, 256>"
    assert bench.kernel_label("attn::sparse_compact_kernel(unsigned char const*)") == \
        "sparse_compact_kernel"


def test_environment_starts_no_child_program(monkeypatch):
    """bench.py's environment record is read from files and in-process calls:
    under a profiler that preloads itself into every process, a child tool
    would initialise the GPU and then exec."""
    import subprocess

    def refuse(*a, **k):
        raise AssertionError("child process started")

    monkeypatch.setattr(subprocess, "run", refuse)
    monkeypatch.setattr(subprocess, "Popen", refuse)
    v = bench.hip_version_string()
    if os.path.exists("/opt/rocm/include/hip/hip_version.h"):
        assert v.startswith("HIP version: ") and v.count(".") >= 2
    mhz = bench.max_sclk_mhz(0)  # None without a GPU
    assert mhz is None or mhz > 0
