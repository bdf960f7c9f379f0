"""Host-side logic of bench.py (CPU only): the HBM traffic figure it takes from
a committed rocprofv3 summary, and its refusal of more than one GPU."""
import hashlib
import os
import subprocess
import sys

import bench


def _summary(tmp_path, src_text: bytes, recorded_sha: str, traffic: str = "1.25e+09"):
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    (root / "src").mkdir()
    (root / "src" / "kernel.hip").write_bytes(src_text)
    (root / "profiles" / "gate_up_gemm_wl_rocprof.md").write_text(
        "# summary\n\n| kernel | calls |\n|---|---|\n| k | 1 |\n\n"
        "dominant_kernel: k\n"
        f"traffic_bytes_per_launch: {traffic}\n"
        f"source_sha256(src/kernel.hip): {recorded_sha}\n")
    return str(root)


def test_traffic_read_when_the_source_is_unchanged(tmp_path, monkeypatch):
    src = b"kernel source\n"
    monkeypatch.setattr(bench, "ROOT", _summary(tmp_path, src, hashlib.sha256(src).hexdigest()))
    assert bench.profiled_traffic("wl", "gate_up_gemm") == 1.25e9


def test_traffic_dropped_when_the_source_changed(tmp_path, monkeypatch):
    src = b"kernel source\n"
    monkeypatch.setattr(bench, "ROOT", _summary(tmp_path, src + b"// edit\n", hashlib.sha256(src).hexdigest()))
    assert bench.profiled_traffic("wl", "gate_up_gemm") is None


def test_traffic_missing_summary_or_value(tmp_path, monkeypatch):
    src = b"kernel source\n"
    root = _summary(tmp_path, src, hashlib.sha256(src).hexdigest(), traffic="n/a")
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.profiled_traffic("wl", "gate_up_gemm") is None
    assert bench.profiled_traffic("other", "gate_up_gemm") is None


def test_committed_summaries_are_complete():
    # every committed summary gives the command it came from, its traffic
    # figure and the hash of the source file its counters were taken on
    prof = os.path.join(bench.ROOT, "profiles")
    for name in sorted(os.listdir(prof)):
        if not (name.startswith("gate_up_gemm_") and name.endswith("_rocprof.md")):
            continue
        text = open(os.path.join(prof, name)).read()
        assert "source_sha256(" in text and "traffic_bytes_per_launch:" in text, name
        assert "rocprofv3" in text, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
