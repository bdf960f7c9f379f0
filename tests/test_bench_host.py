"""Host-side logic of bench.py (CPU only): the HBM traffic figure it takes from
a committed rocprofv3 summary, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench


def _tree(tmp_path, files: dict, recorded_sha: str | None, traffic: str = "1.25e+09"):
    """A fake repository root: library sources under sparse_moe_gemm_amd/csrc
    and one profile summary that records `recorded_sha`."""
    root = tmp_path / "root"
    csrc = root / "sparse_moe_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    (root / "profiles").mkdir()
    for name, text in files.items():
        (csrc / name).write_bytes(text)
    lines = ["# summary", "", "| kernel | calls |", "|---|---|", "| k | 1 |", "",
             "dominant_kernel: k", f"traffic_bytes_per_launch: {traffic}"]
    if recorded_sha is not None:
        lines.append(f"csrc_sha256: {recorded_sha}")
    (root / "profiles" / "gate_up_gemm_wl_rocprof.md").write_text("\n".join(lines) + "\n")
    return str(root)


FILES = {"gemm.hip": b"kernel source\n", "api.cpp": b"launch decisions\n"}


def _digest_of(tmp_path, files):
    root = tmp_path / "digest"
    csrc = root / "sparse_moe_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name, text in files.items():
        (csrc / name).write_bytes(text)
    old = bench.ROOT
    try:
        bench.ROOT = str(root)
        return bench.source_digest()
    finally:
        bench.ROOT = old


def test_traffic_read_when_the_sources_are_unchanged(tmp_path, monkeypatch):
    sha = _digest_of(tmp_path, FILES)
    monkeypatch.setattr(bench, "ROOT", _tree(tmp_path, FILES, sha))
    assert bench.profiled_traffic("wl", "gate_up_gemm") == 1.25e9


def test_traffic_dropped_when_any_source_changed(tmp_path, monkeypatch):
    sha = _digest_of(tmp_path, FILES)
    # the kernel file, a launch-decision file, or a new file: each drops it
    for changed in ({**FILES, "gemm.hip": b"kernel source\n// edit\n"},
                    {**FILES, "api.cpp": b"launch decisions, other tile order\n"},
                    {**FILES, "new.hpp": b"x"}):
        root = _tree(tmp_path / str(len(str(changed))), changed, sha)
        monkeypatch.setattr(bench, "ROOT", root)
        assert bench.profiled_traffic("wl", "gate_up_gemm") is None


def test_traffic_missing_summary_hash_or_value(tmp_path, monkeypatch):
    sha = _digest_of(tmp_path, FILES)
    monkeypatch.setattr(bench, "ROOT", _tree(tmp_path / "a", FILES, sha, traffic="n/a"))
    assert bench.profiled_traffic("wl", "gate_up_gemm") is None
    assert bench.profiled_traffic("other", "gate_up_gemm") is None
    monkeypatch.setattr(bench, "ROOT", _tree(tmp_path / "b", FILES, None))
    assert bench.profiled_traffic("wl", "gate_up_gemm") is None


def test_committed_summaries_are_complete():
    # every committed summary gives the command it came from, its traffic
    # figure and the hash of the library sources its counters were taken on
    prof = os.path.join(bench.ROOT, "profiles")
    for name in sorted(os.listdir(prof)):
        if not name.endswith("_rocprof.md"):
            continue
        text = open(os.path.join(prof, name)).read()
        assert "csrc_sha256:" in text and "rocprofv3" in text, name
        if name.startswith("gate_up_gemm_"):
            assert "traffic_bytes_per_launch:" in text, name


def test_layer_bytes_and_flops():
    import synth

    cfg = synth.CONFIGS["mixtral"]
    counts = np.array([1] * 8)
    # 3 matrices of 4096 x 14336 bf16 per expert, router 4096 x 8, bias, x and y
    want = 8 * 3 * 4096 * 14336 * 2 + 4096 * 8 * 2 + 8 * 4 + 2 * 4096 * 4096 * 2
    assert bench.layer_bytes(cfg, counts) == want
    counts[3] = 0  # an empty expert's weights are not read
    assert bench.layer_bytes(cfg, counts) == want - 3 * 4096 * 14336 * 2
    assert cfg.flops() == 2.0 * 4096 * 4096 * 8 + 6.0 * 4096 * 14336 * 4096 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
