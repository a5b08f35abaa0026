"""Host logic of bench.py (no GPU): the one-GPU guard, the hash that ties the
committed traffic counters to the quantize kernel's code, and the traffic
lookup that falls back to null when the code changed."""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _tree_copy(tmp_path):
    csrc = tmp_path / "fp4_post_weight_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.QUANT_KERNEL_SOURCES:
        shutil.copy(os.path.join(ROOT, "fp4_post_weight_amd", "csrc", name), csrc / name)
    return csrc


def test_source_hash_sees_code_not_comments(tmp_path, monkeypatch):
    csrc = _tree_copy(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash()
    k = csrc / "focus_kernels.hip"
    text = k.read_text()
    k.write_text("// a new comment line\n" + text.replace("\n", "\n  \n", 3) + "\n/* and a block */\n")
    assert bench.kernel_source_hash() == h0           # comments and blank space do not count
    k.write_text(text.replace("kActWaves = 4", "kActWaves = 8", 1))
    assert "kActWaves = 4" in text
    assert bench.kernel_source_hash() != h0           # a change of code does


def test_traffic_only_for_the_measured_code(tmp_path, monkeypatch):
    _tree_copy(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    prof = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(prof))
    assert bench.measured_traffic() is None           # no summary
    prof.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "bytes_per_launch": 1234}))
    assert bench.measured_traffic() == 1234
    prof.write_text(json.dumps({"kernel_source_hash": "0" * 16, "bytes_per_launch": 1234}))
    assert bench.measured_traffic() is None           # taken on other code
    prof.write_text("not json")
    assert bench.measured_traffic() is None
