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


def _oracle_set(orc):
    """A two-layer set of small linears whose 'GPU outputs' are the oracle's
    own (CPU tensors): the benchmark's parity pass must find no mismatch."""
    import types

    import numpy as np
    import torch

    import fp4_post_weight_amd as f
    import synth
    ws = synth.WeightSet("two small layers", 256, 64, 512, 2, 0.02, "lognormal")
    R = types.SimpleNamespace(ws=ws, lins=ws.linears(), W=[], M=[], Q=[], OUT=[], WDQ=[], DEQ=[])
    s2s, ams = [], []
    for lin in R.lins:
        w, m, q = synth.make_linear(ws, lin)
        wb = synth.bits(w)
        s2, am = orc.tensor_scale(wb)
        c, sc, d = orc.quantize(wb, m.numpy(), q.numpy(), s2, True)
        dt = torch.from_numpy(d.view(np.int16)).view(torch.bfloat16)
        R.W.append(w)
        R.M.append(m)
        R.Q.append(q)
        R.OUT.append(f.Quantized(torch.from_numpy(c), torch.from_numpy(sc), dt, None))
        R.WDQ.append(dt)
        R.DEQ.append(dt.clone())
        s2s.append(s2)
        ams.append(am)
    R.S2 = torch.tensor(s2s).view(-1, 1)
    R.AMAX = torch.tensor(ams).view(-1, 1)
    x = synth.make_activations((40, 4096))
    c, sc, s2t, _ = orc.quantize_act_per_token(synth.bits(x))
    act = f.Quantized(torch.from_numpy(c), torch.from_numpy(sc), None, torch.from_numpy(s2t))
    return R, x, act


def test_set_parity_pass_counts_and_finds_planted_mismatches(orc):
    import types
    args = types.SimpleNamespace(cpu_weights=0)
    R, x, act = _oracle_set(orc)
    par, cpu = bench.check_set(R, x, act, args, False, label="small")
    assert par["ok"] and par["tensors"] == 14 and par["weights_checked"] == sum(l.numel for l in R.lins)
    assert par["scale_mismatches"] == par["code_mismatches"] == par["wdeq_mismatches"] == 0
    assert par["act_tokens"] == 40 and cpu["kind"] == "oracle" and cpu["value"] > 0
    # planted on the 'GPU' side: a scale byte, a code nibble, a dequantized
    # value, an activation scale byte and one tensor's s2
    R.OUT[3].scales[5, 2] ^= 1
    R.OUT[5].codes[7, 9] ^= 0x10
    R.DEQ[6][1, 1] = 1.0
    act.scales[3, 3] ^= 2
    R.S2[2, 0] *= 2
    par, _ = bench.check_set(R, x, act, args, False, label="small")
    assert not par["ok"]
    assert par["scale_mismatches"] == 1 and par["dequantize_mismatches"] == 1
    assert par["s2_mismatches"] == 1 and par["act_scale_mismatches"] == 1
    assert any("not explained by sigmoid rounding" in e for e in par["failures"])
