"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, every finding fatal) passes all of its pins, every planted
mutation built the same way is still caught, and its array entry points run
clean over the shapes the parity tests use (ragged tails, per-token rows,
MXFP4, FourOverSix, MixFP4 tiles, the linear layer).  CPU only: a child
process with the ASan runtime preloaded loads the sanitized library."""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import os, sys
sys.path[:0] = [os.path.join(ROOT, "tests"), ROOT]
import numpy as np
import oracle
from oracle import build as oracle_build
import oracle_pins as pins
import synth
import test_oracle_mutations as tm

o = oracle.Oracle(LIB)
for check in pins.ALL_CHECKS:
    check(o)
print("pins", len(pins.ALL_CHECKS), flush=True)

# every array entry point over ragged and tiled shapes
w, m, q = synth.make_single()
wb = synth.bits(w)
s2, _ = o.tensor_scale(wb)
c, s, d = o.quantize(wb, m.numpy(), q.numpy(), s2, True)
o.dequantize(c, s, s2)
o.fo6_quantize(wb, s2)
for shape in [(1, 16), (3, 48), (7, 1040), (33, 2064)]:
    x = synth.activations(shape, seed=shape[0], tensor_id=5)
    o.quantize_act_per_token(synth.bits(x), True)
    o.fo6_quantize_act_per_token(synth.bits(x), True)
xb = synth.bits(synth.activations((5, 96), seed=1, tensor_id=6))
cm, sm, _ = o.mx_quantize(xb, None, None, True)
o.mx_dequantize(cm, sm)
tm_ = np.zeros((16 // 8, 256 // 64), np.uint8)
tm_[0, 1] = 1
wm = synth.bits(synth.weights((16, 256), seed=3, tensor_id=4))
cx, sx, _ = o.mixfp4_quantize(wm, s2, tm_, 8)
o.mixfp4_dequantize(cx, sx, s2, tm_, 8)
xc, xs = synth.nvfp4_operand(3, 48, seed=1, tensor_id=1)
wc, wsc = synth.nvfp4_operand(5, 48, seed=1, tensor_id=2)
o.nvfp4_linear(xc.numpy(), xs.numpy(), np.ones(3, np.float32), wc.numpy(), wsc.numpy(), np.ones(1, np.float32))
print("arrays", flush=True)

# planted mistakes, each built with the sanitizers (in parallel), are still
# caught
from concurrent.futures import ThreadPoolExecutor

def build_mutant(k):
    name, old, new = tm.MUTATIONS[k]
    src = open(oracle_build.SRC).read()
    assert src.count(old) >= 1, name
    cpath = os.path.join(TMP, f"mut{k}.c")
    with open(cpath, "w") as f:
        f.write(src.replace(old, new))
    return oracle_build.build(cpath, os.path.join(TMP, f"libmut{k}.so"), sanitize=True)

with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
    libs = list(ex.map(build_mutant, range(len(tm.MUTATIONS))))
for k, (name, old, new) in enumerate(tm.MUTATIONS):
    mo = oracle.Oracle(libs[k])
    caught = False
    for check in pins.ALL_CHECKS:
        try:
            check(mo)
        except AssertionError:
            caught = True
            break
    assert caught, name
print("mutations", len(tm.MUTATIONS), flush=True)
'''


def test_oracle_under_sanitizers(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.fail("the gcc ASan runtime is not installed")
    lib = oracle_build.build(oracle_build.SRC, str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = libasan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\nTMP = {str(tmp_path)!r}\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "pins" in r.stdout and "arrays" in r.stdout and "mutations" in r.stdout, out[-2000:]
