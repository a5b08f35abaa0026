"""Build libfocus_nvfp4.so in-tree with hipcc for gfx950.

Flags that the arithmetic contract depends on:
  -ffp-contract=off                       no a*b+c fused into one rounding
  -fno-gpu-flush-denormals-to-zero        binary32 subnormals kept
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE binary32 division
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                          no packed FP32 instructions
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfocus_nvfp4.so")
ARCH = os.environ.get("FOCUS_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=()) -> str:
    out = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    errs = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError("hipcc failed")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(out, LIB)
    return LIB


SELFTEST_SRC = os.path.join(ROOT, "tests", "hip", "focus_selftest.hip")
SELFTEST_LIB = os.path.join(ROOT, "tests", "hip", "libfocus_selftest.so")


def build_selftest(verbose: bool = False) -> str:
    """The test-only helper library (tests/hip), built from the same numerics
    header as the product kernels."""
    out = SELFTEST_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, f"-I{CSRC}", SELFTEST_SRC, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError("hipcc failed (selftest)")
    os.replace(out, SELFTEST_LIB)
    return SELFTEST_LIB


STREAM_SRC = os.path.join(ROOT, "tests", "hip", "focus_stream.hip")
STREAM_LIB = os.path.join(ROOT, "tests", "hip", "libfocus_stream.so")


def build_stream(verbose: bool = False) -> str:
    """The streaming-ceiling helper (tests/hip) that bench.py times beside
    the quantizer."""
    out = STREAM_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, STREAM_SRC, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError("hipcc failed (stream helper)")
    os.replace(out, STREAM_LIB)
    return STREAM_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_selftest(verbose=True)
    build_stream(verbose=True)
