"""Build the oracle's shared library with gcc (test infrastructure only).

The flags keep every binary32 operation a single IEEE operation: no
contraction into FMA, no fast-math.  ``build(src, out)`` can build another
copy of the source (the tests build mutated copies to show that the pins
catch planted mistakes).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "focus_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-finite-math-only", "-frounding-math", "-Wall", "-Wextra"]

# A host-only sanitized build (AddressSanitizer + UndefinedBehaviorSanitizer,
# every finding fatal) for the CPU tests; loading it needs the ASan runtime
# preloaded (LD_PRELOAD of `gcc -print-file-name=libasan.so`).
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(src: str = SRC, out: str = LIB, verbose: bool = False, sanitize: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
