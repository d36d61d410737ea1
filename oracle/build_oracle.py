"""Build the CPU oracle shared library with the host C compiler (test infrastructure).

    python oracle/build_oracle.py

Plain C, -O2, no fast-math and no FMA contraction, no BLAS, no intrinsics.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tlg_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler (gcc/cc) found")
    tmp = OUT + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", SRC, "-o", tmp, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
