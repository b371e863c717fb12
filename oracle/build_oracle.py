"""Build the CPU oracle (``oracle/liboracle.so``) with gcc.

Test infrastructure: the oracle is the checker, not the product.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = [
        "gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
        "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", src, "-o", tmp, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
