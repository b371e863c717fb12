"""Build libmlaprolog.so (gfx950) in-tree with hipcc.

Usage: python -m mla_attention_kv_amd.build_lib   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmlaprolog.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "graphs.cpp", "prolog_tiled.hip", "prolog_decode.hip", "kv_cache.hip",
           "norm_rope.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # hipcc -O3 forms packed-fp32 instructions from ordinary float code; keep
    # them off (a compile flag for the device pass; the host pass ignores it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE division / sqrt: the W8A8 codes depend on 127/amax being exact
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return out


def build(verbose: bool = False) -> str:
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv or True))
