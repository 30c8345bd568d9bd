"""Build the HIP library ``libtree_attn.so`` in-tree for gfx950.

Runs hipcc on the device code and the host dispatch; the result sits next to
this file, where the Python binding loads it.  Packed-fp32 instruction
selection is turned off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtree_attn.so")
SOURCES = [os.path.join(CSRC, f) for f in ("attn.hip", "plan.hip", "tree.hip", "commit.hip", "noalloc.hip", "tree_attn.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_cmd(out: str):
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = build_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the gfx feature name; that warning is harmless
    lines = [ln for ln in res.stdout.splitlines()
             if "packed-fp32-ops" not in ln and "--hip-link" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
