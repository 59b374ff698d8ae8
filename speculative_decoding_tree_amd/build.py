"""Compile libgdn_tree.so for gfx950 in-tree with hipcc.

    python -m speculative_decoding_tree_amd.build

hipcc cross-compiles the device code without a GPU, so this runs on any host
with ROCm installed.  The library lands next to this file, where the binding
loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libgdn_tree.so")
SOURCES = ["api.hip", "verify.hip", "commit.hip", "storeall.hip", "budget.hip", "attention.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdn_tree)")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-I", INCLUDE,
        # never let the compiler form packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {LIB}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
