"""Builds the gfx950 shared library ``libkda.so`` in-tree with hipcc.

Usage: ``python -m kimi_delta_attention_chunk_amd.build`` (or ``build_library()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = [os.path.join(CSRC, "kda_kernels.hip"), os.path.join(CSRC, "kda_plan.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build_library(out_path: str = LIB, verbose: bool = False, extra: list | None = None) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result",
           # keep the compiler from forming packed fp32 ops on its own
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", out_path + ".tmp"]
    if extra:
        cmd[1:1] = list(extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(out_path + ".tmp", out_path)
    return out_path


if __name__ == "__main__":
    print(build_library(verbose=True))
