"""Builds libkdraft.so (HIP, gfx950) in-tree with hipcc.

    python -m block_draft_model_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkdraft.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kd_kernels.hip", "kd_mm.hip", "kd_copy.hip", "kd_small.hip", "kd_api.hip")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("kd_device.h", "kd_runtime.h", "kd_small.h")] + [
    os.path.join(ROOT, "include", f) for f in ("kdraft.h", "kdraft_debug.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkdraft)")


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 ops stay off: hipcc would otherwise form v_pk_* fp32 ops
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the first kernel arguments arrive in scalar registers (the kernel
            # keeps a loading prologue for dispatchers that do not preload)
            "-mllvm", "-amdgpu-kernarg-preload-count=4",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    """Compiles the library (always) and returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkdraft")
    if verbose and res.stderr.strip():
        # hipcc's host pass warns that it does not know the packed-fp32 feature
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
