"""Builds libfa2.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python exact_attention_23_amd/build.py [--resource-usage]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", name) for name in ("fa2_fwd.hip", "fa2_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa2.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libfa2.so")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           # keep the compiler from forming packed fp32 VALU ops
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, *SRCS, "-o", LIB + ".tmp"]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and (verbose or resource_usage):
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--resource-usage" in sys.argv)
